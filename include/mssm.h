/*
 * mssm -- Mamba selective scan for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * What the library computes (the selective state-space recurrence):
 *
 *   For every batch row b, channel d and step t (time order), state index n:
 *       Abar      = exp(delta[b,t,d] * A[d,n])          discretisation of the
 *                                                       state matrix
 *                   ("Understanding Mamba", section 2.2, eq. (2))
 *       Bbar      = delta[b,t,d] * B[b,t,n]             first-order input term,
 *                   the form "Selective State Space Models" (section
 *                   "Selection") states Mamba uses, and the Euler form of
 *                   "State Space Models and Mamba" (scalar recurrence section)
 *       h[b,d,n]  = Abar * h[b,d,n] + Bbar * x[b,t,d]   diagonal recurrence
 *                   ("Understanding Mamba", section 2.3, eq. (3)), h = 0 at
 *                   the start of every sequence (mssm_selective_scan_fwd_ex
 *                   also takes an initial state)
 *       y[b,t,d]  = sum_n C[b,t,n] * h[b,d,n]           read-out, eq. (3) with
 *                   the feedthrough term set to zero as in section 2.1
 *
 *   Two evaluation orders, both keeping the [batch, L, D, N] state on chip
 *   ("Understanding Mamba", section 7.3):
 *   - chunked: an associative scan over time.  The affine-pair operator of
 *     section 7.1 (eq. (8)) lets the sequence be cut into chunks that are
 *     scanned independently and then joined; only small per-chunk summaries
 *     reach memory (the workspace).  Any N the library supports, any D.
 *   - single pass: one GPU lane per (channel, state index) runs the whole
 *     sequence in time order; no chunks, no workspace.  Used for N = 16, D a
 *     multiple of 16, inputs aligned to 4 elements and y to 16 bytes, and at
 *     least 8192 channels (batch * D), where it fills the GPU on its own.
 *   The library picks one per call from the shape and the pointers;
 *   mssm_set_tuning(MSSM_TUNE_SCAN_ORDER, ...) pins the choice (the single
 *   pass still needs a shape it supports).  The two orders agree to within
 *   float32 rounding.
 *
 * Layouts: dense, row-major, contiguous.
 *   x, delta    : [batch, L, D]   (d fastest)
 *   B, C        : [batch, L, N]   (n fastest; one B_t, C_t shared by every
 *                                  channel, as in the PyTorch listing of
 *                                  "Selective State Space Models")
 *   A           : [D, N] float32  (the real, negative diagonal; the caller
 *                                  applies any A = -exp(A_log) itself)
 *   y           : [batch, L, D] float32 for every input type
 *   Element type of x, delta, B, C (and of the fused path's weights) is given
 *   by `dtype`; arithmetic, the state and the output are float32 in every
 *   case (bfloat16 inputs are widened exactly).
 *
 * Pointers: device pointers (hipMalloc'ed or equivalent).  The caller owns
 * every buffer.  Outputs must not alias inputs.  Any element-aligned address
 * is accepted.
 *
 * Streams: `stream` is a hipStream_t passed as void*; NULL means the null
 * stream.  Work is enqueued asynchronously; the call does not synchronise.
 * Calls may come from several host threads at once, each with its own
 * stream and buffers (the block's rocBLAS GEMMs share one rocBLAS handle
 * per device, which a call holds until its GEMMs are enqueued).
 *
 * Errors: every entry point returns an mssm_status.  Arguments are checked
 * before any HIP call is made, so argument errors are reported on machines
 * without a GPU.  Nothing is printed and nothing aborts.  On MSSM_ERROR_HIP
 * mssm_last_error_string() gives the HIP error text (thread-local, valid until
 * the next call on the same thread).  Sizes with batch, L or D equal to zero
 * are valid and do nothing.
 */
#ifndef MSSM_H_
#define MSSM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSSM_ABI_VERSION 6

typedef enum {
    MSSM_SUCCESS = 0,
    MSSM_ERROR_INVALID_VALUE = 1,   /* null pointer, negative size, bad enum   */
    MSSM_ERROR_NOT_SUPPORTED = 2,   /* N or R outside what the kernels handle  */
    MSSM_ERROR_SIZE_OVERFLOW = 3,   /* an element count does not fit int64      */
    MSSM_ERROR_WORKSPACE = 4,       /* workspace missing or too small           */
    MSSM_ERROR_HIP = 5              /* a HIP call or kernel launch failed       */
} mssm_status;

typedef enum {
    MSSM_FLOAT32 = 0,
    MSSM_BFLOAT16 = 1
} mssm_dtype;

/* Form of the discretised input term Bbar (Abar = exp(delta A) in both). */
typedef enum {
    MSSM_BBAR_EULER = 0,   /* first order, Bbar = delta * B (the default form)      */
    MSSM_BBAR_ZOH = 1      /* exact zero-order hold, Bbar = (Abar - 1) / A * B,
                              "Understanding Mamba" eq. (2) for a diagonal A.
                              Needs every A[d, n] nonzero (a zero entry gives NaN
                              in that channel); stable A is negative anyway.    */
} mssm_bbar;

/*
 * Tuning settings, process-wide, for tests and performance sweeps.  They
 * start from the environment, read once when the first setting is needed
 * (MSSM_SCAN_DESIGN=chunked|chain, MSSM_CHUNK_LEN=<steps>,
 * MSSM_CPL=1|2); calls never read the environment.  mssm_set_tuning takes
 * effect for calls made after it returns.  A workspace size queried under
 * one setting may be too small under another (the call then returns
 * MSSM_ERROR_WORKSPACE), so set them before sizing buffers.
 *   MSSM_TUNE_SCAN_ORDER      : MSSM_ORDER_AUTO (the default choice by shape,
 *                               pointers and length), MSSM_ORDER_CHUNKED, or
 *                               MSSM_ORDER_SINGLE_PASS where supported.
 *                               Applies to the scan, its backward pass, the
 *                               fused selective SSM and the block.
 *   MSSM_TUNE_CHUNK_LEN       : steps per chunk of the chunked order; 0 picks
 *                               it from the shape.
 *   MSSM_TUNE_CHAINS_PER_LANE : channels per lane of the chunked kernels, 1
 *                               or 2; 0 picks it from the dtype.
 * mssm_set_tuning: MSSM_ERROR_INVALID_VALUE for an unknown key or a value
 * out of range.  mssm_get_tuning writes the current value.
 */
typedef enum {
    MSSM_TUNE_SCAN_ORDER = 0,
    MSSM_TUNE_CHUNK_LEN = 1,
    MSSM_TUNE_CHAINS_PER_LANE = 2
} mssm_tuning;

enum { MSSM_ORDER_AUTO = 0, MSSM_ORDER_CHUNKED = 1, MSSM_ORDER_SINGLE_PASS = 2 };

mssm_status mssm_set_tuning(mssm_tuning key, int64_t value);
mssm_status mssm_get_tuning(mssm_tuning key, int64_t *value);

/* ABI version of the loaded library (MSSM_ABI_VERSION it was built with). */
int mssm_abi_version(void);

/* Static text for a status code. */
const char *mssm_status_string(mssm_status status);

/* Text of the last HIP error seen by this thread, or of the last scratch-size
 * refusal of mssm_selective_scan_fwd_noalloc ("" if none). */
const char *mssm_last_error_string(void);

/* State sizes N the scan kernels are built for (1, 2, 4, 8, 16, 32): returns 1
 * when supported, 0 otherwise. */
int mssm_supports_state_size(int64_t N);

/*
 * Bytes of device workspace mssm_selective_scan_fwd_ws needs for this shape
 * (0 when no chunk summaries are needed).  The figure covers the chunked
 * order, so it holds whichever order a call takes (the single pass uses
 * none).  Returns MSSM_SUCCESS and writes *bytes, or an argument error.
 */
mssm_status mssm_selective_scan_workspace_size(int64_t batch, int64_t L, int64_t D, int64_t N,
                                               mssm_dtype dtype, size_t *bytes);

/*
 * Selective scan forward, y = scan(x, delta, A, B, C) as defined above.
 * Workspace is allocated stream-ordered on `stream` (hipMallocAsync) and
 * released the same way; use mssm_selective_scan_fwd_ws to pass your own.
 * `delta` is the step size after softplus (positive).
 */
mssm_status mssm_selective_scan_fwd(const void *x, const void *delta, const float *A,
                                    const void *B, const void *C, void *y,
                                    int64_t batch, int64_t L, int64_t D, int64_t N,
                                    mssm_dtype dtype, void *stream);

/* As mssm_selective_scan_fwd, with caller-provided device workspace of at
 * least mssm_selective_scan_workspace_size bytes (may be NULL when that size
 * is 0).  The workspace is overwritten; its contents are not needed after the
 * call's work completes on `stream`. */
mssm_status mssm_selective_scan_fwd_ws(const void *x, const void *delta, const float *A,
                                       const void *B, const void *C, void *y,
                                       void *workspace, size_t workspace_bytes,
                                       int64_t batch, int64_t L, int64_t D, int64_t N,
                                       mssm_dtype dtype, void *stream);

/*
 * For callers that cannot allocate device memory during the call (code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation): the scan of mssm_selective_scan_fwd, same arguments, same
 * result (the same kernels and chunking), with the chunked order's chunk
 * summaries kept in a fixed device array that the library holds on every GPU
 * it runs on until the process ends, MSSM_NOALLOC_SCRATCH_BYTES (128 MiB)
 * per GPU.  The call allocates nothing: no hipMalloc, no hipFree, no
 * allocating library routine.  The array's address on a device is looked up
 * on the first call there.
 *   - A shape whose chunk summaries need more than the array holds (see
 *     mssm_selective_scan_workspace_size) gives MSSM_ERROR_WORKSPACE, with
 *     the sizes in mssm_last_error_string(); the single pass needs none.
 *   - Every call on a GPU uses that GPU's one array and leaves its contents
 *     there; the summaries are written in full before they are read, so
 *     nothing has to start at zero.  Calls that overlap in time on one GPU
 *     (several streams or threads at once) race on the array and give wrong
 *     results: serialise them.
 */
#define MSSM_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

mssm_status mssm_selective_scan_fwd_noalloc(const void *x, const void *delta, const float *A,
                                            const void *B, const void *C, void *y,
                                            int64_t batch, int64_t L, int64_t D, int64_t N,
                                            mssm_dtype dtype, void *stream);

/*
 * ---- the scan with its optional parts: input-term form, feedthrough, gate, state ---------
 *
 * mssm_selective_scan_fwd_ex computes, per chain (b, d), starting from
 * h = h0[b, d, :] (zero when h0 is NULL):
 *     h        = Abar * h + Bbar * x[b,t,d]     Bbar per `bbar` (see mssm_bbar)
 *     out      = C[b,t,:] . h + Dskip[d] * x[b,t,d]
 *                  (feedthrough: "Understanding Mamba" eq. (1)/(3), section
 *                   2.1 explains it is a separate term added after the read-out;
 *                   omitted when Dskip is NULL)
 *     y[b,t,d] = out * SiLU(z[b,t,d])           SiLU(v) = v / (1 + exp(-v)), the
 *                  gate of the Mamba block ("Understanding Mamba", section 8.1,
 *                  eq. (9)); omitted when z is NULL
 * and, when h_last is not NULL, writes the state after the last step to
 * h_last[b, d, :].  Passing h_last of one call as h0 of the next continues
 * the sequence (the state summarises the whole past, section 3.2), so a long
 * sequence can be processed in pieces.
 *
 *   Dskip  : [D] float32 or NULL
 *   z      : [batch, L, D] of `dtype` or NULL
 *   h0     : [batch, D, N] float32 (n fastest) or NULL
 *   h_last : [batch, D, N] float32 or NULL; must not overlap h0 or any
 *            other argument (chunks of the sequence run concurrently, so the
 *            last chunk may finish before the first has read h0)
 *   workspace: as mssm_selective_scan_fwd_ws (same size query).
 * With L == 0 and batch, D > 0 the call only sets h_last = h0 (or zero).
 * An invalid `bbar` gives MSSM_ERROR_INVALID_VALUE.
 */
mssm_status mssm_selective_scan_fwd_ex(const void *x, const void *delta, const float *A,
                                       const void *B, const void *C, const float *Dskip,
                                       const void *z, const float *h0, float *y, float *h_last,
                                       mssm_bbar bbar, void *workspace, size_t workspace_bytes,
                                       int64_t batch, int64_t L, int64_t D, int64_t N,
                                       mssm_dtype dtype, void *stream);

/*
 * One recurrent step (decode): the constant-cost-per-token form of
 * "Understanding Mamba" (section 3.2, section 9.1), for every (b, d):
 *     h[b,d,:] = Abar * h[b,d,:] + Bbar * x[b,d]     (in place)
 *     y[b,d]   = (C[b,:] . h[b,d,:] + Dskip[d] x[b,d]) * SiLU(z[b,d])
 * with Abar, Bbar as in the scan (`bbar` selects the form), i.e. exactly one
 * step of mssm_selective_scan_fwd_ex with h0 = h_last = h.
 *
 *   x, delta, z : [batch, D] of `dtype` (z may be NULL)
 *   B, C        : [batch, N] of `dtype`
 *   A           : [D, N] float32;  Dskip : [D] float32 or NULL
 *   h           : [batch, D, N] float32, read and overwritten
 *   y           : [batch, D] float32
 * Needs no workspace.  batch or D equal to zero is a no-op.  batch above
 * 65535 gives MSSM_ERROR_NOT_SUPPORTED (one grid row per batch row).
 */
mssm_status mssm_selective_scan_step(const void *x, const void *delta, const float *A,
                                     const void *B, const void *C, const float *Dskip,
                                     const void *z, float *h, float *y, mssm_bbar bbar,
                                     int64_t batch, int64_t D, int64_t N, mssm_dtype dtype,
                                     void *stream);

/*
 * ---- fused selective SSM: selection projections + scan ----------------------------------
 *
 * The selection mechanism of "Understanding Mamba" (section 5.1, eq. (6)) in
 * the low-rank Mamba shape: each token x_t (D values) is projected by
 * W_xproj [D, R + 2N] to [dt_low (R) | B_t (N) | C_t (N)] (in that order;
 * weights are [in, out], i.e. P = x @ W_xproj); Delta_t = softplus(dt_low @
 * W_dtproj + dt_bias) with W_dtproj [R, D] and one bias per channel
 * (softplus as in section 5.1); then the scan above runs on (x, Delta, A, B,
 * C).  x, W_xproj, W_dtproj are bfloat16; dt_bias, A and y are float32.
 * x_proj runs on the bf16 matrix cores (the library's own kernel, one pass
 * over x) with float32 accumulation; dt_low leaves it as two bfloat16 parts
 * (hi = bf16(dt_low), lo = bf16(dt_low - hi)), i.e. kept to about 16
 * significant bits, for dt_proj, which also runs on the bf16 matrix cores
 * with float32 accumulation; B, C and the pre-softplus values stay float32.
 *
 * Where Delta lives follows the scan order (see the top of this file):
 *   - chunked order: Delta is made per 32-step tile on the matrix cores
 *     inside the scan kernels and never written to memory;
 *   - single pass (N = 16, D a multiple of 16, R <= 256, x and y 16-byte
 *     aligned, at least 8192 channels batch * D, unless the chunked order is
 *     pinned): one matrix-core kernel writes Delta once, as float32
 *     [batch * L, D] (4 bytes per element) into the workspace, and the scan
 *     reads it back.  The workspace size covers it.
 *
 * Supported: dtype MSSM_BFLOAT16 only (MSSM_FLOAT32 -> NOT_SUPPORTED); N in
 * the scan's set; R a multiple of 16 in [16, 1024]; batch*L and D below 2^31.
 * The workspace must be 256-byte aligned and at least
 * mssm_selective_ssm_fused_workspace_size bytes; it is always required (the
 * projection lands there).  The fused path makes no library calls (no
 * rocBLAS).
 */

/* 1 if the fused path is built for state size N and rank R, else 0. */
int mssm_fused_supports(int64_t N, int64_t R);

mssm_status mssm_selective_ssm_fused_workspace_size(int64_t batch, int64_t L, int64_t D,
                                                    int64_t N, int64_t R, mssm_dtype dtype,
                                                    size_t *bytes);

mssm_status mssm_selective_ssm_fused_fwd(const void *x, const void *W_xproj,
                                         const void *W_dtproj, const float *dt_bias,
                                         const float *A, float *y, void *workspace,
                                         size_t workspace_bytes, int64_t batch, int64_t L,
                                         int64_t D, int64_t N, int64_t R, mssm_dtype dtype,
                                         void *stream);

/*
 * ---- the Mamba block around the scan -------------------------------------------------------
 *
 * "Understanding Mamba", section 8.1, eq. (9), and its block listing (section
 * 10.2):
 *     [u | z] = u0 @ W_in                      W_in [Dm, 2 Di]: columns 0..Di-1
 *                                              give u, columns Di..2Di-1 give z
 *     x       = SiLU(causal_conv1d(u) + conv_b)
 *     y       = the fused selective SSM on x  (Delta, B, C from x as in
 *               mssm_selective_ssm_fused_fwd) with feedthrough Dskip * x
 *     out     = (y * SiLU(z)) @ W_out          W_out [Di, Dm]
 * The block has no normalisation and no residual add (they belong to the
 * model around it, section 8.2).
 *
 * causal_conv1d is depthwise: for channel d with taps conv_w[d, 0..k-1],
 *     c[b,t,d] = sum_i conv_w[d, i] * u[b, t - (k-1) + i, d],   u = 0 before t = 0,
 * so tap k-1 weighs the current token (the listing's left padding by k - 1
 * zeros).  k is 1..8.
 *
 * mssm_causal_conv1d_silu: out = SiLU(causal_conv1d(u) + conv_b) alone.
 *   u [batch, L, D] of `dtype`; conv_w [D, k] float32; conv_b [D] float32 or
 *   NULL; out [batch, L, D] float32.  No workspace.
 *
 * mssm_mamba_block_fwd: u0 [batch, L, Dm], W_in, W_x [Di, R + 2N], W_dt [R, Di],
 * W_out bf16 (dtype must be MSSM_BFLOAT16); conv_w, conv_b (may be NULL),
 * dt_bias [Di], A [Di, N], Dskip [Di] (may be NULL) float32; out [batch, L, Dm]
 * float32.  Precision: the projections accumulate in float32; x stays float32
 * for the scan and the feedthrough; x_proj and W_out take their float32 inputs
 * (x, and the gated result) as bf16 hi + lo pairs, about 16 significant bits
 * (x_proj: both parts multiplied into the same sums by the library's own
 * matrix-core kernel; in_proj and out_proj: rocBLAS GEMMs, one per part, on
 * a rocBLAS handle the first call on a device creates and keeps until the
 * process exits).  The workspace (256-byte aligned,
 * mssm_mamba_block_workspace_size bytes) holds u, z, x (float32
 * [batch*L, Di]), the two bf16 pairs and the fused scan's buffers.  batch, L or Dm equal to zero is a no-op; Di equal to zero writes
 * zeros to out.
 */
mssm_status mssm_causal_conv1d_silu(const void *u, const float *conv_w, const float *conv_b,
                                    float *out, int64_t batch, int64_t L, int64_t D, int64_t k,
                                    mssm_dtype dtype, void *stream);

/* 1 if the block is built for state size N, rank R and conv width k, else 0. */
int mssm_mamba_block_supports(int64_t N, int64_t R, int64_t k);

mssm_status mssm_mamba_block_workspace_size(int64_t batch, int64_t L, int64_t Dm, int64_t Di,
                                            int64_t N, int64_t R, int64_t k, mssm_dtype dtype,
                                            size_t *bytes);

mssm_status mssm_mamba_block_fwd(const void *u0, const void *W_in, const float *conv_w,
                                 const float *conv_b, const void *W_x, const void *W_dt,
                                 const float *dt_bias, const float *A, const float *Dskip,
                                 const void *W_out, float *out, void *workspace,
                                 size_t workspace_bytes, int64_t batch, int64_t L, int64_t Dm,
                                 int64_t Di, int64_t N, int64_t R, int64_t k, mssm_dtype dtype,
                                 void *stream);

/*
 * ---- backward ------------------------------------------------------------------------------
 *
 * Gradients of L = sum(dout * y) for y = mssm_selective_scan_fwd_ex(x, delta,
 * A, B, C, Dskip, z, h0) with the first-order input term (MSSM_BBAR_EULER), by
 * the chain rule through the recurrence (the adjoint lam_t = C_t g_t +
 * a_{t+1} lam_{t+1} is a reverse scan).  The states are recomputed from the
 * inputs, never stored in full ("State Space Models and Mamba", the
 * hardware-aware scan recomputes them for the backward pass).  Two orders,
 * chosen like the forward scan's (MSSM_SCAN_DESIGN, shape and alignment):
 *   single pass (N = 16, D % 16 == 0, 16-byte aligned float32 / 8-byte
 *     aligned bfloat16 inputs and float32 gradients, at least 8192 channels
 *     batch * D): one forward pass stores the state after every 16-step tile
 *     in the workspace, then one kernel walks the tiles backwards,
 *     recomputing each tile's states from its checkpoint while sweeping the
 *     adjoint;
 *   chunked (every other case): re-runs the forward chunk summaries, runs the
 *     adjoint's chunk summaries in reverse, then recomputes each 16-step
 *     chunk's states in registers while sweeping it backwards.
 *
 *   dout            : [batch, L, D] float32 (the gradient of the float32 y)
 *   dx, ddelta, dz  : [batch, L, D] float32
 *   dA              : [D, N] float32;   dDskip : [D] float32
 *   dB, dC          : [batch, L, N] float32 (summed over the channels d)
 *   dh0             : [batch, D, N] float32 or NULL
 * Dskip and dDskip are given together (or both NULL), likewise z and dz; dh0
 * needs h0.  Every gradient buffer is overwritten, not accumulated into.
 * dA and dDskip (sums over batch and time) and dB, dC (sums over channels)
 * are formed from partial sums in a fixed order: results are deterministic.
 * The workspace (256-byte aligned, mssm_selective_scan_bwd_workspace_size
 * bytes, enough for either order) holds the checkpoints or the chunk
 * summaries of both directions, and the partial sums.
 * With batch, L or D equal to zero the gradients that still have elements are
 * set to zero.
 */
mssm_status mssm_selective_scan_bwd_workspace_size(int64_t batch, int64_t L, int64_t D, int64_t N,
                                                   mssm_dtype dtype, size_t *bytes);

mssm_status mssm_selective_scan_bwd(const void *x, const void *delta, const float *A,
                                    const void *B, const void *C, const float *Dskip,
                                    const void *z, const float *h0, const float *dout, float *dx,
                                    float *ddelta, float *dA, float *dB, float *dC, float *dDskip,
                                    float *dz, float *dh0, void *workspace, size_t workspace_bytes,
                                    int64_t batch, int64_t L, int64_t D, int64_t N,
                                    mssm_dtype dtype, void *stream);

/*
 * ---- forward and backward sharing saved states (training) -------------------------------
 *
 * The backward pass needs the states h_t, which it recomputes ("State Space
 * Models and Mamba", hardware-aware scan: the backward recomputes the states
 * rather than reading them from memory); the single-pass order restarts that
 * recomputation from checkpoints, the state after every 16-step tile.
 * mssm_selective_scan_bwd writes them with a forward pass of its own.  In
 * training the forward call is made anyway, so mssm_selective_scan_fwd_save
 * writes them there, together with, when z is given, the output before the
 * gate (C . h + Dskip x, which the gate's gradient needs), and
 * mssm_selective_scan_bwd_saved reads them instead of recomputing.
 *
 * Only the single-pass layout has this form: N = 16, D % 16 == 0, float32
 * x / delta / B / C / z 16-byte aligned (bfloat16: 8-byte), y, dout and the
 * float32 gradients dx, ddelta, dz 16-byte aligned; any channel count.  Other
 * shapes give MSSM_ERROR_NOT_SUPPORTED (use mssm_selective_scan_fwd_ex and
 * mssm_selective_scan_bwd), as do unaligned pointers.
 *
 * mssm_selective_scan_saved_size: bytes of the saved buffer for this shape,
 *   with (gate != 0) or without the gate; 0 for shapes without this form.
 * mssm_selective_scan_fwd_save: y (and h_last) exactly as
 *   mssm_selective_scan_fwd_ex with MSSM_BBAR_EULER and the same optional
 *   parts, and the saved tensors, in `saved` (float32, 256-byte aligned, at
 *   least saved_size bytes, caller-owned): states [batch, ceil(L/16), D, N]
 *   (the state after tile j, j < ceil(L/16) - 1; the last tile's slot is not
 *   written), then with z the output before the gate [batch, L, D].  Needs
 *   no workspace.  L == 0 only sets h_last = h0 (or zero).
 * mssm_selective_scan_bwd_saved: the gradients of mssm_selective_scan_bwd
 *   (same arguments, same workspace size query) from `saved` as written by
 *   mssm_selective_scan_fwd_save for the same inputs, Dskip, z and h0.  A
 *   buffer written for other inputs gives wrong gradients; one too small or
 *   unaligned gives MSSM_ERROR_WORKSPACE.
 */
mssm_status mssm_selective_scan_saved_size(int64_t batch, int64_t L, int64_t D, int64_t N,
                                           int gate, size_t *bytes);

mssm_status mssm_selective_scan_fwd_save(const void *x, const void *delta, const float *A,
                                         const void *B, const void *C, const float *Dskip,
                                         const void *z, const float *h0, float *y,
                                         float *h_last, float *saved, size_t saved_bytes,
                                         int64_t batch, int64_t L, int64_t D, int64_t N,
                                         mssm_dtype dtype, void *stream);

mssm_status mssm_selective_scan_bwd_saved(const void *x, const void *delta, const float *A,
                                          const void *B, const void *C, const float *Dskip,
                                          const void *z, const float *h0, const float *saved,
                                          size_t saved_bytes, const float *dout, float *dx,
                                          float *ddelta, float *dA, float *dB, float *dC,
                                          float *dDskip, float *dz, float *dh0, void *workspace,
                                          size_t workspace_bytes, int64_t batch, int64_t L,
                                          int64_t D, int64_t N, mssm_dtype dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MSSM_H_ */
