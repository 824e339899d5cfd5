// Host-side internals shared by the C-ABI front end and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "mssm.h"

namespace mssm {

// Current value of a tuning setting (settings.hip): from the environment,
// read once, or from mssm_set_tuning.
int64_t tuning(mssm_tuning key);

// How one scan call is cut along time.  The sequence is split into K chunks
// of chunk_len steps (the last may be shorter).  Chunks 0..K-2 first produce
// summaries (their local end state from a zero start, and their decay
// exp(A * total step size)); each chunk then folds the summaries before it
// into its carry-in with the affine-pair operator and scans its own steps from
// that carry.
struct ScanPlan {
  bool chain = false;         // single-pass design instead (no chunks, no workspace)
  int cpl = 1;                // chains (adjacent channels) per lane: 1 or 2
  int K = 1;
  int64_t chunk_len = 0;
  size_t sum_h_bytes = 0;     // float [batch][K-1][N][D]: chunk end state from zero
  size_t sum_s_offset = 0;    // byte offset of double [batch][K-1][D]: chunk step-size total
  size_t workspace_bytes = 0;
};



struct ScanArgs {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  void* y;
  int64_t batch, L, D, N;
  mssm_dtype dtype;
  const float* Dskip = nullptr;   // [D] feedthrough, or null
  const void* z = nullptr;        // [batch, L, D] gate input, or null
  const float* h0 = nullptr;      // [batch, D, N] initial state, or null (zero)
  float* h_last = nullptr;        // [batch, D, N] final state out, or null
  mssm_bbar bbar = MSSM_BBAR_EULER;
};

// Plan for `cpl` chains per lane.
ScanPlan plan_scan(int64_t batch, int64_t L, int64_t D, int64_t N, int cpl);

// Whether a call over this many channels (batch * D) takes the single-pass
// order when its shape and pointers allow it: the scan-order setting pins the
// answer, else at least 8192 channels.
bool single_pass_chosen(int64_t channels);

// Single-pass scan with one lane per (channel, state index), for N = 16 and
// shapes with many channels: whether the forward uses it for these arguments
// (shape, alignment, channel count, sequence length: bfloat16 from 16384 steps
// and float32 from 32768 go chunked, the scan-order setting), and its launch.
bool chain_scan_applies(const ScanArgs& a);
hipError_t launch_chain_scan(const ScanArgs& a, hipStream_t stream);

// Whether the arguments fit the single-pass layout (N = 16, D % 16 == 0,
// alignment, sizes), whatever the channel count or the scan-order setting.
bool chain_layout_ok(const ScanArgs& a);
// Forward that also saves the backward pass's inputs (first-order input term):
// the state after every 16-step tile into ck [batch, tiles, D, N] and, with
// the gate, the output before the gate into y_pre [batch, L, D].  Needs the
// single-pass layout.
hipError_t launch_chain_save(const ScanArgs& a, float* ck, float* y_pre, hipStream_t stream);

// Where the saved tensors sit in the caller's buffer (256-byte aligned
// offsets); bytes == 0 when the shape has no saved form.
struct SavedLayout {
  size_t ck_offset = 0, y_pre_offset = 0, bytes = 0;
};
SavedLayout saved_layout(int64_t batch, int64_t L, int64_t D, int64_t N, bool gate);

// The single pass behind the selection projections (fused selective SSM and
// Mamba block): delta is the float32 matrix softplus(dt_low W_dt + bias) and
// B, C are the columns R .. R+2N-1 of P's rows.  Whether it applies (N = 16,
// D % 16 == 0, R <= 256, enough channels, the scan-order setting; x and y as
// given), and the launch.
struct ChainFusedArgs {
  const void* x = nullptr;        // [batch, L, D] bf16, or float32 with x_f32
  bool x_f32 = false;
  const float* delta = nullptr;   // [batch, L, D]
  const float* P = nullptr;       // [batch*L, ldp]
  int64_t ldp = 0, R = 0;
  const float* A = nullptr;
  const float* Dskip = nullptr;   // or null
  const float* z = nullptr;       // [batch, L, D] float32, or null
  void* y = nullptr;              // float32, or bf16 hi part with y_bf16
  void* y_lo = nullptr;           // with y_bf16: bf16(y - hi)
  bool y_bf16 = false;
  int64_t ld_y = 0;               // with y_bf16: row stride of y and y_lo (0: D)
  int64_t batch = 0, L = 0, D = 0;
  const float* bcg = nullptr;     // B, C grouped by four state indices (launch_xproj), or null
};
bool chain_fused_applies(int64_t batch, int64_t D, int64_t N, int64_t R, const void* x,
                         const void* y);
hipError_t launch_chain_fused(const ChainFusedArgs& a, hipStream_t stream);
// The split-state single pass (split_scan.hip): lane = channel, each of a
// block's four wavefronts owns 4 of the N = 16 state indices; used by
// launch_chain_fused from 32768 channels (batch * D) on, D a multiple of 64.
bool split_fused_applies(int64_t batch, int64_t D, int64_t N);
hipError_t launch_split_fused(const ChainFusedArgs& a, hipStream_t stream);

// The plan for these arguments: the single-pass design when it applies, else
// the chunked plan with the chains-per-lane choice below.
ScanPlan plan_for(const ScanArgs& a);

// Workspace that covers the plan of every chains-per-lane choice the launcher
// can make for this shape (the choice also depends on pointer alignment).
size_t workspace_bound(int64_t batch, int64_t L, int64_t D, int64_t N);

// Chains per lane for these arguments: 2 for bfloat16 inputs when D is even
// and x, delta, y are aligned for paired access, else 1.
int choose_cpl(const ScanArgs& a);

// Enqueues the scan kernels on `stream`.  Arguments are already validated and
// the workspace holds at least plan.workspace_bytes.  Returns hipSuccess or
// the launch error.
hipError_t launch_scan(const ScanArgs& a, const ScanPlan& plan, void* workspace,
                       hipStream_t stream);

bool state_size_supported(int64_t N);

// The fixed device scratch of mssm_selective_scan_fwd_noalloc (noalloc.hip):
// its size, and the current device's copy (address looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t scratch_pointer(void** out);


// The carry pass over chunk summaries (shared by the plain, fused and backward
// paths): hloc [batch, K-1, N, D] is overwritten with the carries, sum_s
// [batch, K-1, D] holds each chunk's step-size total, A [D, N]; h0
// ([batch, D, N], or null for a zero start) is the state before chunk 0.
hipError_t launch_carry(float* sum_h, const double* sum_s, const float* A, const float* h0,
                        int64_t batch, int64_t D, int64_t N, int K, hipStream_t stream);

// h_last = h0 (or zero when h0 is null), `count` floats: the final state of an
// empty sequence.
hipError_t launch_state_init(float* h_last, const float* h0, int64_t count, hipStream_t stream);

// One recurrent step per (batch row, channel): h is updated in place.
struct StepArgs {
  const void* x;        // [batch, D]
  const void* delta;    // [batch, D]
  const float* A;       // [D, N]
  const void* B;        // [batch, N]
  const void* C;        // [batch, N]
  const float* Dskip;   // [D] or null
  const void* z;        // [batch, D] or null
  float* h;             // [batch, D, N]
  float* y;             // [batch, D]
  int64_t batch, D, N;
  mssm_dtype dtype;
  mssm_bbar bbar;
};
hipError_t launch_step(const StepArgs& a, hipStream_t stream);

// ---- fused projections + scan ------------------------------------------------------------

struct FusedArgs {
  const void* x;        // [batch, L, D] bf16
  const void* W_x;      // [D, R + 2N] bf16
  const void* W_dt;     // [R, D] bf16
  const float* dt_bias; // [D]
  const float* A;       // [D, N]
  float* y;             // [batch, L, D]
  int64_t batch, L, D, N, R;
};

// Workspace: P = x @ W_x (float32 [batch*L, R+2N]), dt_low as bf16 hi and lo
// parts ([batch*L, R] each), W_dt^T (bf16 [D, R]), then the scan's chunk
// summaries.
struct FusedPlan {
  ScanPlan scan;
  bool chain = false;         // single-pass scan over a float32 delta matrix
  size_t delta_offset = 0;    // with chain: float32 [batch*L, D]
  size_t bcg_offset = 0;      // with the split-state scan: B, C grouped (xproj_bcg_rows(M) rows)
  size_t p_bytes = 0;
  size_t dtl_offset = 0;
  size_t dtl_lo_offset = 0;
  size_t wt_offset = 0;
  size_t wx_t_offset = 0;     // W_x transposed [R + 2N, D padded to 64] for x_proj
  size_t scan_offset = 0;
  size_t workspace_bytes = 0;
};

struct FusedStatus {
  hipError_t hip = hipSuccess;
  bool blas_failed = false;
};

// The fused scan kernels' inputs: x is bf16 (the fused selective SSM) or
// float32 (the Mamba block, where x comes from the conv + SiLU prologue);
// the block also applies the feedthrough and the SiLU(z) gate and stores y as
// a bf16 hi + lo pair (y and y_lo) for the output projection.  P holds [dt_low | B | C] rows; dtl/dtl_lo the bf16 parts of dt_low;
// wT = W_dt^T.
struct FusedScanArgs {
  const void* x = nullptr;
  bool x_f32 = false;
  const float* z = nullptr;       // [batch, L, D] or null
  const float* Dskip = nullptr;   // [D] or null
  void* y = nullptr;
  bool y_bf16 = false;
  void* y_lo = nullptr;           // with y_bf16: bf16(y - hi)
  const float* P = nullptr;
  const uint16_t* dtl = nullptr;
  const uint16_t* dtl_lo = nullptr;
  const uint16_t* wT = nullptr;
  const float* dt_bias = nullptr;
  const float* A = nullptr;
  float* sum_h = nullptr;
  double* sum_s = nullptr;
  int64_t batch = 0, L = 0, D = 0, N = 0, R = 0;
};
hipError_t launch_fused_scan(const FusedScanArgs& a, const ScanPlan& plan, hipStream_t stream);

// x_proj on the matrix cores (xproj.hip): P = x W_x for x [M, K] bf16 (row
// stride lda; with x_lo, x = x + x_lo as a bf16 pair, both multiplied into
// the same float32 sums) and W_x [K, ncol] bf16 (ncol = R + 2N).  Columns
// below R (dt_low) are stored as the bf16 pair dtl = bf16(v), dtl_lo =
// bf16(v - dtl) ([M, R] each); columns R.. to P[m * ldp + c] as float32.
// WxT is workspace for W_x transposed and zero-padded along k:
// ncol * xproj_padded_k(K) bf16.  With bcg (N = 16 only) B and C are also
// stored grouped by four state indices: bcg[(g * xproj_bcg_rows(M) + m) * 8 +
// j] = B[m][4g + j] for j < 4 and C[m][4g + j - 4] for j >= 4; the 8 rows
// past M are set to zero.
int64_t xproj_padded_k(int64_t K);
int64_t xproj_bcg_rows(int64_t M);
hipError_t launch_xproj(const uint16_t* x, const uint16_t* x_lo, int64_t lda, int64_t M,
                        int64_t K, const void* W_x, int64_t ncol, int64_t R, uint16_t* WxT,
                        uint16_t* dtl, uint16_t* dtl_lo, float* P, int64_t ldp, float* bcg,
                        hipStream_t stream);

// wT [D, R] = W_dt^T for the dt_proj kernels.
hipError_t launch_wdt_transpose(const void* W_dt, int64_t R, int64_t D, uint16_t* wT,
                                hipStream_t stream);

// delta[m, d] = softplus(sum_r (dtl + dtl_lo)[m, r] wT[d, r] + bias[d]), float32
// [M, D], on the matrix cores (R a multiple of 16).
hipError_t launch_dtproj_softplus(const uint16_t* dtl, const uint16_t* dtl_lo, const uint16_t* wT,
                                  const float* bias, float* delta, int64_t M, int64_t D,
                                  int64_t R, hipStream_t stream);

// The current device's rocBLAS handle (created on first use, kept until exit),
// bound to `stream` and held by this object until it goes out of scope: the
// handle is shared by every call on the device, so a call keeps it, and the
// stream it is bound to, to itself until its last GEMM is enqueued (calls
// from several host threads then enqueue their GEMMs one call at a time).
// ok() false: rocBLAS failed (hip_error() == hipSuccess) or a HIP call failed.
class BlasLease {
 public:
  explicit BlasLease(hipStream_t stream);
  bool ok() const { return ok_; }
  rocblas_handle get() const { return handle_; }
  hipError_t hip_error() const { return hip_; }

 private:
  std::unique_lock<std::mutex> lock_;
  rocblas_handle handle_ = nullptr;
  hipError_t hip_ = hipSuccess;
  bool ok_ = false;
};

// Row-major C[M, n] (float32, row stride ldc) = A[M, k] B[k, n] + beta C, A
// and B bf16, float32 accumulation, with B given transposed, BT[n, k] (row
// strides lda, ldbt): both operands then run along k in memory, the layout
// rocBLAS's matrix-core GEMMs are fastest with (measured 7 % faster than B as
// [k, n] on the block's projections).  false if rocBLAS fails.
bool gemm_rm_bf16_bt(rocblas_handle h, int64_t M, int64_t n, int64_t k, const void* A,
                     int64_t lda, const void* BT, int64_t ldbt, float* C, int64_t ldc,
                     float beta);
// wT[c * ldt + r] = W[r, c] for a row-major bf16 W[rows, cols], in 64 x 64
// tiles; ldt >= rows, 0 meaning rows.
hipError_t launch_transpose_bf16(const void* W, uint16_t* wT, int64_t rows, int64_t cols,
                                 hipStream_t stream, int64_t ldt = 0);

// ---- the Mamba block ------------------------------------------------------------------------

// out[b,t,d] = SiLU(bias[d] + sum_i w[d,i] u[b, t-k+1+i, d]) (u = 0 before t = 0);
// u float32 or bf16 [batch, L, D]; w [D, k] float32; bias [D] or null;
// out_hi / out_lo (optional, together) receive the bf16 pair hi = bf16(out),
// lo = bf16(out - hi).
hipError_t launch_conv1d_silu(const void* u, bool u_f32, const float* w, const float* bias,
                              float* out, uint16_t* out_hi, uint16_t* out_lo, int64_t batch,
                              int64_t L, int64_t D, int k, hipStream_t stream);

struct BlockArgs {
  const void* u0;        // [batch, L, Dm] bf16
  const void* W_in;      // [Dm, 2 Di] bf16
  const float* conv_w;   // [Di, k]
  const float* conv_b;   // [Di] or null
  const void* W_x;       // [Di, R + 2N] bf16
  const void* W_dt;      // [R, Di] bf16
  const float* dt_bias;  // [Di]
  const float* A;        // [Di, N]
  const float* Dskip;    // [Di] or null
  const void* W_out;     // [Di, Dm] bf16
  float* out;            // [batch, L, Dm]
  int64_t batch, L, Dm, Di, N, R;
  int k;
};

// Workspace: U, Z, X (float32 [M, Di]), bf16 hi/lo pairs of X and of the
// gated result G ([M, Di] each), then the fused scan's P, dt_low parts,
// W_dt^T and chunk summaries.
struct BlockPlan {
  ScanPlan scan;
  bool chain = false;         // single pass; delta goes to the (by then unused) u buffer
  // g_offset: the gated output's bf16 hi + lo pair, 2 * M * Di values
  size_t u_offset = 0, z_offset = 0, x_offset = 0, xb_offset = 0, xl_offset = 0, g_offset = 0;
  size_t p_offset = 0, dtl_offset = 0, dtl_lo_offset = 0, wt_offset = 0, scan_offset = 0;
  size_t bcg_offset = 0;      // with the split-state scan: B, C grouped for it
  // the projection weights transposed for the GEMMs: W_in^T [2Di, Dm], W_x^T
  // [R + 2N, Di], W_out^T twice side by side [Dm, 2Di]
  size_t win_t_offset = 0, wx_t_offset = 0, wout_t_offset = 0;
  size_t workspace_bytes = 0;
};
BlockPlan plan_block(int64_t batch, int64_t L, int64_t Dm, int64_t Di, int64_t N, int64_t R,
                     int cpl, bool chain);
size_t block_workspace_bound(int64_t batch, int64_t L, int64_t Dm, int64_t Di, int64_t N,
                             int64_t R);
FusedStatus launch_block(const BlockArgs& a, const BlockPlan& plan, void* workspace,
                         hipStream_t stream);

// ---- backward ------------------------------------------------------------------------------

struct BwdArgs {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;   // or null
  const void* z;        // or null
  const float* h0;      // or null
  const float* dout;    // [batch, L, D]
  float* dx;
  float* ddelta;
  float* dA;
  float* dB;
  float* dC;
  float* dD;            // with Dskip
  float* dz;            // with z
  float* dh0;           // or null
  int64_t batch, L, D, N;
  mssm_dtype dtype;
  // from a saving forward call (single pass only): the states after each
  // tile, and with the gate the output before it; null: recomputed
  const float* saved_ck = nullptr;
  const float* saved_y_pre = nullptr;
};

// Chunks of `chunk` steps; workspace: forward and reverse chunk summaries
// (end states [batch, K-1, N, D] float32 and step-size totals [batch, K-1, D]
// float64, for each direction), per-wavefront dB/dC partials
// [ceil(D/64), batch, L, 2N], per-chunk dA partials [batch*K, D, N] and dD
// partials [batch*K, D].
struct BwdPlan {
  bool chain = false;         // single-pass order: checkpoints + one reverse kernel
  size_t ck_offset = 0;       // with chain: states after each tile [batch, tiles, D, N]
  int64_t chunk = 0;
  int K = 1;
  size_t fwd_h_offset = 0, fwd_s_offset = 0, rev_h_offset = 0, rev_s_offset = 0;
  size_t part_bc_offset = 0, part_a_offset = 0, part_d_offset = 0;
  size_t workspace_bytes = 0;
};
// chain: the single-pass order (partials per 16-channel block and per batch
// row); the bound covers both orders.
BwdPlan plan_bwd(int64_t batch, int64_t L, int64_t D, int64_t N, bool chain);
size_t bwd_workspace_bound(int64_t batch, int64_t L, int64_t D, int64_t N);
hipError_t launch_bwd(const BwdArgs& a, const BwdPlan& plan, void* workspace, hipStream_t stream);

// The single-pass backward (N = 16, D % 16 == 0, aligned pointers, enough
// channels): whether it applies, and its two kernels (checkpoints, reverse
// sweep) writing the partials that launch_bwd then reduces.
bool chain_bwd_layout_ok(const BwdArgs& a);   // shape and alignment only
bool chain_bwd_applies(const BwdArgs& a);     // and the order is chosen
hipError_t launch_chain_bwd(const BwdArgs& a, float* ck, const float* y_pre, bool saved,
                            float* part_bc, float* part_a, float* part_d, hipStream_t stream);

// chain: the single-pass order (plan_fused ignores cpl then); the bound
// covers every order and layout.
FusedPlan plan_fused(int64_t batch, int64_t L, int64_t D, int64_t N, int64_t R, int cpl,
                     bool chain);
size_t fused_workspace_bound(int64_t batch, int64_t L, int64_t D, int64_t N, int64_t R);
int choose_fused_cpl(int64_t D);
FusedStatus launch_fused(const FusedArgs& a, const FusedPlan& f, void* workspace,
                         hipStream_t stream);

}  // namespace mssm
