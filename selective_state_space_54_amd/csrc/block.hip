// The Mamba block forward around the selective scan ("Understanding Mamba",
// section 8.1, eq. (9), and the block listing of section 10.2):
//
//   [u | z] = u0 W_in                       input projection, split in two
//   x       = SiLU(causal_conv1d(u) + b)    depthwise causal convolution
//   y       = selective SSM on x            Delta, B, C selected from x
//                                           (section 5.1), plus D x
//   out     = (y * SiLU(z)) W_out           gate, output projection
//
// On gfx950: the three projections (W_in, x_proj, W_out) are plain bf16 GEMMs
// with float32 accumulation on rocBLAS; the convolution + SiLU is one
// HBM-bound kernel here; dt_proj, the scan, the feedthrough and the gate run
// in the fused scan kernels (dt_proj on the matrix cores, Delta never in
// memory), which store the gated result for W_out.  x stays float32 for the
// scan and the feedthrough.  The x_proj and W_out GEMMs take their float32
// inputs as bf16 hi + lo pairs (hi = bf16(v), lo = bf16(v - hi), about 16
// significant bits), one accumulating GEMM per part: a single bf16 rounding
// there would move a large element by a whole bf16 step wherever the GPU's
// and an exact evaluation's values fall on opposite sides of a rounding
// boundary.
#include "mssm_internal.h"
#include "scan_device.h"

namespace mssm {

namespace {

constexpr int kConvBlock = 256;
constexpr int kConvTile = 8;      // steps whose loads are issued together

template <typename T>
__device__ __forceinline__ float ld_elem(const T* p) { return to_float(*p); }

// out[b, t, d] = SiLU(bias[d] + sum_{i<K} w[d, i] * u[b, t - (K-1) + i, d]),
// with u taken as zero before t = 0: tap K-1 multiplies the current token, as
// in the causal_conv1d of the block listing (left padding by K - 1 zeros).
// Block (dtile, time chunk, b); lane = channel.  out_hi / out_lo (optional)
// receive hi = bf16(out) and lo = bf16(out - hi).
template <int K, typename TU>
__global__ __launch_bounds__(kConvBlock) void conv1d_silu_kernel(
    const TU* __restrict__ u, const float* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ out, uint16_t* __restrict__ out_hi, uint16_t* __restrict__ out_lo,
    int64_t L, int64_t D, int64_t tchunk, int64_t n_dtiles, int64_t n_tchunks) {
  const int64_t bid = blockIdx.x;
  const int64_t dtile = bid % n_dtiles;
  const int64_t rest = bid / n_dtiles;
  const int64_t tc = rest % n_tchunks;
  const int64_t b = rest / n_tchunks;
  const int64_t d = dtile * kConvBlock + threadIdx.x;
  if (d >= D) return;                       // no barriers in this kernel
  float wk[K];
#pragma unroll
  for (int i = 0; i < K; ++i) wk[i] = w[d * K + i];
  const float bv = bias != nullptr ? bias[d] : 0.0f;
  const int64_t t0 = tc * tchunk;
  const int64_t t1 = t0 + tchunk < L ? t0 + tchunk : L;
  const TU* ub = u + b * L * D + d;
  float win[K > 1 ? K - 1 : 1];             // u at t-K+1 .. t-1
#pragma unroll
  for (int i = 0; i < K - 1; ++i) {
    const int64_t t = t0 - (K - 1) + i;
    win[i] = t >= 0 ? ld_elem(ub + t * D) : 0.0f;
  }
  for (int64_t tb = t0; tb < t1; tb += kConvTile) {
    float uc[kConvTile];
#pragma unroll
    for (int j = 0; j < kConvTile; ++j) {
      const int64_t t = tb + j < t1 ? tb + j : t1 - 1;   // past the chunk: re-read its last row
      uc[j] = ld_elem(ub + t * D);
    }
#pragma unroll
    for (int j = 0; j < kConvTile; ++j) {
      const int64_t t = tb + j;
      if (t < t1) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < K - 1; ++i) acc = __builtin_fmaf(wk[i], win[i], acc);
        acc = __builtin_fmaf(wk[K - 1], uc[j], acc);
        const float v = silu(acc + bv);
        const int64_t o = (b * L + t) * D + d;
        out[o] = v;
        if (out_hi != nullptr) {
          const uint32_t hb = bf16_rne_bits(v);
          out_hi[o] = static_cast<uint16_t>(hb);
          out_lo[o] = static_cast<uint16_t>(bf16_rne_bits(v - __uint_as_float(hb << 16)));
        }
#pragma unroll
        for (int i = 0; i + 1 < K - 1; ++i) win[i] = win[i + 1];
        if constexpr (K > 1) win[K - 2] = uc[j];
      }
    }
  }
}

template <typename TU>
hipError_t launch_conv_t(const TU* u, const float* w, const float* bias, float* out,
                         uint16_t* out_hi, uint16_t* out_lo, int64_t batch, int64_t L, int64_t D,
                         int k, hipStream_t stream) {
  const int64_t tchunk = 64;
  const int64_t n_dtiles = (D + kConvBlock - 1) / kConvBlock;
  const int64_t n_tchunks = (L + tchunk - 1) / tchunk;
  const dim3 grid((unsigned)(n_dtiles * n_tchunks * batch));
  switch (k) {
#define MSSM_CONV_CASE(KK)                                                                    \
  case KK:                                                                                    \
    hipLaunchKernelGGL((conv1d_silu_kernel<KK, TU>), grid, dim3(kConvBlock), 0, stream, u, w, \
                       bias, out, out_hi, out_lo, L, D, tchunk, n_dtiles, n_tchunks);         \
    break;
    MSSM_CONV_CASE(1)
    MSSM_CONV_CASE(2)
    MSSM_CONV_CASE(3)
    MSSM_CONV_CASE(4)
    MSSM_CONV_CASE(5)
    MSSM_CONV_CASE(6)
    MSSM_CONV_CASE(7)
    MSSM_CONV_CASE(8)
#undef MSSM_CONV_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

hipError_t launch_conv1d_silu(const void* u, bool u_f32, const float* w, const float* bias,
                              float* out, uint16_t* out_hi, uint16_t* out_lo, int64_t batch,
                              int64_t L, int64_t D, int k, hipStream_t stream) {
  if (u_f32)
    return launch_conv_t(static_cast<const float*>(u), w, bias, out, out_hi, out_lo, batch, L, D,
                         k, stream);
  return launch_conv_t(static_cast<const uint16_t*>(u), w, bias, out, out_hi, out_lo, batch, L,
                       D, k, stream);
}

BlockPlan plan_block(int64_t batch, int64_t L, int64_t Dm, int64_t Di, int64_t N, int64_t R,
                     int cpl, bool chain) {
  BlockPlan b;
  const size_t M = static_cast<size_t>(batch * L);
  const size_t di = static_cast<size_t>(Di);
  if (chain) {
    b.chain = true;
    b.scan.chain = true;
  } else {
    b.scan = plan_scan(batch, L, Di, N, cpl);
  }
  size_t off = 0;
  b.u_offset = off;      off += align256(sizeof(float) * M * di);
  b.z_offset = off;      off += align256(sizeof(float) * M * di);
  b.x_offset = off;      off += align256(sizeof(float) * M * di);
  b.xb_offset = off;     off += align256(sizeof(uint16_t) * M * di);
  b.xl_offset = off;     off += align256(sizeof(uint16_t) * M * di);
  b.g_offset = off;      off += align256(sizeof(uint16_t) * M * 2 * di);
  b.p_offset = off;      off += align256(sizeof(float) * M * (size_t)(R + 2 * N));
  b.dtl_offset = off;    off += align256(sizeof(uint16_t) * M * (size_t)R);
  b.dtl_lo_offset = off; off += align256(sizeof(uint16_t) * M * (size_t)R);
  b.wt_offset = off;     off += align256(sizeof(uint16_t) * di * (size_t)R);
  b.win_t_offset = off;  off += align256(sizeof(uint16_t) * 2 * di * (size_t)Dm);
  b.wx_t_offset = off;   off += align256(sizeof(uint16_t) * (size_t)(R + 2 * N) * xproj_padded_k(Di));
  b.wout_t_offset = off; off += align256(sizeof(uint16_t) * (size_t)Dm * 2 * di);
  b.scan_offset = off;   off += b.scan.workspace_bytes;
  if (chain && split_fused_applies(batch, Di, N)) {
    b.bcg_offset = off;  off += align256(sizeof(float) * 4 * 8 * (size_t)xproj_bcg_rows(M));
  }
  b.workspace_bytes = off;
  return b;
}

size_t block_workspace_bound(int64_t batch, int64_t L, int64_t Dm, int64_t Di, int64_t N,
                             int64_t R) {
  size_t w = plan_block(batch, L, Dm, Di, N, R, 1, false).workspace_bytes;
  if (Di % 2 == 0) w = std::max(w, plan_block(batch, L, Dm, Di, N, R, 2, false).workspace_bytes);
  if (N == 16 && Di % 16 == 0 && R <= 256)
    w = std::max(w, plan_block(batch, L, Dm, Di, N, R, 1, true).workspace_bytes);
  return w;
}

FusedStatus launch_block(const BlockArgs& a, const BlockPlan& bp, void* workspace,
                         hipStream_t stream) {
  FusedStatus st;
  char* ws = static_cast<char*>(workspace);
  const int64_t M = a.batch * a.L;
  const int64_t Di = a.Di, Dm = a.Dm, ldp = a.R + 2 * a.N;
  float* U = reinterpret_cast<float*>(ws + bp.u_offset);
  float* Z = reinterpret_cast<float*>(ws + bp.z_offset);
  float* X = reinterpret_cast<float*>(ws + bp.x_offset);
  uint16_t* Xb = reinterpret_cast<uint16_t*>(ws + bp.xb_offset);
  uint16_t* Xl = reinterpret_cast<uint16_t*>(ws + bp.xl_offset);
  // the gated SSM output as a bf16 hi + lo pair: with the single pass the two
  // column halves of one [M, 2 Di] matrix (out_proj is then one GEMM over
  // k = 2 Di against W_out^T stacked twice), else two [M, Di] matrices
  uint16_t* G = reinterpret_cast<uint16_t*>(ws + bp.g_offset);
  uint16_t* Gl = bp.chain ? G + Di : G + M * Di;
  float* P = reinterpret_cast<float*>(ws + bp.p_offset);
  uint16_t* dtl = reinterpret_cast<uint16_t*>(ws + bp.dtl_offset);
  uint16_t* dtl_lo = reinterpret_cast<uint16_t*>(ws + bp.dtl_lo_offset);
  uint16_t* wT = reinterpret_cast<uint16_t*>(ws + bp.wt_offset);
  BlasLease blas(stream);
  if (!blas.ok()) {
    st.hip = blas.hip_error();
    st.blas_failed = st.hip == hipSuccess;
    return st;
  }
  const rocblas_handle hb = blas.get();
  // the weights transposed once per call, so every GEMM reads both operands
  // along k (W_in^T rows 0..Di-1 are u's columns, Di..2Di-1 z's)
  uint16_t* WinT = reinterpret_cast<uint16_t*>(ws + bp.win_t_offset);
  uint16_t* WxT = reinterpret_cast<uint16_t*>(ws + bp.wx_t_offset);
  uint16_t* WoutT = reinterpret_cast<uint16_t*>(ws + bp.wout_t_offset);
  st.hip = launch_transpose_bf16(a.W_in, WinT, Dm, 2 * Di, stream);
  // W_out^T [Dm, 2 Di]: columns Di.. repeat columns 0..Di-1
  if (st.hip == hipSuccess) st.hip = launch_transpose_bf16(a.W_out, WoutT, Di, Dm, stream, 2 * Di);
  if (st.hip == hipSuccess)
    st.hip = launch_transpose_bf16(a.W_out, WoutT + Di, Di, Dm, stream, 2 * Di);
  if (st.hip != hipSuccess) return st;
  // input projection: u = u0 W_in[:, :Di], z = u0 W_in[:, Di:]
  if (!gemm_rm_bf16_bt(hb, M, Di, Dm, a.u0, Dm, WinT, Dm, U, Di, 0.0f) ||
      !gemm_rm_bf16_bt(hb, M, Di, Dm, a.u0, Dm, WinT + Di * Dm, Dm, Z, Di, 0.0f)) {
    st.blas_failed = true;
    return st;
  }
  st.hip = launch_conv1d_silu(U, true, a.conv_w, a.conv_b, X, Xb, Xl, a.batch, a.L, Di, a.k,
                              stream);
  if (st.hip != hipSuccess) return st;
  // selection projection of x = hi + lo (dt_low as its bf16 pair, B and C in P)
  float* bcg = (bp.chain && split_fused_applies(a.batch, Di, a.N))
                   ? reinterpret_cast<float*>(ws + bp.bcg_offset)
                   : nullptr;
  st.hip = launch_xproj(Xb, Xl, Di, M, Di, a.W_x, ldp, a.R, WxT, dtl, dtl_lo, P, ldp, bcg,
                        stream);
  if (st.hip == hipSuccess) st.hip = launch_wdt_transpose(a.W_dt, a.R, Di, wT, stream);
  if (st.hip != hipSuccess) return st;
  if (bp.chain) {
    // the single pass: delta written out (into u, which the conv has consumed)
    st.hip = launch_dtproj_softplus(dtl, dtl_lo, wT, a.dt_bias, U, M, Di, a.R, stream);
    if (st.hip != hipSuccess) return st;
    ChainFusedArgs ca;
    ca.x = X;
    ca.x_f32 = true;
    ca.delta = U;
    ca.P = P;
    ca.ldp = ldp;
    ca.R = a.R;
    ca.A = a.A;
    ca.Dskip = a.Dskip;
    ca.z = Z;
    ca.y = G;
    ca.y_lo = Gl;
    ca.ld_y = 2 * Di;
    ca.y_bf16 = true;
    ca.batch = a.batch;
    ca.L = a.L;
    ca.D = Di;
    ca.bcg = bcg;
    st.hip = launch_chain_fused(ca, stream);
  } else {
    FusedScanArgs sa{};
    sa.x = X;
    sa.x_f32 = true;
    sa.z = Z;
    sa.Dskip = a.Dskip;
    sa.y = G;
    sa.y_bf16 = true;
    sa.y_lo = Gl;
    sa.P = P;
    sa.dtl = dtl;
    sa.dtl_lo = dtl_lo;
    sa.wT = wT;
    sa.dt_bias = a.dt_bias;
    sa.A = a.A;
    if (bp.scan.K > 1) {
      sa.sum_h = reinterpret_cast<float*>(ws + bp.scan_offset);
      sa.sum_s = reinterpret_cast<double*>(ws + bp.scan_offset + bp.scan.sum_s_offset);
    }
    sa.batch = a.batch;
    sa.L = a.L;
    sa.D = Di;
    sa.N = a.N;
    sa.R = a.R;
    st.hip = launch_fused_scan(sa, bp.scan, stream);
  }
  if (st.hip != hipSuccess) return st;
  // output projection of the gated result G = hi + lo
  const bool out_ok =
      bp.chain ? gemm_rm_bf16_bt(hb, M, Dm, 2 * Di, G, 2 * Di, WoutT, 2 * Di, a.out, Dm, 0.0f)
               : gemm_rm_bf16_bt(hb, M, Dm, Di, G, Di, WoutT, 2 * Di, a.out, Dm, 0.0f) &&
                     gemm_rm_bf16_bt(hb, M, Dm, Di, Gl, Di, WoutT, 2 * Di, a.out, Dm, 1.0f);
  if (!out_ok)
    st.blas_failed = true;
  return st;
}

}  // namespace mssm
