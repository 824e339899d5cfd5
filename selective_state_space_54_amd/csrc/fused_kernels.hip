// Fused selective SSM for gfx950: selection projections + scan.
//
// The step size, input and output matrices are read off the tokens
// ("Understanding Mamba", section 5.1, eq. (6)): in the low-rank Mamba shape
// x_proj maps each token (D values) to [dt_low (R) | B_t (N) | C_t (N)], dt_proj
// maps dt_low back to D channels, a per-channel bias is added and softplus
// keeps the step size positive.  Here:
//
//   x_proj  : one plain GEMM P = x @ W_x ([batch*L, D] x [D, R+2N], bf16 in,
//             float32 out) through rocBLAS;
//   prep    : dt_low split into two bfloat16 parts, hi = bf16(P[:, :R]) and
//             lo = bf16(P[:, :R] - hi) (round to nearest even), so the matrix
//             cores see dt_low to about 16 significant bits; W_dt transposed
//             to [D, R];
//   scan    : the same chunked two-pass scan as the plain path, except that
//             Delta never exists in memory: every 32-step tile of a wavefront's
//             channels is computed on the matrix cores (v_mfma_f32_32x32x16_bf16,
//             K = R in steps of 16, hi and lo parts accumulated into the same
//             float32 result), gets its bias and softplus on the vector
//             unit, and is parked in the wavefront's slice of LDS for the step
//             loop.  B_t and C_t are read as float32 rows of P (stride R + 2N)
//             through the scalar unit.
#include <rocblas/rocblas.h>

#include <algorithm>
#include <mutex>

#include "mssm_internal.h"
#include "scan_device.h"

namespace mssm {

namespace {

constexpr int kFBlock = 256;     // 4 wavefronts
constexpr int kDTile = 32;       // steps per Delta tile (rows of one MFMA output block)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  const u32x4 u = *reinterpret_cast<const u32x4*>(p);     // 16-byte aligned by construction
  bf16x8 v;
  __builtin_memcpy(&v, &u, sizeof(v));
  return v;
}

// softplus(z) = ln(1 + e^z) as max(z, 0) + log1p(e^{-|z|}).  log1p(e) is
// log(u) * e / (u - 1) with u = 1 + e rounded (Goldberg's correction), which
// keeps full relative accuracy when e is tiny; u == 1 means log1p(e) = e.
__device__ __forceinline__ float softplus_f(float z) {
  const float e = fast_exp2(-fabsf(z) * kLog2e);
  const float u = 1.0f + e;
  const float um1 = u - 1.0f;
  const float lg = __builtin_amdgcn_logf(u) * 0.69314718055994531f;
  const float l1p = (um1 == 0.0f) ? e : lg * (e * __builtin_amdgcn_rcpf(um1));
  return fmaxf(z, 0.0f) + l1p;
}

// Delta for rows [0, 32) of a tile (steps s0..s0+31 of the chunk) and the
// wavefront's 64*CPL channels, written to lds[row * stride + local channel].
// dtl/dtl_lo: the hi and lo bf16 parts of dt_low at the tile's first step
// (row stride R); rows >= rows_valid
// re-read the last valid row (their results are never used).  wT: W_dt^T bf16
// rows of the wavefront's first channel (row stride R).  bias: float32 for the
// wavefront's first channel.
template <int CPL>
__device__ __forceinline__ void delta_tile(const uint16_t* __restrict__ dtl,
                                           const uint16_t* __restrict__ dtl_lo, int rows_valid,
                                           const uint16_t* __restrict__ wT,
                                           const float* __restrict__ bias, int R,
                                           float* __restrict__ lds, int stride, int lane,
                                           int ch_valid) {
  constexpr int kBlocks = 2 * CPL;          // 32-channel column blocks per wavefront
  f32x16 acc[kBlocks];
#pragma unroll
  for (int nb = 0; nb < kBlocks; ++nb) acc[nb] = f32x16{};
  const int row = min(lane % 32, rows_valid - 1);
  const int khalf = 8 * (lane / 32);
  int ch[kBlocks];
#pragma unroll
  for (int nb = 0; nb < kBlocks; ++nb) ch[nb] = min(nb * 32 + lane % 32, ch_valid - 1);
  for (int kk = 0; kk < R; kk += 16) {
    const bf16x8 a = load_bf16x8(dtl + (int64_t)row * R + kk + khalf);
    const bf16x8 a_lo = load_bf16x8(dtl_lo + (int64_t)row * R + kk + khalf);
#pragma unroll
    for (int nb = 0; nb < kBlocks; ++nb) {
      const bf16x8 b = load_bf16x8(wT + (int64_t)ch[nb] * R + kk + khalf);
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[nb], 0, 0, 0);
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo, b, acc[nb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int nb = 0; nb < kBlocks; ++nb) {
    const float bv = bias[ch[nb]];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // output element (row m, column n) of the 32x32 block held by this lane/register
      const int m = 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
      lds[m * stride + nb * 32 + lane % 32] = softplus_f(acc[nb][r] + bv);
    }
  }
}

// The fused step loop: as scan_steps, with Delta from the LDS tile and B/C
// float32 rows of P (row stride ldbc floats).
template <int N, int CPL, bool kWithY>
__device__ __forceinline__ void fused_steps(const uint16_t* __restrict__ xb,
                                            const uint16_t* __restrict__ dtl,
                                            const uint16_t* __restrict__ dtl_lo,
                                            const uint16_t* __restrict__ wT,
                                            const float* __restrict__ bias, int R,
                                            const float* __restrict__ Bb, const float* __restrict__ Cb,
                                            int64_t ldbc, float* __restrict__ yb,
                                            const float (&A2)[CPL][N], float (&h)[CPL][N],
                                            double (&S)[CPL], int wlane, int wave_ch0, int ch_valid,
                                            int64_t D, int nsteps, float* __restrict__ lds,
                                            int stride) {
  constexpr int kTile = (CPL == 1) ? 8 : 4;
  const uint32_t in_bytes = static_cast<uint32_t>((int64_t)nsteps * D * sizeof(uint16_t));
  const buf_t xr = make_buf(xb, in_bytes);
  const int in_row = static_cast<int>(D * sizeof(uint16_t));
  const int lane_blk = wave_ch0 + wlane * CPL;   // lane's first channel inside the block
  const int in_lane = lane_blk * static_cast<int>(sizeof(uint16_t));
  buf_t yr;
  int out_row = 0, out_lane = 0;
  if constexpr (kWithY) {
    yr = make_buf(yb, static_cast<uint32_t>((int64_t)nsteps * D * sizeof(float)));
    out_row = static_cast<int>(D * sizeof(float));
    out_lane = lane_blk * static_cast<int>(sizeof(float));
  }
  const int last = nsteps > 0 ? nsteps - 1 : 0;
  float xc[kTile][CPL];
#pragma unroll
  for (int j = 0; j < kTile; ++j) {
    const int soff = __builtin_amdgcn_readfirstlane(min(j, last) * in_row);
    buf_load_vals<uint16_t, CPL>(xr, in_lane, soff, xc[j]);
  }
  float Bv[2][N], Cv[2][N];
  if (nsteps > 0) {
    load_row<N>(Bb, Bv[0]);
    if constexpr (kWithY) load_row<N>(Cb, Cv[0]);
  }
  for (int base = 0; base < nsteps; base += kTile) {
    if (base % kDTile == 0)
      delta_tile<CPL>(dtl + (int64_t)base * R, dtl_lo + (int64_t)base * R,
                      min(kDTile, nsteps - base), wT, bias, R, lds, stride,
                      static_cast<int>(threadIdx.x % 64), ch_valid);
    float xn[kTile][CPL];
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      const int soff = __builtin_amdgcn_readfirstlane(min(base + kTile + j, last) * in_row);
      buf_load_vals<uint16_t, CPL>(xr, in_lane, soff, xn[j]);
    }
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      const int s = base + j;
      if (s < nsteps) {
        const int cur = j & 1;
        wait_scalar_loads();
        if (s + 1 < nsteps) {
          load_row<N>(Bb + (int64_t)(s + 1) * ldbc, Bv[cur ^ 1]);
          if constexpr (kWithY) load_row<N>(Cb + (int64_t)(s + 1) * ldbc, Cv[cur ^ 1]);
        }
        const float* drow = lds + (s % kDTile) * stride + wlane * CPL;
        float dt[CPL], dx[CPL], yv[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          dt[c] = drow[c];
          dx[c] = dt[c] * xc[j][c];
          yv[c] = 0.0f;
        }
#pragma unroll
        for (int n = 0; n < N; ++n) {
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const float a = fast_exp2(dt[c] * A2[c][n]);
            h[c][n] = __builtin_fmaf(a, h[c][n], dx[c] * Bv[cur][n]);
            if constexpr (kWithY) yv[c] = __builtin_fmaf(Cv[cur][n], h[c][n], yv[c]);  // C . h
          }
        }
        if constexpr (kWithY) {
          // lanes past the last channel repeat the last valid channel (clamped
          // addressing), so they store the same value to the same place
          buf_store_vals<CPL>(yr, out_lane, s * out_row, yv);
        } else {
#pragma unroll
          for (int c = 0; c < CPL; ++c) S[c] += static_cast<double>(dt[c]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kTile; ++j)
#pragma unroll
      for (int c = 0; c < CPL; ++c) xc[j][c] = xn[j][c];
  }
}

struct FusedCoord {
  int64_t d0;       // first channel of the block
  int wave_ch0;     // first channel of this wavefront inside the block
  int wlane;        // lane index inside the wavefront (clamped if inactive)
  bool active;
  int ch_valid;     // channels of this wavefront that exist (>= 1)
  int k;
  int64_t b;
};

template <int CPL>
__device__ __forceinline__ FusedCoord fused_coord(int64_t n_dtiles, int K, int64_t D) {
  const int64_t bid = blockIdx.x;
  const int64_t dtile = bid % n_dtiles;
  const int64_t rest = bid / n_dtiles;
  FusedCoord c;
  c.k = static_cast<int>(rest % K);
  c.b = rest / K;
  c.d0 = dtile * kFBlock * CPL;
  const int wave = threadIdx.x / 64;
  c.wave_ch0 = wave * 64 * CPL;
  const int64_t wave_first = c.d0 + c.wave_ch0;
  const int64_t left = D - wave_first;                       // channels from this wave on
  c.ch_valid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(64 * CPL, left)));
  const int lane = threadIdx.x % 64;
  c.active = (int64_t)lane * CPL < left;
  c.wlane = c.active ? lane : (c.ch_valid - 1) / CPL;
  return c;
}

template <int CPL>
constexpr int lds_stride() { return 64 * CPL + 2 * CPL; }   // padded against bank conflicts

template <int N, int CPL>
__global__ __launch_bounds__(kFBlock) void fused_summary_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ dtlow,
    const uint16_t* __restrict__ dtlow_lo,
    const uint16_t* __restrict__ wT, const float* __restrict__ bias,
    const float* __restrict__ A, const float* __restrict__ P, float* __restrict__ sum_h,
    float* __restrict__ sum_p, int64_t L, int64_t D, int R, int64_t chunk_len, int K,
    int64_t n_dtiles) {
  __shared__ float lds_all[4][kDTile * lds_stride<CPL>()];
  const FusedCoord c = fused_coord<CPL>(n_dtiles, K - 1, D);
  if (c.d0 + c.wave_ch0 >= D) return;   // wavefront past the last channel (no barriers here)
  float* lds = lds_all[threadIdx.x / 64];
  const int64_t wave_d = c.d0 + c.wave_ch0;
  const int64_t dl = wave_d + (int64_t)c.wlane * CPL;
  float A2[CPL][N], h[CPL][N];
  double S[CPL];
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    S[q] = 0.0;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      A2[q][n] = A[(dl + q) * N + n] * kLog2e;
      h[q][n] = 0.0f;
    }
  }
  const int64_t t0 = (int64_t)c.k * chunk_len;
  const int nsteps = static_cast<int>(chunk_len);
  const int64_t ldbc = R + 2 * N;
  const int64_t tok0 = c.b * L + t0;
  fused_steps<N, CPL, false>(x + tok0 * D + c.d0, dtlow + tok0 * R, dtlow_lo + tok0 * R,
                             wT + wave_d * R, bias + wave_d,
                             R, P + tok0 * ldbc + R, nullptr, ldbc, nullptr, A2, h, S, c.wlane,
                             c.wave_ch0, c.ch_valid, D, nsteps, lds, lds_stride<CPL>());
  if (c.active) {
    const int64_t row = c.b * (K - 1) + c.k;
#pragma unroll
    for (int q = 0; q < CPL; ++q)
#pragma unroll
      for (int n = 0; n < N; ++n) {
        sum_h[(row * N + n) * D + dl + q] = h[q][n];
        sum_p[(row * N + n) * D + dl + q] =
            fast_exp2(static_cast<float>(static_cast<double>(A2[q][n]) * S[q]));
      }
  }
}

template <int N, int CPL>
__global__ __launch_bounds__(kFBlock) void fused_output_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ dtlow,
    const uint16_t* __restrict__ dtlow_lo,
    const uint16_t* __restrict__ wT, const float* __restrict__ bias,
    const float* __restrict__ A, const float* __restrict__ P, const float* __restrict__ sum_h,
    float* __restrict__ y, int64_t L, int64_t D, int R, int64_t chunk_len, int K,
    int64_t n_dtiles) {
  __shared__ float lds_all[4][kDTile * lds_stride<CPL>()];
  const FusedCoord c = fused_coord<CPL>(n_dtiles, K, D);
  if (c.d0 + c.wave_ch0 >= D) return;   // wavefront past the last channel (no barriers here)
  float* lds = lds_all[threadIdx.x / 64];
  const int64_t wave_d = c.d0 + c.wave_ch0;
  const int64_t dl = wave_d + (int64_t)c.wlane * CPL;
  float A2[CPL][N], h[CPL][N];
  double S_unused[CPL];
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    S_unused[q] = 0.0;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      A2[q][n] = A[(dl + q) * N + n] * kLog2e;
      h[q][n] = 0.0f;
    }
  }
  if (c.k > 0) {
    const float* cp = sum_h + ((c.b * (K - 1) + (c.k - 1)) * N) * D + dl;
#pragma unroll
    for (int q = 0; q < CPL; ++q)
#pragma unroll
      for (int n = 0; n < N; ++n) h[q][n] = cp[(int64_t)n * D + q];
  }
  const int64_t t0 = (int64_t)c.k * chunk_len;
  const int nsteps = static_cast<int>(std::min<int64_t>(chunk_len, L - t0));
  const int64_t ldbc = R + 2 * N;
  const int64_t tok0 = c.b * L + t0;
  fused_steps<N, CPL, true>(x + tok0 * D + c.d0, dtlow + tok0 * R, dtlow_lo + tok0 * R,
                            wT + wave_d * R, bias + wave_d,
                            R, P + tok0 * ldbc + R, P + tok0 * ldbc + R + N, ldbc,
                            y + tok0 * D + c.d0, A2, h, S_unused, c.wlane, c.wave_ch0, c.ch_valid,
                            D, nsteps, lds, lds_stride<CPL>());
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  uint32_t v = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  if ((u & 0x7fffffffu) > 0x7f800000u) v = (u >> 16) | 0x40u;   // NaN stays NaN
  return static_cast<uint16_t>(v);
}

// hi[m, r] = bf16(P[m, r]), lo[m, r] = bf16(P[m, r] - hi[m, r]) (round to nearest
// even), m < M, r < R: hi + lo carries P to about 16 significant bits.
__global__ void dtlow_split_kernel(const float* __restrict__ P, uint16_t* __restrict__ hi,
                                   uint16_t* __restrict__ lo, int64_t M, int R, int64_t ldp) {
  const int64_t total = M * R;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / R;
    const int r = static_cast<int>(i % R);
    const float v = P[m * ldp + r];
    const uint16_t h = bf16_rne(v);
    hi[i] = h;
    lo[i] = bf16_rne(v - __uint_as_float(static_cast<uint32_t>(h) << 16));
  }
}

// wT[d, r] = W[r, d]
__global__ void transpose_bf16_kernel(const uint16_t* __restrict__ W, uint16_t* __restrict__ wT,
                                      int R, int64_t D) {
  const int64_t total = (int64_t)R * D;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t d = i / R;
    const int r = static_cast<int>(i % R);
    wT[i] = W[(int64_t)r * D + d];
  }
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// one rocBLAS handle per device, created on first use and kept until exit
std::mutex g_blas_mutex;
rocblas_handle g_blas[64] = {};

}  // namespace

FusedPlan plan_fused(int64_t batch, int64_t L, int64_t D, int64_t N, int64_t R, int cpl) {
  FusedPlan f;
  const int64_t M = batch * L;
  f.scan = plan_scan(batch, L, D, N, cpl);
  f.p_bytes = align256(sizeof(float) * (size_t)M * (size_t)(R + 2 * N));
  f.dtl_offset = f.p_bytes;
  f.dtl_lo_offset = f.dtl_offset + align256(sizeof(uint16_t) * (size_t)M * (size_t)R);
  f.wt_offset = f.dtl_lo_offset + align256(sizeof(uint16_t) * (size_t)M * (size_t)R);
  f.scan_offset = f.wt_offset + align256(sizeof(uint16_t) * (size_t)D * (size_t)R);
  f.workspace_bytes = f.scan_offset + f.scan.workspace_bytes;
  return f;
}

size_t fused_workspace_bound(int64_t batch, int64_t L, int64_t D, int64_t N, int64_t R) {
  size_t w = plan_fused(batch, L, D, N, R, 1).workspace_bytes;
  if (D % 2 == 0) w = std::max(w, plan_fused(batch, L, D, N, R, 2).workspace_bytes);
  return w;
}

int choose_fused_cpl(int64_t D) {
  if (const char* env = std::getenv("MSSM_CPL")) {       // tuning experiments only
    if (std::atoi(env) == 1) return 1;
  }
  return D % 2 == 0 ? 2 : 1;
}

template <int N, int CPL>
static hipError_t launch_fused_scan(const FusedArgs& a, const FusedPlan& f, char* ws,
                                    hipStream_t stream) {
  const ScanPlan& p = f.scan;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const float* P = reinterpret_cast<const float*>(ws);
  const uint16_t* dtl = reinterpret_cast<const uint16_t*>(ws + f.dtl_offset);
  const uint16_t* dtl_lo = reinterpret_cast<const uint16_t*>(ws + f.dtl_lo_offset);
  const uint16_t* wT = reinterpret_cast<const uint16_t*>(ws + f.wt_offset);
  float* sum_h = nullptr;
  float* sum_p = nullptr;
  const int64_t n_dtiles = (a.D + kFBlock * CPL - 1) / (kFBlock * CPL);
  const int R = static_cast<int>(a.R);
  if (p.K > 1) {
    sum_h = reinterpret_cast<float*>(ws + f.scan_offset);
    sum_p = reinterpret_cast<float*>(ws + f.scan_offset + p.sum_p_offset);
    const int64_t grid = n_dtiles * (p.K - 1) * a.batch;
    hipLaunchKernelGGL((fused_summary_kernel<N, CPL>), dim3((unsigned)grid), dim3(kFBlock), 0, stream,
                       x, dtl, dtl_lo, wT, a.dt_bias, a.A, P, sum_h, sum_p, a.L, a.D, R, p.chunk_len,
                       p.K,
                       n_dtiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_carry(sum_h, sum_p, nullptr, a.batch, a.D, a.N, p.K, stream);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = n_dtiles * p.K * a.batch;
  hipLaunchKernelGGL((fused_output_kernel<N, CPL>), dim3((unsigned)grid), dim3(kFBlock), 0, stream,
                     x, dtl, dtl_lo, wT, a.dt_bias, a.A, P, sum_h, a.y, a.L, a.D, R, p.chunk_len,
                     p.K,
                     n_dtiles);
  return hipGetLastError();
}

template <int N>
static hipError_t launch_fused_n(const FusedArgs& a, const FusedPlan& f, char* ws,
                                 hipStream_t stream) {
  return f.scan.cpl == 2 ? launch_fused_scan<N, 2>(a, f, ws, stream)
                         : launch_fused_scan<N, 1>(a, f, ws, stream);
}

FusedStatus launch_fused(const FusedArgs& a, const FusedPlan& f, void* workspace,
                         hipStream_t stream) {
  FusedStatus st;
  char* ws = static_cast<char*>(workspace);
  float* P = reinterpret_cast<float*>(ws);
  const int64_t M = a.batch * a.L;
  const int64_t ldp = a.R + 2 * a.N;
  // x_proj on rocBLAS (column-major view: P^T[ldp, M] = W_x^T[ldp, D] * x^T[D, M])
  {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) { st.hip = e; return st; }
    if (dev < 0 || dev >= 64) { st.hip = hipErrorInvalidDevice; return st; }
    std::lock_guard<std::mutex> lock(g_blas_mutex);
    if (!g_blas[dev]) {
      if (rocblas_create_handle(&g_blas[dev]) != rocblas_status_success) {
        g_blas[dev] = nullptr;
        st.blas_failed = true;
        return st;
      }
    }
    rocblas_handle hb = g_blas[dev];
    if (rocblas_set_stream(hb, stream) != rocblas_status_success) { st.blas_failed = true; return st; }
    const float alpha = 1.0f, beta = 0.0f;
    const rocblas_status bs = rocblas_gemm_ex(
        hb, rocblas_operation_none, rocblas_operation_none, (rocblas_int)ldp, (rocblas_int)M,
        (rocblas_int)a.D, &alpha, a.W_x, rocblas_datatype_bf16_r, (rocblas_int)ldp, a.x,
        rocblas_datatype_bf16_r, (rocblas_int)a.D, &beta, P, rocblas_datatype_f32_r,
        (rocblas_int)ldp, P, rocblas_datatype_f32_r, (rocblas_int)ldp, rocblas_datatype_f32_r,
        rocblas_gemm_algo_standard, 0, 0);
    if (bs != rocblas_status_success) { st.blas_failed = true; return st; }
  }
  uint16_t* dtl = reinterpret_cast<uint16_t*>(ws + f.dtl_offset);
  uint16_t* dtl_lo = reinterpret_cast<uint16_t*>(ws + f.dtl_lo_offset);
  uint16_t* wT = reinterpret_cast<uint16_t*>(ws + f.wt_offset);
  hipLaunchKernelGGL(dtlow_split_kernel, dim3(2048), dim3(256), 0, stream, P, dtl, dtl_lo, M,
                     static_cast<int>(a.R), ldp);
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3(1024), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a.W_dt), wT, static_cast<int>(a.R), a.D);
  st.hip = hipGetLastError();
  if (st.hip != hipSuccess) return st;
  switch (a.N) {
    case 1: st.hip = launch_fused_n<1>(a, f, ws, stream); break;
    case 2: st.hip = launch_fused_n<2>(a, f, ws, stream); break;
    case 4: st.hip = launch_fused_n<4>(a, f, ws, stream); break;
    case 8: st.hip = launch_fused_n<8>(a, f, ws, stream); break;
    case 16: st.hip = launch_fused_n<16>(a, f, ws, stream); break;
    case 32: st.hip = launch_fused_n<32>(a, f, ws, stream); break;
    default: st.hip = hipErrorInvalidValue;
  }
  return st;
}

}  // namespace mssm
