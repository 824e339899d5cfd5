// Chunked selective-scan kernels for gfx950 and their launchers.
//
// The recurrence h_t = Abar_t h_{t-1} + Bbar_t x_t is an affine map of the
// previous state, and two consecutive maps compose into one with the pair
// operator (a_i, b_i) . (a_j, b_j) = (a_i a_j, a_j b_i + b_j)
// ("Understanding Mamba", section 7.1, eq. (8)).  Because the operator is
// associative, the sequence is cut into K chunks:
//
//   summary pass  (chunks 0..K-2, all in parallel): scan the chunk from a zero
//                 state; keep its end state hloc_k and its total step size
//                 S_k.  The chunk's decay is prod_t exp(delta_t A) =
//                 exp(S_k A), so the pair for the whole chunk is
//                 (exp(S_k A), hloc_k) and needs N + 1 numbers per chain.
//   output pass   (all chunks in parallel): fold the pairs of the chunks
//                 before this one into the carry-in, then scan the chunk's
//                 steps from it and write y.
//
// Only the summaries ([batch, K-1, N, D] floats and [batch, K-1, D] doubles)
// travel through memory; per-step states stay in registers ("Understanding
// Mamba", section 7.3).  S_k is accumulated in float64 so that exp(S_k A)
// matches the product of the per-step factors to float32 rounding.
#include "mssm_internal.h"
#include "scan_device.h"

#include <algorithm>
#include <cstdlib>

namespace mssm {

constexpr int kBlock = 256;   // 4 wavefronts, 256 consecutive channels

struct BlockCoord {
  int64_t d;      // channel of this lane
  int k;          // chunk
  int64_t b;      // batch row
};

__device__ __forceinline__ BlockCoord block_coord(int64_t n_dtiles, int K) {
  const int64_t bid = blockIdx.x;
  const int64_t dtile = bid % n_dtiles;
  const int64_t rest = bid / n_dtiles;
  BlockCoord c;
  c.k = static_cast<int>(rest % K);
  c.b = rest / K;
  c.d = dtile * kBlock + threadIdx.x;
  return c;
}

template <int N, typename T, bool kPairs>
__global__ __launch_bounds__(kBlock) void chunk_summary_kernel(
    const T* __restrict__ x, const T* __restrict__ delta, const float* __restrict__ A,
    const T* __restrict__ Bm, float* __restrict__ sum_h, double* __restrict__ sum_dt,
    int64_t L, int64_t D, int64_t chunk_len, int K, int64_t n_dtiles) {
  // grid: n_dtiles * (K - 1) * batch blocks; block (dtile, k, b), k < K - 1
  const BlockCoord c = block_coord(n_dtiles, K - 1);
  const bool active = c.d < D;
  const int64_t dl = active ? c.d : D - 1;
  float A2[N], h[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    A2[n] = A[dl * N + n] * kLog2e;
    h[n] = 0.0f;
  }
  const int64_t t0 = (int64_t)c.k * chunk_len;
  const int nsteps = static_cast<int>(chunk_len);   // chunks before the last are full
  double S = 0.0;
  scan_steps<N, T, kPairs, false>(x, delta, Bm, nullptr, nullptr, A2, h, S,
                                  (c.b * L + t0) * D + dl, (c.b * L + t0) * N, D, nsteps,
                                  active);
  if (active) {
    const int64_t row = c.b * (K - 1) + c.k;
#pragma unroll
    for (int n = 0; n < N; ++n) sum_h[(row * N + n) * D + c.d] = h[n];
    sum_dt[row * D + c.d] = S;
  }
}

template <int N, typename T, bool kPairs>
__global__ __launch_bounds__(kBlock) void chunk_output_kernel(
    const T* __restrict__ x, const T* __restrict__ delta, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, float* __restrict__ y,
    const float* __restrict__ sum_h, const double* __restrict__ sum_dt, int64_t L, int64_t D,
    int64_t chunk_len, int K, int64_t n_dtiles) {
  const BlockCoord c = block_coord(n_dtiles, K);
  const bool active = c.d < D;
  const int64_t dl = active ? c.d : D - 1;
  float A2[N], h[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    A2[n] = A[dl * N + n] * kLog2e;
    h[n] = 0.0f;
  }
  // carry-in: fold (exp(S_j A), hloc_j) of chunks j < k, oldest first
  for (int j = 0; j < c.k; ++j) {
    const int64_t row = c.b * (K - 1) + j;
    const double S = sum_dt[row * D + dl];
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const float decay = fast_exp2(static_cast<float>(static_cast<double>(A2[n]) * S));
      h[n] = __builtin_fmaf(decay, h[n], sum_h[(row * N + n) * D + dl]);
    }
  }
  const int64_t t0 = (int64_t)c.k * chunk_len;
  const int nsteps = static_cast<int>(std::min<int64_t>(chunk_len, L - t0));
  double S_unused = 0.0;
  scan_steps<N, T, kPairs, true>(x, delta, Bm, Cm, y, A2, h, S_unused, (c.b * L + t0) * D + dl,
                                 (c.b * L + t0) * N, D, nsteps, active);
}

bool state_size_supported(int64_t N) {
  return N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32;
}

static size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

ScanPlan plan_scan(int64_t batch, int64_t L, int64_t D, int64_t N) {
  ScanPlan p;
  if (batch <= 0 || L <= 0 || D <= 0) return p;
  // Enough wavefronts to give every SIMD of the 256 compute units about two,
  // with chunks no shorter than 64 steps.  MSSM_CHUNK_LEN overrides the
  // chunk length (used for tuning sweeps and chunk-boundary tests).
  const int64_t waves_per_chunk = batch * ((D + 63) / 64);
  const int64_t target_waves = 2048;
  int64_t K = (target_waves + waves_per_chunk - 1) / waves_per_chunk;
  const int64_t min_chunk = 64;
  K = std::max<int64_t>(1, std::min<int64_t>(K, (L + min_chunk - 1) / min_chunk));
  int64_t chunk = (L + K - 1) / K;
  if (const char* env = std::getenv("MSSM_CHUNK_LEN")) {
    const long long v = std::atoll(env);
    if (v > 0) chunk = v;
  }
  const int64_t max_chunk = int64_t(1) << 30;
  chunk = std::min<int64_t>(chunk, max_chunk);
  K = (L + chunk - 1) / chunk;
  if (K > 65535) {   // keep the summary fold short and the grid within limits
    K = 65535;
    chunk = (L + K - 1) / K;
    K = (L + chunk - 1) / chunk;
  }
  p.K = static_cast<int>(K);
  p.chunk_len = chunk;
  if (K > 1) {
    p.sum_h_bytes = round_up(sizeof(float) * (size_t)batch * (size_t)(K - 1) * (size_t)N * (size_t)D, 256);
    p.sum_dt_offset = p.sum_h_bytes;
    p.workspace_bytes = p.sum_dt_offset + round_up(sizeof(double) * (size_t)batch * (size_t)(K - 1) * (size_t)D, 256);
  }
  return p;
}

template <int N, typename T, bool kPairs>
static hipError_t launch_typed(const ScanArgs& a, const ScanPlan& p, void* ws, hipStream_t stream) {
  const T* x = static_cast<const T*>(a.x);
  const T* delta = static_cast<const T*>(a.delta);
  const T* Bm = static_cast<const T*>(a.B);
  const T* Cm = static_cast<const T*>(a.C);
  float* y = static_cast<float*>(a.y);
  const int64_t n_dtiles = (a.D + kBlock - 1) / kBlock;
  float* sum_h = nullptr;
  double* sum_dt = nullptr;
  if (p.K > 1) {
    sum_h = static_cast<float*>(ws);
    sum_dt = reinterpret_cast<double*>(static_cast<char*>(ws) + p.sum_dt_offset);
    const int64_t grid = n_dtiles * (p.K - 1) * a.batch;
    hipLaunchKernelGGL((chunk_summary_kernel<N, T, kPairs>), dim3((unsigned)grid), dim3(kBlock), 0,
                       stream, x, delta, a.A, Bm, sum_h, sum_dt, a.L, a.D, p.chunk_len, p.K,
                       n_dtiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t grid = n_dtiles * p.K * a.batch;
  hipLaunchKernelGGL((chunk_output_kernel<N, T, kPairs>), dim3((unsigned)grid), dim3(kBlock), 0,
                     stream, x, delta, a.A, Bm, Cm, y, sum_h, sum_dt, a.L, a.D, p.chunk_len, p.K,
                     n_dtiles);
  return hipGetLastError();
}

template <int N>
static hipError_t launch_n(const ScanArgs& a, const ScanPlan& p, void* ws, hipStream_t stream) {
  if (a.dtype == MSSM_FLOAT32) return launch_typed<N, float, false>(a, p, ws, stream);
  const bool pairs = (N % 2 == 0) && (reinterpret_cast<uintptr_t>(a.B) % 4 == 0) &&
                     (reinterpret_cast<uintptr_t>(a.C) % 4 == 0);
  if (pairs) return launch_typed<N, uint16_t, true>(a, p, ws, stream);
  return launch_typed<N, uint16_t, false>(a, p, ws, stream);
}

hipError_t launch_scan(const ScanArgs& a, const ScanPlan& p, void* ws, hipStream_t stream) {
  switch (a.N) {
    case 1: return launch_n<1>(a, p, ws, stream);
    case 2: return launch_n<2>(a, p, ws, stream);
    case 4: return launch_n<4>(a, p, ws, stream);
    case 8: return launch_n<8>(a, p, ws, stream);
    case 16: return launch_n<16>(a, p, ws, stream);
    case 32: return launch_n<32>(a, p, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mssm
