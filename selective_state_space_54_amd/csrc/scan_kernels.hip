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
//   carry pass    (per chain and state index): walk the chunk pairs in time
//                 order, c_{k+1} = P_k c_k + hloc_k, giving the state that
//                 enters every chunk.
//   output pass   (all chunks in parallel): scan the chunk's steps from its
//                 carry-in and write y.
//
// Only the summaries (two [batch, K-1, N, D] float arrays: hloc and the decay
// P = exp(S A)) travel through memory; per-step states stay in registers
// ("Understanding Mamba", section 7.3).  S_k is accumulated in float64 so
// that exp(S_k A) matches the product of the per-step factors to float32
// rounding.
#include "mssm_internal.h"
#include "scan_device.h"

#include <algorithm>
#include <cstdlib>

namespace mssm {

constexpr int kBlock = 256;   // 4 wavefronts; a block covers 256 * CPL consecutive channels

struct BlockCoord {
  int64_t d0;     // first channel of the block
  int64_t d;      // first channel of this lane (it owns d .. d + CPL - 1)
  int lane;       // lane index used for addressing; clamped to the last lane if inactive
  bool active;    // d < D
  int k;          // chunk
  int64_t b;      // batch row
};

template <int CPL>
__device__ __forceinline__ BlockCoord block_coord(int64_t n_dtiles, int K, int64_t D) {
  const int64_t bid = blockIdx.x;
  const int64_t dtile = bid % n_dtiles;
  const int64_t rest = bid / n_dtiles;
  BlockCoord c;
  c.k = static_cast<int>(rest % K);
  c.b = rest / K;
  c.d0 = dtile * kBlock * CPL;
  c.d = c.d0 + (int64_t)CPL * threadIdx.x;
  c.active = c.d < D;       // D is a multiple of CPL
  c.lane = c.active ? static_cast<int>(threadIdx.x) : static_cast<int>((D - c.d0) / CPL - 1);
  return c;
}

template <int N, int CPL, typename T, bool kPairs>
__global__ __launch_bounds__(kBlock) void chunk_summary_kernel(
    const T* __restrict__ x, const T* __restrict__ delta, const float* __restrict__ A,
    const T* __restrict__ Bm, float* __restrict__ sum_h, float* __restrict__ sum_p,
    int64_t L, int64_t D, int64_t chunk_len, int K, int64_t n_dtiles) {
  // grid: n_dtiles * (K - 1) * batch blocks; block (dtile, k, b), k < K - 1
  const BlockCoord c = block_coord<CPL>(n_dtiles, K - 1, D);
  const int64_t dl = c.d0 + (int64_t)CPL * c.lane;
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
  const int nsteps = static_cast<int>(chunk_len);   // chunks before the last are full
  const int64_t row0 = (c.b * L + t0) * D + c.d0;
  scan_steps<N, CPL, T, kPairs, false>(x + row0, delta + row0, Bm + (c.b * L + t0) * N, nullptr,
                                       nullptr, A2, h, S, c.lane, D, nsteps);
  if (c.active) {
    const int64_t row = c.b * (K - 1) + c.k;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
#pragma unroll
      for (int n = 0; n < N; ++n) {
        sum_h[(row * N + n) * D + c.d + q] = h[q][n];
        // the chunk's decay prod_t exp(delta_t A) = exp(S A); S was summed in float64
        sum_p[(row * N + n) * D + c.d + q] =
            fast_exp2(static_cast<float>(static_cast<double>(A2[q][n]) * S[q]));
      }
    }
  }
}

// Carry pass: one lane per (batch row, state n, channel d).  Walks the chunk
// pairs in time order, c_{j+1} = P_j c_j + hloc_j (c_0 = 0), and overwrites
// hloc_j with c_{j+1}, the state entering chunk j + 1.  The loads of up to
// kBatch chunks are all issued before the dependent multiply-add chain, so a
// lane pays one memory latency per kBatch chunks.
__global__ __launch_bounds__(kBlock) void chunk_carry_kernel(float* __restrict__ sum_h,
                                                             const float* __restrict__ sum_p,
                                                             int64_t D, int N, int K,
                                                             int64_t n_dtiles) {
  constexpr int kBatch = 32;
  const int64_t bid = blockIdx.x;
  const int64_t dtile = bid % n_dtiles;
  const int64_t rest = bid / n_dtiles;
  const int n = static_cast<int>(rest % N);
  const int64_t b = rest / N;
  const int64_t d = dtile * kBlock + threadIdx.x;
  if (d >= D) return;                       // no barriers in this kernel
  const int64_t stride = (int64_t)N * D;    // from chunk j to chunk j + 1
  float* hp = sum_h + (b * (K - 1) * N + n) * D + d;
  const float* pp = sum_p + (b * (K - 1) * N + n) * D + d;
  float c = 0.0f;
  for (int j0 = 0; j0 < K - 1; j0 += kBatch) {
    float hv[kBatch], pv[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (j0 + i < K - 1) {
        hv[i] = hp[(int64_t)(j0 + i) * stride];
        pv[i] = pp[(int64_t)(j0 + i) * stride];
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (j0 + i < K - 1) {
        c = __builtin_fmaf(pv[i], c, hv[i]);
        hp[(int64_t)(j0 + i) * stride] = c;
      }
    }
  }
}

template <int N, int CPL, typename T, bool kPairs>
__global__ __launch_bounds__(kBlock) void chunk_output_kernel(
    const T* __restrict__ x, const T* __restrict__ delta, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, float* __restrict__ y,
    const float* __restrict__ sum_h, int64_t L, int64_t D, int64_t chunk_len, int K,
    int64_t n_dtiles) {
  const BlockCoord c = block_coord<CPL>(n_dtiles, K, D);
  const int64_t dl = c.d0 + (int64_t)CPL * c.lane;
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
  // carry-in: the state entering chunk k, left by the carry pass in slot k - 1
  if (c.k > 0) {
    const float* cp = sum_h + ((c.b * (K - 1) + (c.k - 1)) * N) * D + dl;
#pragma unroll
    for (int q = 0; q < CPL; ++q)
#pragma unroll
      for (int n = 0; n < N; ++n) h[q][n] = cp[(int64_t)n * D + q];
  }
  const int64_t t0 = (int64_t)c.k * chunk_len;
  const int nsteps = static_cast<int>(std::min<int64_t>(chunk_len, L - t0));
  const int64_t row0 = (c.b * L + t0) * D + c.d0;
  scan_steps<N, CPL, T, kPairs, true>(x + row0, delta + row0, Bm + (c.b * L + t0) * N,
                                      Cm + (c.b * L + t0) * N, y + row0, A2, h, S_unused, c.lane,
                                      D, nsteps);
}

bool state_size_supported(int64_t N) {
  return N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32;
}

static size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Two chains per lane pay off for bfloat16 inputs (one 32-bit load brings both
// channels' x and delta; MI355X sweeps: about 10-13% faster), not for float32
// (register pressure lowers occupancy more than the extra ILP gains).
hipError_t launch_carry(float* sum_h, const float* sum_p, int64_t batch, int64_t D, int64_t N,
                        int K, hipStream_t stream) {
  const int64_t carry_tiles = (D + kBlock - 1) / kBlock;
  const int64_t cgrid = carry_tiles * N * batch;
  hipLaunchKernelGGL(chunk_carry_kernel, dim3((unsigned)cgrid), dim3(kBlock), 0, stream, sum_h,
                     sum_p, D, static_cast<int>(N), K, carry_tiles);
  return hipGetLastError();
}

int default_cpl(int64_t D, mssm_dtype dtype) {
  if (const char* env = std::getenv("MSSM_CPL")) {       // tuning experiments only
    const int v = std::atoi(env);
    if (v == 1 || v == 2) return (v == 2 && D % 2 == 0) ? 2 : 1;
  }
  return (dtype == MSSM_BFLOAT16 && D % 2 == 0) ? 2 : 1;
}

ScanPlan plan_scan(int64_t batch, int64_t L, int64_t D, int64_t N, int cpl) {
  ScanPlan p;
  p.cpl = cpl;
  if (batch <= 0 || L <= 0 || D <= 0) return p;
  // Chunk count: enough blocks to give every compute unit about eight (two
  // wavefronts per SIMD over the kernel's life), with chunks of at least 64
  // steps (128 with two chains per lane).  Measured on MI355X with chunk-length sweeps of the synthetic
  // workloads (the per-chunk cost after the carry pass is small, so more
  // chunks help until chunks get short).  MSSM_CHUNK_LEN overrides the chunk
  // length (tuning sweeps and chunk-boundary tests).
  const int64_t blocks_per_chunk = batch * ((D + kBlock * cpl - 1) / (kBlock * cpl));
  const int64_t target_blocks = 2048;
  int64_t K = (target_blocks + blocks_per_chunk / 2) / blocks_per_chunk;
  const int64_t min_chunk = cpl == 1 ? 64 : 128;
  K = std::max<int64_t>(1, std::min<int64_t>(K, L / min_chunk));
  int64_t chunk = (L + K - 1) / K;
  if (const char* env = std::getenv("MSSM_CHUNK_LEN")) {
    const long long v = std::atoll(env);
    if (v > 0) chunk = v;
  }
  // buffer offsets inside one chunk are 32-bit: keep chunk * D * 4 < 2^31
  const int64_t max_chunk = std::max<int64_t>(1, ((int64_t(1) << 31) - 1) / (D * 4));
  chunk = std::min<int64_t>(chunk, max_chunk);
  K = (L + chunk - 1) / chunk;
  if (K > 65535) {
    K = 65535;
    chunk = (L + K - 1) / K;
    K = (L + chunk - 1) / chunk;
  }
  p.K = static_cast<int>(K);
  p.chunk_len = chunk;
  if (K > 1) {
    p.sum_h_bytes = round_up(sizeof(float) * (size_t)batch * (size_t)(K - 1) * (size_t)N * (size_t)D, 256);
    p.sum_p_offset = p.sum_h_bytes;
    p.workspace_bytes = 2 * p.sum_h_bytes;
  }
  return p;
}

size_t workspace_bound(int64_t batch, int64_t L, int64_t D, int64_t N) {
  size_t w = plan_scan(batch, L, D, N, 1).workspace_bytes;
  if (D % 2 == 0) w = std::max(w, plan_scan(batch, L, D, N, 2).workspace_bytes);
  return w;
}

int choose_cpl(const ScanArgs& a) {
  int cpl = default_cpl(a.D, a.dtype);
  const size_t align = 2 * (a.dtype == MSSM_FLOAT32 ? 4 : 2);
  if (cpl == 2 && (reinterpret_cast<uintptr_t>(a.x) % align != 0 ||
                   reinterpret_cast<uintptr_t>(a.delta) % align != 0 ||
                   reinterpret_cast<uintptr_t>(a.y) % 8 != 0))
    cpl = 1;
  return cpl;
}

template <int N, int CPL, typename T, bool kPairs>
static hipError_t launch_typed(const ScanArgs& a, const ScanPlan& p, void* ws, hipStream_t stream) {
  const T* x = static_cast<const T*>(a.x);
  const T* delta = static_cast<const T*>(a.delta);
  const T* Bm = static_cast<const T*>(a.B);
  const T* Cm = static_cast<const T*>(a.C);
  float* y = static_cast<float*>(a.y);
  const int64_t n_dtiles = (a.D + kBlock * CPL - 1) / (kBlock * CPL);
  float* sum_h = nullptr;
  float* sum_p = nullptr;
  if (p.K > 1) {
    sum_h = static_cast<float*>(ws);
    sum_p = reinterpret_cast<float*>(static_cast<char*>(ws) + p.sum_p_offset);
    const int64_t grid = n_dtiles * (p.K - 1) * a.batch;
    hipLaunchKernelGGL((chunk_summary_kernel<N, CPL, T, kPairs>), dim3((unsigned)grid),
                       dim3(kBlock), 0, stream, x, delta, a.A, Bm, sum_h, sum_p, a.L, a.D,
                       p.chunk_len, p.K, n_dtiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_carry(sum_h, sum_p, a.batch, a.D, N, p.K, stream);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = n_dtiles * p.K * a.batch;
  hipLaunchKernelGGL((chunk_output_kernel<N, CPL, T, kPairs>), dim3((unsigned)grid), dim3(kBlock),
                     0, stream, x, delta, a.A, Bm, Cm, y, sum_h, a.L, a.D, p.chunk_len, p.K,
                     n_dtiles);
  return hipGetLastError();
}

template <int N, int CPL>
static hipError_t launch_nc(const ScanArgs& a, const ScanPlan& p, void* ws, hipStream_t stream) {
  if (a.dtype == MSSM_FLOAT32) return launch_typed<N, CPL, float, false>(a, p, ws, stream);
  const bool pairs = (N % 2 == 0) && (reinterpret_cast<uintptr_t>(a.B) % 4 == 0) &&
                     (reinterpret_cast<uintptr_t>(a.C) % 4 == 0);
  if (pairs) return launch_typed<N, CPL, uint16_t, true>(a, p, ws, stream);
  return launch_typed<N, CPL, uint16_t, false>(a, p, ws, stream);
}

template <int N>
static hipError_t launch_n(const ScanArgs& a, const ScanPlan& p, void* ws, hipStream_t stream) {
  return p.cpl == 2 ? launch_nc<N, 2>(a, p, ws, stream) : launch_nc<N, 1>(a, p, ws, stream);
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
