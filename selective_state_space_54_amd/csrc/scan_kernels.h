// Chunked selective-scan kernels for gfx950 (templates; the launchers that
// instantiate them live in one small source file per variant so the build
// compiles them in parallel).
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
//                 (exp(S_k A), hloc_k) and needs N + 1 numbers per chain
//                 (N floats and S_k as one double).
//   carry pass    (per chain and state index): walk the chunk pairs in time
//                 order, c_{k+1} = P_k c_k + hloc_k from c_0 = h0, giving the
//                 state that enters every chunk.
//   output pass   (all chunks in parallel): scan the chunk's steps from its
//                 carry-in and write y; the last chunk also writes the final
//                 state when asked.
//
// Only the summaries (hloc as [batch, K-1, N, D] floats and S as
// [batch, K-1, D] doubles) travel through memory; per-step states stay in
// registers ("Understanding Mamba", section 7.3).  S_k is accumulated in
// float64 so that exp(S_k A) matches the product of the per-step factors to
// float32 rounding.  The decay does not depend on the input term, so the summary
// pass differs between the first-order and the zero-order-hold forms only in
// Bbar.
#pragma once

#include <algorithm>

#include "mssm_internal.h"
#include "scan_device.h"

namespace mssm {

constexpr int kBlock = 256;   // 4 wavefronts; a block covers 256 * CPL consecutive channels

// Everything a chunk kernel reads or writes.  Element pointers are typed by
// the kernel (float or bfloat16 bits).  The kernels take the pointers as
// separate __restrict__ parameters: only then can the compiler prove that the
// stores to y never overwrite B and C, which lets it read B_t and C_t with
// scalar loads into SGPRs (shared by the wavefront) instead of vector loads.
struct ScanParams {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;   // [D] or null
  const void* z;        // [batch, L, D] or null
  const float* h0;      // [batch, D, N] or null (zero start)
  float* h_last;        // [batch, D, N] or null
  float* y;
  float* sum_h;         // chunk end states from zero, [batch, K-1, N, D]
  double* sum_s;        // chunk step-size totals, [batch, K-1, D]
  int64_t L, D, chunk_len;
  int K;
  int64_t n_dtiles;
};

// The sizes part of ScanParams, passed by value next to the pointers.
struct ScanDims {
  int64_t L, D, chunk_len;
  int K;
  int64_t n_dtiles;
};

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

// Per-lane constants for channels dl .. dl + CPL - 1.
template <int N, int CPL, class V>
__device__ __forceinline__ void load_chain_consts(const float* __restrict__ A,
                                                  const float* __restrict__ Dskip, int64_t dl,
                                                  ChainConsts<N, CPL>& k) {
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const float a = A[(dl + q) * N + n];
      k.A2[q][n] = a * kLog2e;
      if constexpr (V::kZoh) k.Ainv[q][n] = 1.0f / a;
    }
    if constexpr (V::kSkip) k.Dd[q] = Dskip[dl + q];
  }
}

template <int N, int CPL, typename T, bool kPairs, bool kZoh>
__global__ __launch_bounds__(kBlock) void chunk_summary_kernel(
    const T* __restrict__ x, const T* __restrict__ delta, const float* __restrict__ A,
    const T* __restrict__ Bm, float* __restrict__ sum_h, double* __restrict__ sum_s, ScanDims dm) {
  using V = Variant<kZoh, false, false>;
  // grid: n_dtiles * (K - 1) * batch blocks; block (dtile, k, b), k < K - 1
  const int64_t D = dm.D, L = dm.L;
  const int K = dm.K;
  const BlockCoord c = block_coord<CPL>(dm.n_dtiles, K - 1, D);
  const int64_t dl = c.d0 + (int64_t)CPL * c.lane;
  ChainConsts<N, CPL> k;
  load_chain_consts<N, CPL, V>(A, nullptr, dl, k);
  float h[CPL][N];
  double S[CPL];
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    S[q] = 0.0;
#pragma unroll
    for (int n = 0; n < N; ++n) h[q][n] = 0.0f;
  }
  const int64_t t0 = (int64_t)c.k * dm.chunk_len;
  const int nsteps = static_cast<int>(dm.chunk_len);   // chunks before the last are full
  const int64_t row0 = (c.b * L + t0) * D + c.d0;
  scan_steps<N, CPL, T, kPairs, false, V>(x + row0, delta + row0, Bm + (c.b * L + t0) * N,
                                          nullptr, nullptr, nullptr, k, h, S, c.lane, D, nsteps);
  if (c.active) {
    const int64_t row = c.b * (K - 1) + c.k;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
#pragma unroll
      for (int n = 0; n < N; ++n) sum_h[(row * N + n) * D + c.d + q] = h[q][n];
      // the chunk's decay prod_t exp(delta_t A) = exp(S A) is formed by the
      // carry pass from S, summed here in float64
      sum_s[row * D + c.d + q] = S[q];
    }
  }
}

template <int N, int CPL, typename T, bool kPairs, class V>
__global__ __launch_bounds__(kBlock) void chunk_output_kernel(
    const T* __restrict__ x, const T* __restrict__ delta, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ Dskip,
    const T* __restrict__ z, const float* __restrict__ h0, float* __restrict__ h_last,
    float* __restrict__ y, const float* __restrict__ sum_h, ScanDims dm) {
  const int64_t D = dm.D, L = dm.L;
  const int K = dm.K;
  const BlockCoord c = block_coord<CPL>(dm.n_dtiles, K, D);
  const int64_t dl = c.d0 + (int64_t)CPL * c.lane;
  ChainConsts<N, CPL> k;
  load_chain_consts<N, CPL, V>(A, Dskip, dl, k);
  float h[CPL][N];
  double S_unused[CPL];
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    S_unused[q] = 0.0;
#pragma unroll
    for (int n = 0; n < N; ++n) h[q][n] = 0.0f;
  }
  if (c.k > 0) {
    // carry-in: the state entering chunk k, left by the carry pass in slot k - 1
    const float* cp = sum_h + ((c.b * (K - 1) + (c.k - 1)) * N) * D + dl;
#pragma unroll
    for (int q = 0; q < CPL; ++q)
#pragma unroll
      for (int n = 0; n < N; ++n) h[q][n] = cp[(int64_t)n * D + q];
  } else if (h0 != nullptr) {
    const float* hp = h0 + (c.b * D + dl) * N;
#pragma unroll
    for (int q = 0; q < CPL; ++q)
#pragma unroll
      for (int n = 0; n < N; ++n) h[q][n] = hp[q * N + n];
  }
  const int64_t t0 = (int64_t)c.k * dm.chunk_len;
  const int nsteps = static_cast<int>(std::min<int64_t>(dm.chunk_len, L - t0));
  const int64_t row0 = (c.b * L + t0) * D + c.d0;
  scan_steps<N, CPL, T, kPairs, true, V>(x + row0, delta + row0, Bm + (c.b * L + t0) * N,
                                         Cm + (c.b * L + t0) * N, V::kGate ? z + row0 : nullptr,
                                         y + row0, k, h, S_unused, c.lane, D, nsteps);
  if constexpr (V::kState) {
    if (c.k == K - 1) {
      // lanes past the last channel hold that channel's state: same value, same place
      float* hp = h_last + (c.b * D + c.d0) * N;
      const int lo = c.lane * CPL * N;
#pragma unroll
      for (int q = 0; q < CPL; ++q)
#pragma unroll
        for (int n = 0; n < N; ++n) hp[lo + q * N + n] = h[q][n];
    }
  }
}

// ---- launch helpers ------------------------------------------------------------------------

// Calls op.template run<N, CPL, T, kPairs>() for the shape and element type of
// `a` (bfloat16 B/C rows are read as 32-bit pairs when N is even and both are
// 4-byte aligned).
template <int N, int CPL, class Op>
hipError_t dispatch_type(const ScanArgs& a, const Op& op) {
  if (a.dtype == MSSM_FLOAT32) return op.template run<N, CPL, float, false>();
  const bool pairs = (N % 2 == 0) && (reinterpret_cast<uintptr_t>(a.B) % 4 == 0) &&
                     (reinterpret_cast<uintptr_t>(a.C) % 4 == 0);
  if (pairs) return op.template run<N, CPL, uint16_t, true>();
  return op.template run<N, CPL, uint16_t, false>();
}

template <int N, class Op>
hipError_t dispatch_cpl(const ScanArgs& a, int cpl, const Op& op) {
  return cpl == 2 ? dispatch_type<N, 2>(a, op) : dispatch_type<N, 1>(a, op);
}

template <class Op>
hipError_t dispatch_shape(const ScanArgs& a, int cpl, const Op& op) {
  switch (a.N) {
    case 1: return dispatch_cpl<1>(a, cpl, op);
    case 2: return dispatch_cpl<2>(a, cpl, op);
    case 4: return dispatch_cpl<4>(a, cpl, op);
    case 8: return dispatch_cpl<8>(a, cpl, op);
    case 16: return dispatch_cpl<16>(a, cpl, op);
    case 32: return dispatch_cpl<32>(a, cpl, op);
    default: return hipErrorInvalidValue;
  }
}

template <bool kZoh>
struct SummaryLaunch {
  const ScanParams& p;
  int64_t batch;
  hipStream_t stream;
  template <int N, int CPL, typename T, bool kPairs>
  hipError_t run() const {
    const int64_t grid = p.n_dtiles * (p.K - 1) * batch;
    const ScanDims dm{p.L, p.D, p.chunk_len, p.K, p.n_dtiles};
    hipLaunchKernelGGL((chunk_summary_kernel<N, CPL, T, kPairs, kZoh>), dim3((unsigned)grid),
                       dim3(kBlock), 0, stream, static_cast<const T*>(p.x),
                       static_cast<const T*>(p.delta), p.A, static_cast<const T*>(p.B), p.sum_h,
                       p.sum_s, dm);
    return hipGetLastError();
  }
};

template <class V>
struct OutputLaunch {
  const ScanParams& p;
  int64_t batch;
  hipStream_t stream;
  template <int N, int CPL, typename T, bool kPairs>
  hipError_t run() const {
    const int64_t grid = p.n_dtiles * p.K * batch;
    const ScanDims dm{p.L, p.D, p.chunk_len, p.K, p.n_dtiles};
    hipLaunchKernelGGL((chunk_output_kernel<N, CPL, T, kPairs, V>), dim3((unsigned)grid),
                       dim3(kBlock), 0, stream, static_cast<const T*>(p.x),
                       static_cast<const T*>(p.delta), p.A, static_cast<const T*>(p.B),
                       static_cast<const T*>(p.C), p.Dskip, static_cast<const T*>(p.z), p.h0,
                       p.h_last, p.y, p.sum_h, dm);
    return hipGetLastError();
  }
};

// Defined, one variant per source file, by the scan_out_*.hip files.
template <class V>
hipError_t launch_output_variant(const ScanArgs& a, const ScanPlan& plan, const ScanParams& p,
                                 hipStream_t stream);

// Defines the launchers of one (input term, feedthrough, gate) combination,
// with and without the final-state store.
#define MSSM_DEFINE_OUTPUT_VARIANT(ZOH, SKIP, GATE)                                           \
  template <>                                                                                 \
  hipError_t launch_output_variant<Variant<ZOH, SKIP, GATE, false>>(                          \
      const ScanArgs& a, const ScanPlan& plan, const ScanParams& p, hipStream_t stream) {     \
    return dispatch_shape(a, plan.cpl,                                                        \
                          OutputLaunch<Variant<ZOH, SKIP, GATE, false>>{p, a.batch, stream}); \
  }                                                                                           \
  template <>                                                                                 \
  hipError_t launch_output_variant<Variant<ZOH, SKIP, GATE, true>>(                           \
      const ScanArgs& a, const ScanPlan& plan, const ScanParams& p, hipStream_t stream) {     \
    return dispatch_shape(a, plan.cpl,                                                        \
                          OutputLaunch<Variant<ZOH, SKIP, GATE, true>>{p, a.batch, stream});  \
  }

// Defined by scan_summary_{euler,zoh}.hip.
hipError_t launch_summary_euler(const ScanArgs& a, const ScanPlan& plan, const ScanParams& p,
                                hipStream_t stream);
hipError_t launch_summary_zoh(const ScanArgs& a, const ScanPlan& plan, const ScanParams& p,
                              hipStream_t stream);

}  // namespace mssm
