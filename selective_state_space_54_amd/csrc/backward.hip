// Backward pass of the selective scan with recomputation (first-order input
// term, optional feedthrough D x, SiLU(z) gate and initial state).
//
// Chain rule through h_t = a_t h_{t-1} + delta_t B_t x_t, y_t = C_t . h_t + D x_t,
// out_t = y_t SiLU(z_t), a_t = exp(delta_t A), for an upstream gradient dout:
//   g_t   = dout_t SiLU(z_t)                    dz_t = dout_t y_t SiLU'(z_t)
//   lam_t = C_t g_t + a_{t+1} lam_{t+1}          (the adjoint, a reverse scan
//                                                 with the same pair operator,
//                                                 "Understanding Mamba" eq. (8))
//   dC_t += g_t h_t,  dB_t += lam_t delta_t x_t  (summed over channels)
//   dx_t  = g_t D + sum_n lam_t delta_t B_t
//   ddelta_t = sum_n lam_t (B_t x_t + A a_t h_{t-1}),   dA += lam_t delta_t a_t h_{t-1}
//   dD += g_t x_t,  dh0 = a_0 lam_0
// with a_t h_{t-1} = h_t - delta_t B_t x_t, so only h_t is needed.
//
// The states are recomputed, never stored ("State Space Models and Mamba",
// hardware-aware scan: the backward recomputes the states).  The sequence is
// cut into chunks of kChunk steps:
//   1. forward summaries + carries (the forward pass's kernels): the state
//      entering every chunk;
//   2. reverse summaries + carries: the adjoint entering every chunk from the
//      right (the reverse sweep from zero over a chunk, and its decay, fed to
//      the same carry kernel in reversed chunk order);
//   3. per chunk and per group of four state indices: recompute the chunk's
//      states into registers, sweep backwards, accumulate every gradient;
//      dB/dC are summed over the wavefront's 64 channels with a
//      reduce-scatter across lanes and written as per-wavefront partials;
//      dA/dD as per-chunk partials;
//   4. small kernels add the partials up (a fixed order: deterministic).
#include <algorithm>

#include "mssm_internal.h"
#include "scan_kernels.h"

namespace mssm {

namespace {

constexpr int kBwdBlock = 256;
constexpr int kChunk = 16;          // steps per backward chunk (register arrays)

__device__ __forceinline__ float silu_slope(float v) {
  const float s = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-v * kLog2e));
  return s * (1.0f + v * (1.0f - s));
}

// DPP lane moves within 16-lane rows (row_ror:8 swaps the row's two halves,
// row_half_mirror reverses each group of 8, the quad permutations swap lanes
// 2 apart and 1 apart).
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppRowRor8 = 0x128, kDppRowHalfMirror = 0x141, kDppQuadXor2 = 0x4E,
              kDppQuadXor1 = 0xB1;

// a + b per lane after exchanging halves: permlane32_swap leaves lanes 0..31
// holding (a, a from lanes 32..63) and lanes 32..63 holding (b from lanes
// 0..31, b); the sum is a summed over lane pairs 32 apart in lanes 0..31 and b
// in lanes 32..63.  permlane16_swap does the same for rows 16 apart.
__device__ __forceinline__ float fold32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float fold16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum of v[i] over the wavefront's 64 lanes for i = 0..7, scattered: lane L
// returns the total of v[L >> 3].  Three halving rounds (lanes 32, 16 and 8
// apart) keep the half selected by the lane's bit, then three plain DPP rounds
// within each group of 8 lanes finish the sums.  Every lane must take part.
__device__ __forceinline__ float wave_reduce_scatter8(const float (&v)[8], int lane) {
  float w4[4], w2[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) w4[i] = fold32(v[i], v[i + 4]);     // index 4*bit5 + i
#pragma unroll
  for (int i = 0; i < 2; ++i) w2[i] = fold16(w4[i], w4[i + 2]);   // + 2*bit4
  const bool up = (lane & 8) != 0;                                 // + bit3
  float w = (up ? w2[1] : w2[0]) + dpp<kDppRowRor8>(up ? w2[0] : w2[1]);
  w += dpp<kDppRowHalfMirror>(w);
  w += dpp<kDppQuadXor2>(w);
  w += dpp<kDppQuadXor1>(w);
  return w;
}

// Reverse summary of chunk k (1..K-1): the adjoint sweep from zero at the
// chunk's end, nu = a_{s_k} lam_{s_k}, and the chunk's step-size total (its
// decay is exp(A sum delta)), stored in reversed chunk order (slot K-1-k) so
// that the forward carry kernel produces the adjoint entering each chunk from
// the right.
template <int N, typename T, bool kGate>
__global__ __launch_bounds__(kBwdBlock) void bwd_rev_summary_kernel(
    const T* __restrict__ delta, const float* __restrict__ A, const T* __restrict__ Cm,
    const T* __restrict__ z, const float* __restrict__ dout, float* __restrict__ rev_h,
    double* __restrict__ rev_s, int64_t L, int64_t D, int64_t chunk, int K, int64_t n_dtiles) {
  const int64_t bid = blockIdx.x;
  const int64_t dtile = bid % n_dtiles;
  const int64_t rest = bid / n_dtiles;
  const int k = static_cast<int>(rest % (K - 1)) + 1;
  const int64_t b = rest / (K - 1);
  const int64_t d = dtile * kBwdBlock + threadIdx.x;
  if (d >= D) return;                       // no barriers or cross-lane operations here
  float A2[N], lamc[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    A2[n] = A[d * N + n] * kLog2e;
    lamc[n] = 0.0f;
  }
  double S = 0.0;
  const int64_t t0 = (int64_t)k * chunk;
  const int64_t nsteps = std::min<int64_t>(chunk, L - t0);
  for (int64_t s = nsteps - 1; s >= 0; --s) {
    const int64_t t = t0 + s;
    const int64_t i = (b * L + t) * D + d;
    const float dv = to_float(delta[i]);
    float g = dout[i];
    if constexpr (kGate) g *= silu(to_float(z[i]));
    S += static_cast<double>(dv);
    const T* Cr = Cm + (b * L + t) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const float lam = __builtin_fmaf(to_float(Cr[n]), g, lamc[n]);
      lamc[n] = fast_exp2(dv * A2[n]) * lam;
    }
  }
  const int64_t slot = b * (K - 1) + (K - 1 - k);
#pragma unroll
  for (int n = 0; n < N; ++n) rev_h[(slot * N + n) * D + d] = lamc[n];
  rev_s[slot * D + d] = S;
}

struct BwdParams {
  const float* Dskip;
  const float* h0;
  const float* dout;
  const float* sum_h;     // forward carries, slot k-1 = state entering chunk k
  const float* rev_h;     // reverse carries, slot K-2-k = adjoint entering chunk k
  float* dx;
  float* ddelta;
  float* dz;
  float* dh0;
  float* partBC;          // [n_wt, batch, L, 2N]
  float* partA;           // [batch * K, D, N]
  float* partD;           // [batch * K, D]
  int64_t batch, L, D, chunk, n_dtiles, n_wt;
  int K;
};

template <typename T>
__device__ __forceinline__ float buf_load1(buf_t r, int voff, int soff) {
  float v[1];
  buf_load_vals<T, 1>(r, voff, soff, v);
  return v[0];
}

__device__ __forceinline__ void buf_store1(buf_t r, int voff, int soff, float v) {
  const float w[1] = {v};
  buf_store_vals<1>(r, voff, soff, w);
}

template <int N, typename T, bool kSkip, bool kGate>
__global__ __launch_bounds__(kBwdBlock) void bwd_chunk_kernel(
    const T* __restrict__ x, const T* __restrict__ delta, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const T* __restrict__ z, BwdParams p) {
  constexpr int G = N < 4 ? N : 4;          // state indices per pass over the chunk
  const int64_t bid = blockIdx.x;
  const int64_t dtile = bid % p.n_dtiles;
  const int64_t rest = bid / p.n_dtiles;
  const int k = static_cast<int>(rest % p.K);
  const int64_t b = rest / p.K;
  const int lane = static_cast<int>(threadIdx.x % 64);
  const int64_t wt = dtile * (kBwdBlock / 64) + threadIdx.x / 64;
  if (wt >= p.n_wt) return;                 // a whole wavefront past the last channel
  const int64_t D = p.D, L = p.L;
  const int64_t d_raw = dtile * kBwdBlock + threadIdx.x;
  const bool active = d_raw < D;
  const int64_t d = active ? d_raw : D - 1; // inactive lanes repeat the last channel
  const int64_t t0 = (int64_t)k * p.chunk;
  const int nsteps = static_cast<int>(std::min<int64_t>(p.chunk, L - t0));
  // per-lane [batch, L, D] arrays of this chunk through buffer descriptors: a
  // uniform row offset per step and a constant per-lane offset
  const int64_t row0 = (b * L + t0) * D;
  const uint32_t in_bytes = static_cast<uint32_t>((int64_t)nsteps * D * sizeof(T));
  const uint32_t f_bytes = static_cast<uint32_t>((int64_t)nsteps * D * sizeof(float));
  const buf_t xr = make_buf(x + row0, in_bytes);
  const buf_t dr = make_buf(delta + row0, in_bytes);
  const buf_t gr = make_buf(p.dout + row0, f_bytes);
  buf_t zr;
  if constexpr (kGate) zr = make_buf(z + row0, in_bytes);
  const int in_lane = static_cast<int>(d * sizeof(T));
  const int f_lane = static_cast<int>(d * sizeof(float));
  const int in_row = static_cast<int>(D * sizeof(T));
  const int f_row = static_cast<int>(D * sizeof(float));
  const T* Bc = Bm + (b * L + t0) * N;
  const T* Cc = Cm + (b * L + t0) * N;
  const float Dd = kSkip ? p.Dskip[d] : 0.0f;
  float dxa[kChunk], dda[kChunk], ya[kGate ? kChunk : 1];
#pragma unroll
  for (int s = 0; s < kChunk; ++s) {
    dxa[s] = 0.0f;
    dda[s] = 0.0f;
    if constexpr (kGate) ya[s] = 0.0f;
  }
  for (int n0 = 0; n0 < N; n0 += G) {
    float A2[G], Ar[G], h[G], lamc[G], dAacc[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      Ar[j] = A[d * N + n0 + j];
      A2[j] = Ar[j] * kLog2e;
      dAacc[j] = 0.0f;
      if (k == 0)
        h[j] = p.h0 != nullptr ? p.h0[(b * D + d) * N + n0 + j] : 0.0f;
      else
        h[j] = p.sum_h[((b * (p.K - 1) + (k - 1)) * N + n0 + j) * D + d];
      lamc[j] = (k == p.K - 1) ? 0.0f
                               : p.rev_h[((b * (p.K - 1) + (p.K - 2 - k)) * N + n0 + j) * D + d];
    }
    // recompute the chunk's states for these state indices
    float hist[kChunk][G];
#pragma unroll
    for (int s = 0; s < kChunk; ++s) {
      if (s < nsteps) {
        const int soff = s * in_row;
        const float xv = buf_load1<T>(xr, in_lane, soff);
        const float dv = buf_load1<T>(dr, in_lane, soff);
        const float dxv = dv * xv;
        float yv = 0.0f;
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const float a = fast_exp2(dv * A2[j]);
          h[j] = __builtin_fmaf(a, h[j], dxv * to_float(Bc[s * N + n0 + j]));
          hist[s][j] = h[j];
          if constexpr (kGate) yv = __builtin_fmaf(to_float(Cc[s * N + n0 + j]), h[j], yv);
        }
        if constexpr (kGate) ya[s] += yv;
      }
    }
    // backwards through the chunk
#pragma unroll
    for (int s = kChunk - 1; s >= 0; --s) {
      if (s < nsteps) {
        const int soff = s * in_row;
        const float xv = buf_load1<T>(xr, in_lane, soff);
        const float dv = buf_load1<T>(dr, in_lane, soff);
        float gv = buf_load1<float>(gr, f_lane, s * f_row);
        if constexpr (kGate) gv *= silu(buf_load1<T>(zr, in_lane, soff));
        const float dxv = dv * xv;
        // lanes past the last channel add nothing to dB, dC
        const float xact = active ? xv : 0.0f, gact = active ? gv : 0.0f;
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.0f;
        float q = 0.0f, r = 0.0f;    // sum_n lam B, sum_n lam A a h_{t-1}
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const float Bj = to_float(Bc[s * N + n0 + j]);
          const float lam = __builtin_fmaf(to_float(Cc[s * N + n0 + j]), gv, lamc[j]);
          const float hb = hist[s][j];
          const float hpa = __builtin_fmaf(-dxv, Bj, hb);     // a_t h_{t-1}
          q = __builtin_fmaf(lam, Bj, q);
          r = __builtin_fmaf(lam * Ar[j], hpa, r);
          const float ldv = lam * dv;
          dAacc[j] = __builtin_fmaf(ldv, hpa, dAacc[j]);
          v[j] = ldv * xact;                                    // dB_t[n]
          v[4 + j] = gact * hb;                                 // dC_t[n]
          lamc[j] = fast_exp2(dv * A2[j]) * lam;
        }
        dxa[s] = __builtin_fmaf(dv, q, dxa[s]);
        dda[s] += __builtin_fmaf(xv, q, r);
        const float red = wave_reduce_scatter8(v, lane);
        if ((lane & 7) == 0) {
          const int idx = lane >> 3;
          const int j = idx & 3;
          if (j < G) {
            const int col = idx < 4 ? n0 + j : N + n0 + j;
            p.partBC[((wt * p.batch + b) * L + t0 + s) * (2 * N) + col] = red;
          }
        }
      }
    }
    if (active) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        p.partA[(((b * p.K) + k) * D + d) * N + n0 + j] = dAacc[j];
        if (k == 0 && p.dh0 != nullptr) p.dh0[(b * D + d) * N + n0 + j] = lamc[j];
      }
    }
  }
  const buf_t dxr = make_buf(p.dx + row0, f_bytes);
  const buf_t ddr = make_buf(p.ddelta + row0, f_bytes);
  buf_t dzr;
  if constexpr (kGate) dzr = make_buf(p.dz + row0, f_bytes);
  float dD = 0.0f;
#pragma unroll
  for (int s = 0; s < kChunk; ++s) {
    if (s < nsteps) {
      const int soff = s * in_row;
      const float xv = buf_load1<T>(xr, in_lane, soff);
      const float go = buf_load1<float>(gr, f_lane, s * f_row);
      float gv = go;
      float zv = 0.0f;
      if constexpr (kGate) {
        zv = buf_load1<T>(zr, in_lane, soff);
        gv *= silu(zv);
      }
      float dxv = dxa[s];
      if constexpr (kSkip) {
        dxv = __builtin_fmaf(gv, Dd, dxv);
        dD = __builtin_fmaf(gv, xv, dD);
      }
      // inactive lanes repeat the last channel's values: same value, same place
      if constexpr (kGate) {
        const float y = kSkip ? __builtin_fmaf(Dd, xv, ya[s]) : ya[s];
        buf_store1(dzr, f_lane, s * f_row, go * y * silu_slope(zv));
      }
      buf_store1(dxr, f_lane, s * f_row, dxv);
      buf_store1(ddr, f_lane, s * f_row, dda[s]);
    }
  }
  if (kSkip && active) p.partD[(b * p.K + k) * D + d] = dD;
}

// dB[r, n] and dC[r, n] (r = b * L + t): the sum of the n_wt partials
// part[w * total + e], added in w order.  When total is a multiple of 4 a
// thread takes 4 adjacent outputs (16-byte loads) and issues 8 partials'
// loads before adding them, so enough reads are in flight to stream the
// partials at HBM rate.
constexpr int kBcUnroll = 8;
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(const float* __restrict__ part,
                                                            float* __restrict__ dB,
                                                            float* __restrict__ dC, int64_t rows,
                                                            int N, int64_t n_wt) {
  const int64_t total = rows * 2 * N;
  const bool vec = total % 4 == 0;
  const int64_t groups = vec ? total / 4 : total;
  auto emit = [&](int64_t e, float v) {
    const int64_t r = e / (2 * N);
    const int c = static_cast<int>(e % (2 * N));
    if (c < N)
      dB[r * N + c] = v;
    else
      dC[r * N + c - N] = v;
  };
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups;
       g += (int64_t)gridDim.x * blockDim.x) {
    if (vec) {
      const float4* p = reinterpret_cast<const float4*>(part) + g;
      const int64_t stride = total / 4;
      float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      int64_t w = 0;
      for (; w + kBcUnroll <= n_wt; w += kBcUnroll) {
        float4 v[kBcUnroll];
#pragma unroll
        for (int u = 0; u < kBcUnroll; ++u) v[u] = p[(w + u) * stride];
#pragma unroll
        for (int u = 0; u < kBcUnroll; ++u) {
          s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
        }
      }
      for (; w < n_wt; ++w) {
        const float4 v = p[w * stride];
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
      }
      emit(4 * g, s.x);
      emit(4 * g + 1, s.y);
      emit(4 * g + 2, s.z);
      emit(4 * g + 3, s.w);
    } else {
      float s = 0.0f;
      for (int64_t w = 0; w < n_wt; ++w) s += part[w * total + g];
      emit(g, s);
    }
  }
}

// Grid of the kernel above for `rows` rows of 2N outputs.
inline unsigned reduce_bc_grid(int64_t rows, int64_t N) {
  const int64_t total = rows * 2 * N;
  const int64_t groups = total % 4 == 0 ? total / 4 : total;
  return static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>((groups + 255) / 256, 8192)));
}

// out[e] = sum_r part[r * count + e], r < nparts.  A block takes 16 outputs;
// its 16 row groups each sum every 16th row (rows issued 4 at a time), then
// the groups' sums are added in LDS in a fixed order: deterministic.
constexpr int kRedCols = 16, kRedGroups = 16;
__global__ __launch_bounds__(kRedCols * kRedGroups) void bwd_reduce_rows_kernel(
    const float* __restrict__ part, float* __restrict__ out, int64_t count, int64_t nparts) {
  __shared__ float acc[kRedGroups][kRedCols];
  const int col = threadIdx.x % kRedCols;
  const int grp = threadIdx.x / kRedCols;
  const int64_t e = (int64_t)blockIdx.x * kRedCols + col;
  float s = 0.0f;
  if (e < count) {
    int64_t r = grp;
    for (; r + 3 * kRedGroups < nparts; r += 4 * kRedGroups) {
      const float v0 = part[r * count + e];
      const float v1 = part[(r + kRedGroups) * count + e];
      const float v2 = part[(r + 2 * kRedGroups) * count + e];
      const float v3 = part[(r + 3 * kRedGroups) * count + e];
      s += v0;
      s += v1;
      s += v2;
      s += v3;
    }
    for (; r < nparts; r += kRedGroups) s += part[r * count + e];
  }
  acc[grp][col] = s;
  block_sync();
  if (grp == 0 && e < count) {
    float t = 0.0f;
#pragma unroll
    for (int g = 0; g < kRedGroups; ++g) t += acc[g][col];
    out[e] = t;
  }
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

template <int N, typename T, bool kSkip, bool kGate>
hipError_t launch_bwd_t(const BwdArgs& a, const BwdPlan& bp, char* ws, hipStream_t stream) {
  const int K = bp.K;
  const int64_t n_dtiles = (a.D + kBwdBlock - 1) / kBwdBlock;
  const T* x = static_cast<const T*>(a.x);
  const T* delta = static_cast<const T*>(a.delta);
  const T* Bm = static_cast<const T*>(a.B);
  const T* Cm = static_cast<const T*>(a.C);
  const T* z = static_cast<const T*>(a.z);
  float* sum_h = reinterpret_cast<float*>(ws + bp.fwd_h_offset);
  double* sum_s = reinterpret_cast<double*>(ws + bp.fwd_s_offset);
  float* rev_h = reinterpret_cast<float*>(ws + bp.rev_h_offset);
  double* rev_s = reinterpret_cast<double*>(ws + bp.rev_s_offset);
  hipError_t e;
  if (K > 1) {
    // 1. forward: the state entering every chunk (the forward pass's own kernels)
    ScanArgs sa{a.x, a.delta, a.A, a.B, a.C, nullptr, a.batch, a.L, a.D, a.N, a.dtype};
    ScanPlan plan;
    plan.cpl = 1;
    plan.K = K;
    plan.chunk_len = bp.chunk;
    ScanParams sp{};
    sp.x = a.x;
    sp.delta = a.delta;
    sp.A = a.A;
    sp.B = a.B;
    sp.C = a.C;
    sp.sum_h = sum_h;
    sp.sum_s = sum_s;
    sp.L = a.L;
    sp.D = a.D;
    sp.chunk_len = bp.chunk;
    sp.K = K;
    sp.n_dtiles = (a.D + kBlock - 1) / kBlock;
    e = launch_summary_euler(sa, plan, sp, stream);
    if (e != hipSuccess) return e;
    e = launch_carry(sum_h, sum_s, a.A, a.h0, a.batch, a.D, a.N, K, stream);
    if (e != hipSuccess) return e;
    // 2. reverse: the adjoint entering every chunk from the right
    const int64_t rgrid = n_dtiles * (K - 1) * a.batch;
    hipLaunchKernelGGL((bwd_rev_summary_kernel<N, T, kGate>), dim3((unsigned)rgrid),
                       dim3(kBwdBlock), 0, stream, delta, a.A, Cm, z, a.dout, rev_h, rev_s, a.L,
                       a.D, bp.chunk, K, n_dtiles);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_carry(rev_h, rev_s, a.A, nullptr, a.batch, a.D, a.N, K, stream);
    if (e != hipSuccess) return e;
  }
  // 3. recompute + backwards sweep per chunk
  BwdParams p{};
  p.Dskip = a.Dskip;
  p.h0 = a.h0;
  p.dout = a.dout;
  p.sum_h = sum_h;
  p.rev_h = rev_h;
  p.dx = a.dx;
  p.ddelta = a.ddelta;
  p.dz = a.dz;
  p.dh0 = a.dh0;
  p.partBC = reinterpret_cast<float*>(ws + bp.part_bc_offset);
  p.partA = reinterpret_cast<float*>(ws + bp.part_a_offset);
  p.partD = reinterpret_cast<float*>(ws + bp.part_d_offset);
  p.batch = a.batch;
  p.L = a.L;
  p.D = a.D;
  p.chunk = bp.chunk;
  p.n_dtiles = n_dtiles;
  p.n_wt = (a.D + 63) / 64;
  p.K = K;
  const int64_t grid = n_dtiles * K * a.batch;
  hipLaunchKernelGGL((bwd_chunk_kernel<N, T, kSkip, kGate>), dim3((unsigned)grid),
                     dim3(kBwdBlock), 0, stream, x, delta, a.A, Bm, Cm, z, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 4. sums of the partials
  hipLaunchKernelGGL(bwd_reduce_bc_kernel, dim3(reduce_bc_grid(a.batch * a.L, a.N)), dim3(256), 0,
                     stream, p.partBC, a.dB, a.dC, a.batch * a.L, static_cast<int>(a.N), p.n_wt);
  const int64_t da_count = a.D * a.N;
  hipLaunchKernelGGL(bwd_reduce_rows_kernel, dim3((unsigned)((da_count + kRedCols - 1) / kRedCols)),
                     dim3(kRedCols * kRedGroups), 0, stream, p.partA, a.dA, da_count,
                     a.batch * K);
  if (kSkip)
    hipLaunchKernelGGL(bwd_reduce_rows_kernel, dim3((unsigned)((a.D + kRedCols - 1) / kRedCols)),
                       dim3(kRedCols * kRedGroups), 0, stream, p.partD, a.dD, a.D, a.batch * K);
  return hipGetLastError();
}

template <int N, typename T>
hipError_t launch_bwd_nt(const BwdArgs& a, const BwdPlan& bp, char* ws, hipStream_t stream) {
  const bool skip = a.Dskip != nullptr, gate = a.z != nullptr;
  if (skip && gate) return launch_bwd_t<N, T, true, true>(a, bp, ws, stream);
  if (skip) return launch_bwd_t<N, T, true, false>(a, bp, ws, stream);
  if (gate) return launch_bwd_t<N, T, false, true>(a, bp, ws, stream);
  return launch_bwd_t<N, T, false, false>(a, bp, ws, stream);
}

template <int N>
hipError_t launch_bwd_n(const BwdArgs& a, const BwdPlan& bp, char* ws, hipStream_t stream) {
  if (a.dtype == MSSM_FLOAT32) return launch_bwd_nt<N, float>(a, bp, ws, stream);
  return launch_bwd_nt<N, uint16_t>(a, bp, ws, stream);
}

}  // namespace

BwdPlan plan_bwd(int64_t batch, int64_t L, int64_t D, int64_t N, bool chain) {
  BwdPlan b;
  if (chain) {
    // checkpoints [batch, tiles, D, N]; dB/dC partials per 16-channel block
    // [D/16, batch*L, 2N]; dA partials [batch, D, N]; dD partials [batch, D]
    const size_t tiles = (size_t)((L + 15) / 16);
    b.chain = true;
    size_t off = 0;
    b.ck_offset = off;      off += align256(sizeof(float) * (size_t)batch * tiles * (size_t)D * (size_t)N);
    b.part_bc_offset = off; off += align256(sizeof(float) * (size_t)(D / 16) * (size_t)batch * (size_t)L * 2 * (size_t)N);
    b.part_a_offset = off;  off += align256(sizeof(float) * (size_t)batch * (size_t)D * (size_t)N);
    b.part_d_offset = off;  off += align256(sizeof(float) * (size_t)batch * (size_t)D);
    b.workspace_bytes = off;
    return b;
  }
  b.chunk = kChunk;
  b.K = static_cast<int>((L + kChunk - 1) / kChunk);
  const size_t sums = b.K > 1 ? align256(sizeof(float) * (size_t)batch * (size_t)(b.K - 1) *
                                         (size_t)N * (size_t)D)
                              : 0;
  const size_t totals =
      b.K > 1 ? align256(sizeof(double) * (size_t)batch * (size_t)(b.K - 1) * (size_t)D) : 0;
  const size_t n_wt = (size_t)((D + 63) / 64);
  size_t off = 0;
  b.fwd_h_offset = off;   off += sums;
  b.fwd_s_offset = off;   off += totals;
  b.rev_h_offset = off;   off += sums;
  b.rev_s_offset = off;   off += totals;
  b.part_bc_offset = off; off += align256(sizeof(float) * n_wt * (size_t)batch * (size_t)L * 2 * (size_t)N);
  b.part_a_offset = off;  off += align256(sizeof(float) * (size_t)batch * (size_t)b.K * (size_t)D * (size_t)N);
  b.part_d_offset = off;  off += align256(sizeof(float) * (size_t)batch * (size_t)b.K * (size_t)D);
  b.workspace_bytes = off;
  return b;
}

SavedLayout saved_layout(int64_t batch, int64_t L, int64_t D, int64_t N, bool gate) {
  SavedLayout s;
  if (N != 16 || D % 16 != 0 || batch <= 0 || L <= 0 || D <= 0) return s;
  const size_t tiles = (size_t)((L + 15) / 16);
  s.ck_offset = 0;
  s.bytes = align256(sizeof(float) * (size_t)batch * tiles * (size_t)D * (size_t)N);
  if (gate) {
    s.y_pre_offset = s.bytes;
    s.bytes += align256(sizeof(float) * (size_t)batch * (size_t)L * (size_t)D);
  }
  return s;
}

size_t bwd_workspace_bound(int64_t batch, int64_t L, int64_t D, int64_t N) {
  size_t w = plan_bwd(batch, L, D, N, false).workspace_bytes;
  if (N == 16 && D % 16 == 0) w = std::max(w, plan_bwd(batch, L, D, N, true).workspace_bytes);
  return w;
}

hipError_t launch_bwd(const BwdArgs& a, const BwdPlan& bp, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  if (bp.chain) {
    float* part_bc = reinterpret_cast<float*>(ws + bp.part_bc_offset);
    float* part_a = reinterpret_cast<float*>(ws + bp.part_a_offset);
    float* part_d = reinterpret_cast<float*>(ws + bp.part_d_offset);
    const bool saved = a.saved_ck != nullptr;
    float* ck = saved ? const_cast<float*>(a.saved_ck) : reinterpret_cast<float*>(ws + bp.ck_offset);
    hipError_t e = launch_chain_bwd(a, ck, a.saved_y_pre, saved, part_bc, part_a, part_d, stream);
    if (e != hipSuccess) return e;
    // per-block dB/dC partials, per-batch-row dA / dD partials, in a fixed order
    hipLaunchKernelGGL(bwd_reduce_bc_kernel, dim3(reduce_bc_grid(a.batch * a.L, a.N)), dim3(256), 0,
                       stream, part_bc, a.dB, a.dC, a.batch * a.L, static_cast<int>(a.N), a.D / 16);
    const int64_t da_count = a.D * a.N;
    hipLaunchKernelGGL(bwd_reduce_rows_kernel,
                       dim3((unsigned)((da_count + kRedCols - 1) / kRedCols)),
                       dim3(kRedCols * kRedGroups), 0, stream, part_a, a.dA, da_count, a.batch);
    if (a.Dskip)
      hipLaunchKernelGGL(bwd_reduce_rows_kernel, dim3((unsigned)((a.D + kRedCols - 1) / kRedCols)),
                         dim3(kRedCols * kRedGroups), 0, stream, part_d, a.dD, a.D, a.batch);
    return hipGetLastError();
  }
  switch (a.N) {
    case 1: return launch_bwd_n<1>(a, bp, ws, stream);
    case 2: return launch_bwd_n<2>(a, bp, ws, stream);
    case 4: return launch_bwd_n<4>(a, bp, ws, stream);
    case 8: return launch_bwd_n<8>(a, bp, ws, stream);
    case 16: return launch_bwd_n<16>(a, bp, ws, stream);
    case 32: return launch_bwd_n<32>(a, bp, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mssm
