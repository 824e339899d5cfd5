// Device-side building blocks of the selective scan (gfx950).
//
// One lane owns one (batch row, channel) chain and keeps its N state values in
// registers.  The 64 lanes of a wavefront take 64 consecutive channels of the
// same batch row, so at every step they read x and delta as one coalesced
// 256-byte (float32) or 128-byte (bfloat16) row segment, and they all need the
// same B_t and C_t: those come through the scalar unit (s_load into SGPRs) and
// are broadcast to the lanes as instruction operands.  Per element the
// arithmetic is one multiply for the exponent, one v_exp_f32, one multiply for
// the input term and two fused multiply-adds (state update, read-out).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mssm {

constexpr float kLog2e = 1.4426950408889634f;

// ---- element access: float32, or bfloat16 stored as uint16_t ----------------------------

__device__ __forceinline__ float to_float(float v) { return v; }
__device__ __forceinline__ float to_float(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}


// Row of N values shared by the whole wavefront (B_t or C_t).  With a
// wave-uniform address the compiler turns these into scalar loads.
template <int N>
__device__ __forceinline__ void load_row(const float* __restrict__ p, float (&v)[N]) {
#pragma unroll
  for (int n = 0; n < N; ++n) v[n] = p[n];
}

// bfloat16 rows read as 32-bit pairs (requires a 4-byte aligned row: N even
// and an aligned base, checked on the host); the odd-N / unaligned case reads
// one element at a time.
template <int N, bool kPairs>
__device__ __forceinline__ void load_row_bf16(const uint16_t* __restrict__ p, float (&v)[N]) {
  if constexpr (kPairs && (N % 2 == 0)) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const uint32_t u = q[i];
      v[2 * i] = __uint_as_float(u << 16);
      v[2 * i + 1] = __uint_as_float(u & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] = to_float(p[n]);
  }
}

template <int N, bool kPairs>
__device__ __forceinline__ void load_row_any(const float* __restrict__ p, float (&v)[N]) {
  load_row<N>(p, v);
}
template <int N, bool kPairs>
__device__ __forceinline__ void load_row_any(const uint16_t* __restrict__ p, float (&v)[N]) {
  load_row_bf16<N, kPairs>(p, v);
}

// exp2 on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// ---- the per-lane sequential pass over a range of steps -----------------------------------
//
// Runs steps [0, nsteps) of one chunk for the lane's chain.  `ld` indexes
// x/delta/y at the first step (b, t0, d); `bn` indexes B/C at (b, t0, 0).
// kWithY: also form y_t = sum_n C_t[n] h_t[n] and store it (output pass);
// otherwise accumulate the chunk's total step size in `S` (summary pass).
// x and delta are prefetched kTile steps ahead; B_t and C_t one step ahead.
template <int N, typename T, bool kPairs, bool kWithY>
__device__ __forceinline__ void scan_steps(const T* __restrict__ x, const T* __restrict__ delta,
                                           const T* __restrict__ Bm, const T* __restrict__ Cm,
                                           float* __restrict__ y, const float (&A2)[N], float (&h)[N],
                                           double& S, int64_t ld, int64_t bn, int64_t D,
                                           int nsteps, bool active) {
  constexpr int kTile = 8;
  T xc[kTile], dc[kTile];
#pragma unroll
  for (int j = 0; j < kTile; ++j) {
    if (j < nsteps) {
      xc[j] = x[ld + (int64_t)j * D];
      dc[j] = delta[ld + (int64_t)j * D];
    }
  }
  float Bv[N], Cv[N];
  if (nsteps > 0) {
    load_row_any<N, kPairs>(Bm + bn, Bv);
    if constexpr (kWithY) load_row_any<N, kPairs>(Cm + bn, Cv);
  }
  for (int base = 0; base < nsteps; base += kTile) {
    T xn[kTile], dn[kTile];
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      const int s = base + kTile + j;
      if (s < nsteps) {
        xn[j] = x[ld + (int64_t)s * D];
        dn[j] = delta[ld + (int64_t)s * D];
      }
    }
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      const int s = base + j;
      if (s < nsteps) {
        float Bnext[N], Cnext[N];
        if (s + 1 < nsteps) {
          load_row_any<N, kPairs>(Bm + bn + (int64_t)(s + 1) * N, Bnext);
          if constexpr (kWithY) load_row_any<N, kPairs>(Cm + bn + (int64_t)(s + 1) * N, Cnext);
        }
        const float dt = to_float(dc[j]);
        const float dx = dt * to_float(xc[j]);
        float yv = 0.0f;
#pragma unroll
        for (int n = 0; n < N; ++n) {
          const float a = fast_exp2(dt * A2[n]);           // Abar = exp(delta * A)
          h[n] = __builtin_fmaf(a, h[n], dx * Bv[n]);      // h = Abar h + (delta B) x
          if constexpr (kWithY) yv = __builtin_fmaf(Cv[n], h[n], yv);   // y = C . h
        }
        if constexpr (kWithY) {
          if (active) y[ld + (int64_t)s * D] = yv;
        } else {
          S += static_cast<double>(dt);
        }
        if (s + 1 < nsteps) {
#pragma unroll
          for (int n = 0; n < N; ++n) {
            Bv[n] = Bnext[n];
            if constexpr (kWithY) Cv[n] = Cnext[n];
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      xc[j] = xn[j];
      dc[j] = dn[j];
    }
  }
}

}  // namespace mssm
