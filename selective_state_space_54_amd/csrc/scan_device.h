// Device-side building blocks of the selective scan (gfx950).
//
// A lane owns CPL adjacent channels of one batch row (CPL = 1 or 2) and keeps
// their N state values each in registers.  The 64 lanes of a wavefront take
// 64 * CPL consecutive channels, so at every step they read x and delta as one
// coalesced row segment, and they all need the same B_t and C_t: those come
// through the scalar unit (s_load into SGPRs) and are broadcast to the lanes as
// instruction operands.  Per element the arithmetic is one multiply for the
// exponent, one v_exp_f32, one multiply for the input term and two fused
// multiply-adds (state update, read-out).  Two chains per lane give the
// scheduler two independent dependency chains and halve the scalar loads per
// element.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mssm {

constexpr float kLog2e = 1.4426950408889634f;

// Block-wide barrier that first waits until this wavefront's LDS operations
// have completed.  The compiler's own lowering of __syncthreads can leave out
// that wait on gfx950 (which can back off a barrier): in a loop whose body
// ends with an LDS store and starts with a barrier, the store issued before
// the back edge was still in flight when other wavefronts passed the barrier
// and read the tile, which then held stale values now and then.
__device__ __forceinline__ void block_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __syncthreads();
}

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

// A prefetched row as it was loaded: float32 values, or bfloat16 pairs kept
// packed, two to a 32-bit register, and widened only where a value is used.
// Widening at the load would need the loaded data at once, so the load could
// no longer run a step ahead of its use.
template <int N, typename T, bool kPairs>
struct RawRow {
  static constexpr bool kPinnable = false;
  float w[N];
  __device__ __forceinline__ void load(const float* __restrict__ p) { load_row<N>(p, w); }
  __device__ __forceinline__ float get(int n) const { return w[n]; }
};
template <int N, bool kPairs>
struct RawRow<N, uint16_t, kPairs> {
  static constexpr bool kPacked = kPairs && (N % 2 == 0);
  static constexpr bool kPinnable = kPacked && N <= 16;
  uint32_t w[kPacked ? N / 2 : N];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ p) {
    if constexpr (kPacked) {
      const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
      for (int i = 0; i < N / 2; ++i) w[i] = q[i];
    } else {
#pragma unroll
      for (int n = 0; n < N; ++n) w[n] = static_cast<uint32_t>(p[n]) << 16;
    }
  }
  __device__ __forceinline__ float get(int n) const {
    if constexpr (kPacked) return __uint_as_float((n & 1) ? (w[n / 2] & 0xffff0000u) : (w[n / 2] << 16));
    else return __uint_as_float(w[n]);
  }
};

// exp2 on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// Wait until every scalar-memory (and LDS) access issued so far has returned:
// s_waitcnt lgkmcnt(0), with the vector-memory and export counters left at
// their maximum (gfx9 encoding).  Scalar loads can return out of order, so
// the only usable wait is "all of them": the step loop waits here for the
// current step's B_t/C_t *before* issuing the next step's loads, so the next
// loads overlap the current step's arithmetic instead of being waited for.
__device__ __forceinline__ void wait_scalar_loads() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// ---- buffer (descriptor-based) access ------------------------------------------------------
//
// A buffer resource holds a wave-uniform base address and a byte limit; each
// access adds a per-lane byte offset (VGPR) and a wave-uniform byte offset
// (SGPR), so stepping through time costs no vector address arithmetic.  The
// hardware range check covers only the per-lane part, so callers keep the
// uniform offset inside the buffer themselves.  Word 3 is the gfx9-family
// default descriptor format.
using buf_t = __amdgpu_buffer_rsrc_t;
constexpr int kBufferWord3 = 0x00020000;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ buf_t make_buf(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferWord3);
}

// CPL adjacent values of element type T at (voff + soff) bytes, widened to float.
template <typename T, int CPL>
__device__ __forceinline__ void buf_load_vals(buf_t r, int voff, int soff, float (&v)[CPL]) {
  if constexpr (sizeof(T) == 4 && CPL == 1) {
    v[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
  } else if constexpr (sizeof(T) == 4 && CPL == 2) {
    const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    v[0] = __uint_as_float(u.x);
    v[1] = __uint_as_float(u.y);
  } else if constexpr (sizeof(T) == 2 && CPL == 1) {
    v[0] = __uint_as_float(
        static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0)) << 16);
  } else {
    static_assert(sizeof(T) == 2 && CPL == 2, "unsupported element/lane combination");
    const uint32_t u = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    v[0] = __uint_as_float(u << 16);          // lower address = first channel
    v[1] = __uint_as_float(u & 0xffff0000u);
  }
}

// float32 -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  uint32_t v = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  if ((u & 0x7fffffffu) > 0x7f800000u) v = (u >> 16) | 0x40u;
  return v;
}

// CPL adjacent bfloat16 values (rounded from float32) at (voff + soff) bytes.
template <int CPL>
__device__ __forceinline__ void buf_store_bf16(buf_t r, int voff, int soff, const float (&v)[CPL]) {
  if constexpr (CPL == 1) {
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(bf16_rne_bits(v[0])), r,
                                          voff, soff, 0);
  } else {
    static_assert(CPL == 2, "CPL is 1 or 2");
    __builtin_amdgcn_raw_buffer_store_b32(bf16_rne_bits(v[0]) | (bf16_rne_bits(v[1]) << 16), r,
                                          voff, soff, 0);
  }
}

// kAux: the cache-policy bits of the store (2: non-temporal, for outputs
// streamed past the caches: y, and the fused path's Delta, which at four
// times the last-level cache's size would not stay there for the scan)
template <int CPL, int kAux = 0>
__device__ __forceinline__ void buf_store_vals(buf_t r, int voff, int soff, const float (&v)[CPL]) {
  if constexpr (CPL == 1) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), r, voff, soff, kAux);
  } else {
    static_assert(CPL == 2, "CPL is 1 or 2");
    u32x2 u;
    u.x = __float_as_uint(v[0]);
    u.y = __float_as_uint(v[1]);
    __builtin_amdgcn_raw_buffer_store_b64(u, r, voff, soff, kAux);
  }
}
constexpr int kStoreNT = 2;

// SiLU(v) = v * sigmoid(v), the gate of the Mamba block ("Understanding
// Mamba", section 8.1, eq. (9)).  exp2 and the reciprocal run on the
// transcendental unit (about 1 ulp each).
__device__ __forceinline__ float silu(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + fast_exp2(-v * kLog2e));
}

// Which optional parts of the recurrence and the read-out a kernel carries.
//   kZoh : exact zero-order-hold input term Bbar = (Abar - 1) / A * B
//          ("Understanding Mamba", eq. (2)) instead of the first-order Delta B
//   kSkip: feedthrough y += Dskip[d] * x ("Understanding Mamba", eq. (1)/(3))
//   kGate: y *= SiLU(z)  (the gate branch of the Mamba block, eq. (9))
//   kState: the output pass also writes the final state.  A compile-time
//          switch because keeping the store's address live across the step
//          loop costs registers, and with them a wavefront per SIMD.
template <bool kZoh_, bool kSkip_, bool kGate_, bool kState_ = false>
struct Variant {
  static constexpr bool kZoh = kZoh_;
  static constexpr bool kSkip = kSkip_;
  static constexpr bool kGate = kGate_;
  static constexpr bool kState = kState_;
};
using PlainVariant = Variant<false, false, false>;

// Per-lane constants of one chain: A * log2(e), and 1 / A for the exact
// zero-order hold (only read when kZoh).
template <int N, int CPL>
struct ChainConsts {
  float A2[CPL][N];
  float Ainv[CPL][N];
  float Dd[CPL];      // feedthrough (only read when kSkip)
};

// ---- the per-lane sequential pass over a range of steps -----------------------------------
//
// Runs steps [0, nsteps) of one chunk for the lane's CPL chains.  xb/db/yb/zb
// point at (b, t0, first channel of the block); `lane` is the lane index in the
// block (its channels are lane*CPL + c); rows are D elements apart.  Bb/Cb
// point at row (b, t0) of B/C, read through the scalar unit.  The caller
// guarantees nsteps * D * sizeof(float) < 2^31.
// kWithY: also form y_t = sum_n C_t[n] h_t[n] (plus the variant's feedthrough
// and gate) and store it (output pass); otherwise accumulate each chain's
// total step size in S (summary pass).
// x, delta (and z) are prefetched kTile steps ahead.  B_t and C_t are loaded
// one step ahead into two alternating register sets (kTile is even, so the
// set used by a step is fixed at compile time and no copies are needed).
// Lanes past the last channel run the last channel's chain (their addressing
// is clamped), so their stores repeat that channel's value at its address.
template <int N, int CPL, typename T, bool kPairs, bool kWithY, class V = PlainVariant>
__device__ __forceinline__ void scan_steps(const T* __restrict__ xb, const T* __restrict__ db,
                                           const T* __restrict__ Bb, const T* __restrict__ Cb,
                                           const T* __restrict__ zb, float* __restrict__ yb,
                                           const ChainConsts<N, CPL>& k, float (&h)[CPL][N],
                                           double (&S)[CPL], int lane, int64_t D, int nsteps) {
  constexpr int kTile = (CPL == 1) ? 8 : 4;
  constexpr bool kGate = kWithY && V::kGate;
  static_assert(kTile % 2 == 0, "alternating B/C register sets need an even tile");
  const uint32_t in_bytes = static_cast<uint32_t>((int64_t)nsteps * D * sizeof(T));
  const buf_t xr = make_buf(xb, in_bytes);
  const buf_t dr = make_buf(db, in_bytes);
  buf_t zr;
  if constexpr (kGate) zr = make_buf(zb, in_bytes);
  const int in_row = static_cast<int>(D * sizeof(T));
  const int in_lane = lane * CPL * static_cast<int>(sizeof(T));
  buf_t yr;
  int out_row = 0, out_lane = 0;
  if constexpr (kWithY) {
    yr = make_buf(yb, static_cast<uint32_t>((int64_t)nsteps * D * sizeof(float)));
    out_row = static_cast<int>(D * sizeof(float));
    out_lane = lane * CPL * static_cast<int>(sizeof(float));
  }
  // prefetches past the chunk re-read its last row (the SGPR offset is not
  // range-checked by the hardware, so it is clamped here)
  const int last = nsteps > 0 ? nsteps - 1 : 0;
  float xc[kTile][CPL], dc[kTile][CPL], zc[kGate ? kTile : 1][CPL];
#pragma unroll
  for (int j = 0; j < kTile; ++j) {
    const int soff = __builtin_amdgcn_readfirstlane(min(j, last) * in_row);
    buf_load_vals<T, CPL>(xr, in_lane, soff, xc[j]);
    buf_load_vals<T, CPL>(dr, in_lane, soff, dc[j]);
    if constexpr (kGate) buf_load_vals<T, CPL>(zr, in_lane, soff, zc[j]);
  }
  RawRow<N, T, kPairs> Bv[2], Cv[2];
  if (nsteps > 0) {
    Bv[0].load(Bb);
    if constexpr (kWithY) Cv[0].load(Cb);
  }
  for (int base = 0; base < nsteps; base += kTile) {
    float xn[kTile][CPL], dn[kTile][CPL], zn[kGate ? kTile : 1][CPL];
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      const int soff = __builtin_amdgcn_readfirstlane(min(base + kTile + j, last) * in_row);
      buf_load_vals<T, CPL>(xr, in_lane, soff, xn[j]);
      buf_load_vals<T, CPL>(dr, in_lane, soff, dn[j]);
      if constexpr (kGate) buf_load_vals<T, CPL>(zr, in_lane, soff, zn[j]);
    }
    // No branch around a step: steps past the chunk (the last tile's tail) run
    // with delta = 0, which gives Abar = 1 and a zero input term, so the state
    // is left exactly as it was, and store nothing.  (A branch made the
    // compiler merge every state register at its end: a copy per state and
    // step.)
    // The summary's step-size total: the tile's (at most 8) steps are summed
    // in float32, each tile's sum added to the float64 total (one conversion
    // and one float64 add per tile instead of per step; a tile's sum of
    // values below 1 carries a relative error near 2^-24).
    float St[CPL] = {};
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      const int s = base + j;
      const bool live = s < nsteps;              // uniform
      const int cur = j & 1;
      wait_scalar_loads();
      const int64_t nxt = s + 1 < nsteps ? s + 1 : last;
      Bv[cur ^ 1].load(Bb + nxt * N);
      if constexpr (kWithY) Cv[cur ^ 1].load(Cb + nxt * N);
      // The next step's rows are requested here, a whole step ahead of their
      // use; the scheduler would otherwise lift this step's arithmetic above
      // the wait and the loads, leaving each step to wait out its own loads.
      // Only for packed bfloat16 rows: float32 rows take twice the scalar
      // registers, and pinned there they spill.
      if constexpr (RawRow<N, T, kPairs>::kPinnable) __builtin_amdgcn_sched_barrier(0);
      float dl[CPL], dx[CPL], yv[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        dl[c] = live ? dc[j][c] : 0.0f;
        dx[c] = dl[c] * xc[j][c];
        yv[c] = 0.0f;
      }
#pragma unroll
      for (int n = 0; n < N; ++n) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float a = fast_exp2(dl[c] * k.A2[c][n]);               // Abar = exp(delta A)
          if constexpr (V::kZoh) {
            // (Abar - 1) / A * B * x: u = x B / A, then a u - u in one rounding
            const float u = (xc[j][c] * k.Ainv[c][n]) * Bv[cur].get(n);
            h[c][n] = __builtin_fmaf(a, h[c][n], __builtin_fmaf(a, u, -u));
          } else {
            h[c][n] = __builtin_fmaf(a, h[c][n], dx[c] * Bv[cur].get(n));  // h = Abar h + (delta B) x
          }
          if constexpr (kWithY) yv[c] = __builtin_fmaf(Cv[cur].get(n), h[c][n], yv[c]);  // C . h
        }
      }
      if constexpr (kWithY) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          if constexpr (V::kSkip) yv[c] = __builtin_fmaf(k.Dd[c], xc[j][c], yv[c]);
          if constexpr (kGate) yv[c] *= silu(zc[j][c]);
        }
        if constexpr (RawRow<N, T, kPairs>::kPinnable) {
          // No branch around the store here: with one, the compiler moved the
          // read-out and a fresh load of C_t into it, and every step waited
          // for that load.  A dead step's store gets a per-lane offset of
          // 2^31, past the buffer's byte limit (nsteps * D * 4 < 2^31), which
          // the hardware range check drops.
          buf_store_vals<CPL, kStoreNT>(yr, live ? out_lane : int(0x80000000u), live ? s * out_row : 0, yv);
        } else {
          // (float32 rows: holding both prefetched rows costs more scalar
          // registers than there are, and the branch lets the compiler
          // reload C_t instead)
          if (live) buf_store_vals<CPL, kStoreNT>(yr, out_lane, s * out_row, yv);
        }
      } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) St[c] += dl[c];
      }
    }
    if constexpr (!kWithY) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) S[c] += static_cast<double>(St[c]);
    }
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        xc[j][c] = xn[j][c];
        dc[j][c] = dn[j][c];
        if constexpr (kGate) zc[j][c] = zn[j][c];
      }
    }
  }
}

}  // namespace mssm
