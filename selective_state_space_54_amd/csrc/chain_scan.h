// Single-pass selective scan with one lane per (channel, state index), N = 16.
//
// The chunked kernels give a lane a channel's N states and cut time into
// chunks for parallelism, which costs a summary pass over every chunk but the
// last and a second read of x and delta.  When batch * D channels already fill
// the chip with one lane per state (12288 channels x 16 states = 3072
// wavefronts, three per SIMD on MI355X), each lane can instead run its
// (channel, n) chain over the whole sequence once.
//
// Layout.  A wavefront holds 4 channels x 16 state indices: DPP row c (16
// lanes) is channel c, lane n of the row is state n.  A block is 4 wavefronts,
// 16 adjacent channels of one batch row (D is a multiple of 16).  Time goes in
// tiles of 16 steps:
//   * inputs enter through LDS.  Each wavefront loads one whole 16 x 16 tile
//     per step of the pipeline (wavefront 0: x, and z with the gate; 1: delta;
//     2: B; 3: C), 4 values per lane, so every load instruction covers 16
//     rows x 64 bytes instead of each wavefront fetching 16 rows x 16 bytes
//     of each input (that version spent most of its time in the texture
//     address unit).  B and C are written transposed so that lane n reads
//     B[t0 .. t0 + 15][n] with four 16-byte LDS reads;
//   * loads run two tiles ahead and keep their raw bits until they are
//     written to LDS, so no wait for them sits inside a tile;
//   * per step: a = exp2(delta A[n] log2 e); h = a h + (delta x) B_t[n]
//     (first order) or h = a h + (a - 1) (x B_t[n] / A[n]) (exact zero-order
//     hold); p_t = C_t[n] h ("Understanding Mamba", eq. (2)-(3)).  delta and
//     delta x reach the row's lanes as DPP row_newbcast operands, which cost
//     no extra instruction;
//   * y_t = sum over the row of p_t: after the 16 steps a reduce-scatter over
//     the row leaves lane n holding y of step t0 + n of its channel, which is
//     the (step, channel) of the x value the lane loaded, so the feedthrough
//     D x and the SiLU(z) gate are applied there;
//   * y leaves through LDS too: one wavefront per tile (in turn) stores the
//     block's 16 x 16 tile with 16-byte stores.
// One barrier per tile; LDS buffers alternate between tiles.  Steps past the
// end of the sequence (the last, partial tile) read the last step's values
// with delta = 0, which leaves the state unchanged, and store nothing.
#pragma once

#include "mssm_internal.h"
#include "scan_device.h"

namespace mssm {
namespace chain {

constexpr int kWaves = 4;                // wavefronts per block
constexpr int kBlock = 64 * kWaves;
constexpr int kStates = 16;              // N handled by this design
constexpr int kTile = 16;                // steps per tile = lanes per DPP row
constexpr int kChannels = 4 * kWaves;    // channels per block
// LDS row stride (floats) of the [16][16] tiles: rows stay 16-byte aligned,
// so 4-value accesses along a row are single 16-byte ones.  The LDS serves
// 32 banks of 4 bytes per half wavefront (measured: a stride of 32 words
// costs as much as 64), so the per-lane column accesses (lane (c, n) at row
// n, column 4w + c) meet each bank twice; a stride of 18 avoids that but
// splits the row accesses, and measured slower.
constexpr int kRow = 20;

// 4 consecutive floats of an LDS tile row, starting at a multiple of 4
// columns: one 16-byte access when rows are 16-byte aligned, else two 8-byte
// ones.
__device__ __forceinline__ float4 lds_get4(const float* p) {
  if constexpr (kRow % 4 == 0) return *reinterpret_cast<const float4*>(p);
  const float2 a = *reinterpret_cast<const float2*>(p);
  const float2 b = *reinterpret_cast<const float2*>(p + 2);
  return make_float4(a.x, a.y, b.x, b.y);
}
__device__ __forceinline__ void lds_put4(float* p, float a, float b, float c, float d) {
  if constexpr (kRow % 4 == 0) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  } else {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
    *reinterpret_cast<float2*>(p + 2) = make_float2(c, d);
  }
}

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
// Value of lane s of the lane's DPP row (row_newbcast).
template <int s>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + s, 0xF, 0xF, true));
}
constexpr int kQuadXor2 = 0x4E, kQuadXor1 = 0xB1;

// row_bcast for an index known after unrolling (s must fold to a constant)
__device__ __forceinline__ float row_bcast_dyn(float v, int s) {
  switch (s) {
    case 0: return row_bcast<0>(v);   case 1: return row_bcast<1>(v);
    case 2: return row_bcast<2>(v);   case 3: return row_bcast<3>(v);
    case 4: return row_bcast<4>(v);   case 5: return row_bcast<5>(v);
    case 6: return row_bcast<6>(v);   case 7: return row_bcast<7>(v);
    case 8: return row_bcast<8>(v);   case 9: return row_bcast<9>(v);
    case 10: return row_bcast<10>(v); case 11: return row_bcast<11>(v);
    case 12: return row_bcast<12>(v); case 13: return row_bcast<13>(v);
    case 14: return row_bcast<14>(v); default: return row_bcast<15>(v);
  }
}

// The same value under a name the compiler cannot see through (no
// instruction).  A DPP move is folded into its consumer only when every use
// of it can take the DPP operand; broadcasting separate copies for separate
// consumers keeps each move single-use, where otherwise one shared move would
// be kept in a register per step of the tile and cost an instruction.
__device__ __forceinline__ float opaque(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// The first two reduce levels below, for 16 values, as one asm block: one
// s_nop 1 covers the two wait states a DPP read needs after a VALU write of
// its source (for the inputs, written by compiler code the asm cannot see);
// inside the block every DPP source was written at least 6 instructions
// earlier.
#define MSSM_L1(I, J)                                                              \
  "v_add_f32_dpp %[q" #I "], %[p" #I "], %[p" #I "] row_ror:8 row_mask:0xf bank_mask:0x3\n\t" \
  "v_add_f32_dpp %[q" #I "], %[p" #J "], %[p" #J "] row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
#define MSSM_L2(I, A, B)                                                                     \
  "v_add_f32_dpp %[r" #I "], %[q" #A "], %[q" #A "] row_half_mirror row_mask:0xf bank_mask:0x5\n\t" \
  "v_add_f32_dpp %[r" #I "], %[q" #B "], %[q" #B "] row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
__device__ __forceinline__ void reduce_levels12(const float (&p)[16], float (&q4)[4]) {
  float q8[8];
  asm volatile("s_nop 1\n\t"
               MSSM_L1(0, 8) MSSM_L1(1, 9) MSSM_L1(2, 10) MSSM_L1(3, 11)
               MSSM_L1(4, 12) MSSM_L1(5, 13) MSSM_L1(6, 14) MSSM_L1(7, 15)
               MSSM_L2(0, 0, 4) MSSM_L2(1, 1, 5) MSSM_L2(2, 2, 6) MSSM_L2(3, 3, 7)
               : [q0] "=&v"(q8[0]), [q1] "=&v"(q8[1]), [q2] "=&v"(q8[2]), [q3] "=&v"(q8[3]),
                 [q4] "=&v"(q8[4]), [q5] "=&v"(q8[5]), [q6] "=&v"(q8[6]), [q7] "=&v"(q8[7]),
                 [r0] "=&v"(q4[0]), [r1] "=&v"(q4[1]), [r2] "=&v"(q4[2]), [r3] "=&v"(q4[3])
               : [p0] "v"(p[0]), [p1] "v"(p[1]), [p2] "v"(p[2]), [p3] "v"(p[3]),
                 [p4] "v"(p[4]), [p5] "v"(p[5]), [p6] "v"(p[6]), [p7] "v"(p[7]),
                 [p8] "v"(p[8]), [p9] "v"(p[9]), [p10] "v"(p[10]), [p11] "v"(p[11]),
                 [p12] "v"(p[12]), [p13] "v"(p[13]), [p14] "v"(p[14]), [p15] "v"(p[15]));
}
// Level 2 alone (for sums whose first level ran step by step).
__device__ __forceinline__ void reduce_level2(const float (&q8)[8], float (&q4)[4]) {
  asm volatile("s_nop 1\n\t"
               MSSM_L2(0, 0, 4) MSSM_L2(1, 1, 5) MSSM_L2(2, 2, 6) MSSM_L2(3, 3, 7)
               : [r0] "=&v"(q4[0]), [r1] "=&v"(q4[1]), [r2] "=&v"(q4[2]), [r3] "=&v"(q4[3])
               : [q0] "v"(q8[0]), [q1] "v"(q8[1]), [q2] "v"(q8[2]), [q3] "v"(q8[3]),
                 [q4] "v"(q8[4]), [q5] "v"(q8[5]), [q6] "v"(q8[6]), [q7] "v"(q8[7]));
}
#undef MSSM_L1
#undef MSSM_L2

// Levels 3 and 4: within each bank of 4 lanes (quad_perm partners n ^ 2,
// then n ^ 1), selecting which value a lane keeps and which it sends.
__device__ __forceinline__ float reduce_levels34(const float (&q4)[4], int n) {
  float q2[2];
  bool up = (n & 2) != 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float keep = up ? q4[i + 2] : q4[i], send = up ? q4[i] : q4[i + 2];
    q2[i] = keep + dpp<kQuadXor2>(send);
  }
  up = (n & 1) != 0;
  const float keep = up ? q2[1] : q2[0], send = up ? q2[0] : q2[1];
  return keep + dpp<kQuadXor1>(send);
}

// Row total of p[i], scattered: lane n of each DPP row returns the sum over
// the row's 16 lanes of p[n].  Four halving levels.  The first two use the
// DPP bank mask (a bank is 4 lanes of a row) to write each half of the row
// from its own pair of sums, which saves the selects: lanes 0-7 take
// p[i] + p[i] of lane n ^ 8 (row_ror:8), lanes 8-15 take p[i+8] + its
// partner's; then within each half-row (row_half_mirror, partner 7 - n)
// banks 0 and 2 keep the lower index, banks 1 and 3 the upper.  The last two
// levels split lanes inside a bank, so they select.
__device__ __forceinline__ float row_reduce_scatter16(const float (&p)[16], int n) {
  float q4[4];
  reduce_levels12(p, q4);
  return reduce_levels34(q4, n);
}

// Raw bits of 4 consecutive input values of `esz` bytes each (4: float32,
// 2: bfloat16), as loaded: 16 or 8 bytes.
__device__ __forceinline__ uint4 load_raw(const char* p, int esz) {
  if (esz == 4) return *reinterpret_cast<const uint4*>(p);
  const uint2 q = *reinterpret_cast<const uint2*>(p);
  return make_uint4(q.x, q.y, 0u, 0u);
}
__device__ __forceinline__ void unpack_raw(const uint4& q, int esz, float (&v)[4]) {
  if (esz == 4) {
    v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
    v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
  } else {                                   // bfloat16 -> float32, exact
    v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xFFFF0000u);
    v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xFFFF0000u);
  }
}

// Block index -> logical block such that consecutive logical blocks (adjacent
// channels, which share cache lines) run on one XCD: the hardware hands block
// i to XCD i % 8.
__device__ __forceinline__ int64_t xcd_local_block(int64_t bid, int64_t nblk) {
  constexpr int kXcds = 8;
  const int64_t per = nblk / kXcds, rem = nblk % kXcds;
  const int64_t xcd = bid % kXcds, idx = bid / kXcds;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// Element types of what the kernel reads and writes:
//   TX : x and z            TD : delta            TBC : B and C
//   TY : y; float, or uint16_t for a bfloat16 pair y = bf16(y), y_lo =
//        bf16(y - bf16(y)) (round to nearest even), which carries y to about
//        16 significant bits (the Mamba block's input to its output GEMM)
template <typename TX_, typename TD_, typename TBC_, typename TY_>
struct ChainIO {
  using TX = TX_;
  using TD = TD_;
  using TBC = TBC_;
  using TY = TY_;
};

// Pointers and sizes of one call.  B and C are rows of ld_bc elements (N for
// the plain scan; R + 2N when they are columns of the selection projection's
// output).  Dskip / z / h0 / h_last / y_lo are read or written only by the
// variants that use them.
struct ChainParams {
  const void* x;
  const void* delta;
  const void* B;
  const void* C;
  const void* z;
  const float* A;
  const float* Dskip;
  const float* h0;
  float* h_last;
  void* y;
  void* y_lo;
  int64_t L, D, ld_bc;
  float* ck = nullptr;    // [batch, tiles, D, N] states after each tile (the last tile's unused)
  float* y_pre = nullptr; // [batch, L, D] float32 output before the gate
  int64_t ld_y = 0;       // bfloat16 pair output (TY = uint16_t): row stride of y and y_lo
};

// grid: batch * D / 16 blocks of kBlock lanes.  Requirements (checked by the
// launchers): N = 16, D % 16 == 0, float32 inputs 16-byte and bfloat16 inputs
// 8-byte aligned (rows too: ld_bc a multiple of 4), y 16-byte aligned,
// 16 * D * 4 < 2^31.
// kMode: what the launch produces (checkpoints are for the backward pass):
//   kOut     y (and h_last);
//   kCkOnly  no read-out and no y, only the state after every tile but the
//            last, to ck[b, tile, d, n];
//   kOutSave y, those states, and with the gate also y_pre, the output before
//            the gate (which the gate's gradient needs).
constexpr int kOut = 0, kCkOnly = 1, kOutSave = 2;
template <class IO, class V, int kMode = kOut>
__global__ __launch_bounds__(kBlock) void chain_scan_kernel(ChainParams prm) {
  using TX = typename IO::TX;
  using TY = typename IO::TY;
  constexpr bool kCk = kMode == kCkOnly;
  constexpr bool kSave = kMode == kOutSave;
  constexpr bool kPre = kSave && V::kGate;
  constexpr int kTiles = V::kGate ? 5 : 4;     // x, delta, B^T, C^T (, z)
  __shared__ __align__(16) float tin[2][kTiles][kTile][kRow];
  __shared__ __align__(16) float tout[2][kTile][kRow];
  __shared__ __align__(16) float tpre[kPre ? 2 : 1][kTile][kRow];   // y before the gate
  const int64_t L = prm.L, D = prm.D;

  const int64_t n_dgroups = D / kChannels;
  const int64_t blk = xcd_local_block(blockIdx.x, gridDim.x);
  const int64_t dg = blk % n_dgroups;
  const int64_t b = blk / n_dgroups;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int ch = wave * 4 + (lane >> 4);       // channel within the block
  const int64_t d0 = dg * kChannels;
  const int64_t chain_idx = (b * D + d0 + ch) * kStates + n;   // [batch, D, N] index
  const float a_dn = prm.A[(d0 + ch) * kStates + n];
  const float A2 = a_dn * kLog2e;
  float Ainv = 0.0f;
  if constexpr (V::kZoh) Ainv = 1.0f / a_dn;
  float Dd = 0.0f;
  if constexpr (V::kSkip) Dd = prm.Dskip[d0 + ch];
  float h = prm.h0 ? prm.h0[chain_idx] : 0.0f;

  // Loader lane: step ls of the tile, 4 values from column lq, of the tile
  // this wavefront loads (0: x (and z), 1: delta, 2: B, 3: C).
  const int ls = lane >> 2, lq = (lane & 3) * 4;
  const char* src;
  int esz;              // bytes per element of this wavefront's tile
  int64_t rs;           // elements between rows (steps)
  if (wave == 0) {
    src = static_cast<const char*>(prm.x) + (b * L * D + d0) * sizeof(TX);
    esz = sizeof(TX);
    rs = D;
  } else if (wave == 1) {
    src = static_cast<const char*>(prm.delta) + (b * L * D + d0) * sizeof(typename IO::TD);
    esz = sizeof(typename IO::TD);
    rs = D;
  } else {
    src = static_cast<const char*>(wave == 2 ? prm.B : prm.C) +
          b * L * prm.ld_bc * sizeof(typename IO::TBC);
    esz = sizeof(typename IO::TBC);
    rs = prm.ld_bc;
  }
  const char* zsrc = V::kGate ? static_cast<const char*>(prm.z) + (b * L * D + d0) * sizeof(TX)
                              : nullptr;   // loaded by wavefront 0
  // y rows: D apart, or ld_y apart for the bfloat16 pair (y and y_lo may then
  // be the two column halves of one [batch * L, 2 D] matrix)
  int64_t ldy = D;
  if constexpr (sizeof(TY) == 2) ldy = prm.ld_y;
  char* yb = static_cast<char*>(prm.y) + (b * L * ldy + d0) * sizeof(TY);
  char* yb_lo = sizeof(TY) == 2 ? static_cast<char*>(prm.y_lo) + (b * L * ldy + d0) * sizeof(TY)
                                : nullptr;
  const int64_t ntiles = (L + kTile - 1) / kTile;
  const int64_t last = ntiles - 1;
  const int tail_steps = static_cast<int>(L - last * kTile);   // steps of the last tile, 1..16
  const int ls_tail = ls < tail_steps ? ls : tail_steps - 1;
  const int64_t rs_bytes = rs * esz;
  const uint32_t off_full = static_cast<uint32_t>(ls * rs_bytes + lq * esz);
  const uint32_t off_tail = static_cast<uint32_t>(ls_tail * rs_bytes + lq * esz);
  const uint32_t zoff_full = static_cast<uint32_t>((ls * D + lq) * sizeof(TX));
  const uint32_t zoff_tail = static_cast<uint32_t>((ls_tail * D + lq) * sizeof(TX));
  const bool pad_lane = ls >= tail_steps;
  const uint32_t yoff = static_cast<uint32_t>((ls * ldy + lq) * sizeof(TY));

  struct Regs {
    uint4 v, zv;
  };
  auto load = [&](Regs& r, int64_t k) {
    r.v = load_raw(src + k * kTile * rs_bytes + (k == last ? off_tail : off_full), esz);
    if constexpr (V::kGate) {
      if (wave == 0)
        r.zv = load_raw(zsrc + k * kTile * D * static_cast<int64_t>(sizeof(TX)) +
                            (k == last ? zoff_tail : zoff_full),
                        sizeof(TX));
    }
  };
  // Tile k's loaded values into LDS buffer `buf`.
  auto put = [&](const Regs& r, int buf, int64_t k) {
    float v[4];
    unpack_raw(r.v, esz, v);
    if (wave == 1 && k == last) {   // a uniform branch: the other tiles pay nothing
      if (pad_lane) v[0] = v[1] = v[2] = v[3] = 0.0f;   // delta of steps past the end
    }
    if (wave < 2) {
      lds_put4(&tin[buf][wave][ls][lq], v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) tin[buf][wave][lq + i][ls] = v[i];
    }
    if constexpr (V::kGate) {
      if (wave == 0) {
        unpack_raw(r.zv, sizeof(TX), v);
        lds_put4(&tin[buf][4][ls][lq], v[0], v[1], v[2], v[3]);
      }
    }
  };
  auto store_y = [&](int64_t k) {
    if constexpr (kCk) return;
    const float4 v = lds_get4(&tout[k & 1][ls][lq]);
    float4 u;
    if constexpr (kPre) u = lds_get4(&tpre[k & 1][ls][lq]);
    if (k == last && ls >= tail_steps) return;
    if constexpr (kPre)
      *reinterpret_cast<float4*>(prm.y_pre + (b * L + k * kTile + ls) * D + d0 + lq) = u;
    const int64_t step_bytes = k * kTile * ldy * static_cast<int64_t>(sizeof(TY));
    if constexpr (sizeof(TY) == 4) {
      *reinterpret_cast<float4*>(yb + step_bytes + yoff) = v;
    } else {
      const float w[4] = {v.x, v.y, v.z, v.w};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[i] = bf16_rne_bits(w[i]);
        lo[i] = bf16_rne_bits(w[i] - __uint_as_float(hi[i] << 16));
      }
      *reinterpret_cast<uint2*>(yb + step_bytes + yoff) =
          make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
      *reinterpret_cast<uint2*>(yb_lo + step_bytes + yoff) =
          make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
    }
  };
  auto checkpoint = [&](int64_t k) {
    const int buf = k & 1;
    const float xv = tin[buf][0][n][ch];
    const float dv = tin[buf][1][n][ch];
    float Bt[kTile];
#pragma unroll
    for (int j = 0; j < kTile / 4; ++j) {
      const float4 vb = lds_get4(&tin[buf][2][n][4 * j]);
      Bt[4 * j] = vb.x; Bt[4 * j + 1] = vb.y; Bt[4 * j + 2] = vb.z; Bt[4 * j + 3] = vb.w;
    }
    const float uv = dv * xv;
#pragma unroll
    for (int s = 0; s < kTile; ++s) {
      const float a = fast_exp2(row_bcast_dyn(dv, s) * A2);
      h = __builtin_fmaf(a, h, row_bcast_dyn(uv, s) * Bt[s]);
    }
    if (k < last) prm.ck[((b * ntiles + k) * D + d0 + ch) * kStates + n] = h;
  };
  auto compute = [&](int64_t k) {
    if constexpr (kCk) {
      checkpoint(k);
      return;
    }
    const int buf = k & 1;
    const float xv = tin[buf][0][n][ch];
    const float dv = tin[buf][1][n][ch];
    float Bt[kTile], Ct[kTile];
#pragma unroll
    for (int j = 0; j < kTile / 4; ++j) {
      const float4 vb = lds_get4(&tin[buf][2][n][4 * j]);
      const float4 vc = lds_get4(&tin[buf][3][n][4 * j]);
      Bt[4 * j] = vb.x; Bt[4 * j + 1] = vb.y; Bt[4 * j + 2] = vb.z; Bt[4 * j + 3] = vb.w;
      Ct[4 * j] = vc.x; Ct[4 * j + 1] = vc.y; Ct[4 * j + 2] = vc.z; Ct[4 * j + 3] = vc.w;
    }
    float p[kTile];
    if constexpr (V::kZoh) {
#pragma unroll
      for (int s = 0; s < kTile; ++s) Bt[s] *= Ainv;
    }
    const float uv = V::kZoh ? xv : dv * xv;   // broadcast input factor of the step
#define MSSM_CHAIN_STEP(S)                                                    \
    {                                                                         \
      const float a = fast_exp2(row_bcast<S>(dv) * A2);                       \
      const float w = row_bcast<S>(uv) * Bt[S];                               \
      h = __builtin_fmaf(a, h, V::kZoh ? __builtin_fmaf(a, w, -w) : w);       \
      p[S] = Ct[S] * h;                                                       \
    }
    MSSM_CHAIN_STEP(0) MSSM_CHAIN_STEP(1) MSSM_CHAIN_STEP(2) MSSM_CHAIN_STEP(3)
    MSSM_CHAIN_STEP(4) MSSM_CHAIN_STEP(5) MSSM_CHAIN_STEP(6) MSSM_CHAIN_STEP(7)
    MSSM_CHAIN_STEP(8) MSSM_CHAIN_STEP(9) MSSM_CHAIN_STEP(10) MSSM_CHAIN_STEP(11)
    MSSM_CHAIN_STEP(12) MSSM_CHAIN_STEP(13) MSSM_CHAIN_STEP(14) MSSM_CHAIN_STEP(15)
#undef MSSM_CHAIN_STEP
    float yv = row_reduce_scatter16(p, n);     // y of step n of this row's channel
    if constexpr (V::kSkip) yv = __builtin_fmaf(Dd, xv, yv);
    if constexpr (kPre) tpre[buf][n][ch] = yv;
    if constexpr (kSave) {
      if (k < last) prm.ck[((b * ntiles + k) * D + d0 + ch) * kStates + n] = h;
    }
    if constexpr (V::kGate) yv *= silu(tin[buf][4][n][ch]);
    tout[buf][n][ch] = yv;
  };

  // Pipeline.  Iteration k: barrier; the y tile of k - 1 goes out; tile k + 1
  // (loaded two iterations earlier) goes into LDS; tile k + 3 is loaded;
  // tile k is computed.  Unrolled by two so the two register sets have fixed
  // names.  Loads past the last tile repeat it and are never used.
  Regs r0, r1;
  load(r0, 0);
  load(r1, 1 < last ? 1 : last);
  put(r0, 0, 0);
  load(r0, 2 < last ? 2 : last);
  int64_t k = 0;
  for (; k + 2 <= ntiles; k += 2) {
    block_sync();
    if (k >= 1 && wave == ((k - 1) & 3)) store_y(k - 1);
    put(r1, 1, k + 1);
    load(r1, k + 3 < last ? k + 3 : last);
    compute(k);
    block_sync();
    if (wave == (k & 3)) store_y(k);
    put(r0, 0, k + 2);
    load(r0, k + 4 < last ? k + 4 : last);
    compute(k + 1);
  }
  if (k < ntiles) {
    block_sync();
    if (k >= 1 && wave == ((k - 1) & 3)) store_y(k - 1);
    compute(k);
  }
  block_sync();
  if (wave == (last & 3)) store_y(last);
  if constexpr (V::kState) prm.h_last[chain_idx] = h;
}

// Launch on `stream` for `batch` rows; returns the launch status.
template <class IO, class V, int kMode = kOut>
hipError_t launch_io(const ChainParams& p, int64_t batch, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(batch * (p.D / kChannels)));
  hipLaunchKernelGGL((chain_scan_kernel<IO, V, kMode>), grid, dim3(kBlock), 0, stream, p);
  return hipGetLastError();
}

template <class V>
hipError_t launch_variant(const ScanArgs& a, hipStream_t stream);
// y plus the saved states (and y_pre with the gate), first-order input term
template <class V>
hipError_t launch_save(const ScanArgs& a, float* ck, float* y_pre, hipStream_t stream);

}  // namespace chain

// The plain and extended scan: x, delta, B, C (and z) all of the call's dtype,
// B and C rows of N = 16, y float32.
#define MSSM_DEFINE_CHAIN_VARIANT(ZOH, SKIP, GATE, STATE)                                     \
  template <>                                                                                 \
  hipError_t chain::launch_variant<Variant<ZOH, SKIP, GATE, STATE>>(const ScanArgs& a,        \
                                                                    hipStream_t stream) {    \
    using V = Variant<ZOH, SKIP, GATE, STATE>;                                                \
    const chain::ChainParams p{a.x,      a.delta, a.B,      a.C, a.z, a.A, a.Dskip, a.h0,      \
                               a.h_last, a.y,     nullptr,  a.L, a.D, chain::kStates};         \
    if (a.dtype == MSSM_FLOAT32)                                                              \
      return chain::launch_io<chain::ChainIO<float, float, float, float>, V>(p, a.batch,      \
                                                                             stream);         \
    return chain::launch_io<chain::ChainIO<uint16_t, uint16_t, uint16_t, float>, V>(          \
        p, a.batch, stream);                                                                  \
  }

// The forward that also saves what the backward reads: y float32, first-order
// input term, the optional parts of V.
#define MSSM_DEFINE_CHAIN_SAVE(SKIP, GATE, STATE)                                              \
  template <>                                                                                 \
  hipError_t chain::launch_save<Variant<false, SKIP, GATE, STATE>>(                           \
      const ScanArgs& a, float* ck, float* y_pre, hipStream_t stream) {                       \
    using V = Variant<false, SKIP, GATE, STATE>;                                              \
    chain::ChainParams p{a.x,      a.delta, a.B,      a.C, a.z, a.A, a.Dskip, a.h0,            \
                         a.h_last, a.y,     nullptr,  a.L, a.D, chain::kStates};               \
    p.ck = ck;                                                                                \
    p.y_pre = y_pre;                                                                          \
    if (a.dtype == MSSM_FLOAT32)                                                              \
      return chain::launch_io<chain::ChainIO<float, float, float, float>, V, chain::kOutSave>( \
          p, a.batch, stream);                                                                \
    return chain::launch_io<chain::ChainIO<uint16_t, uint16_t, uint16_t, float>, V,           \
                            chain::kOutSave>(p, a.batch, stream);                             \
  }

}  // namespace mssm
