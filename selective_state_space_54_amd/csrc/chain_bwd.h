// Backward pass of the selective scan in the single-pass layout (one lane per
// channel and state index, N = 16, D % 16 == 0): the gradients of
// "Understanding Mamba" eq. (2)-(3) with the first-order input term, the
// feedthrough D x and the SiLU(z) gate, by recomputation ("State Space Models
// and Mamba", hardware-aware scan: the backward recomputes the states).
//
// With g_t = dout_t SiLU(z_t), a_t = exp(delta_t A), u_t = delta_t x_t B_t:
//   lam_t = C_t g_t + a_{t+1} lam_{t+1}            (the adjoint, lam_L = 0)
//   dx_t = g_t D + delta_t sum_n lam_t B_t       ddelta_t = x_t sum_n lam_t B_t
//                                                          + sum_n lam_t A a_t h_{t-1}
//   dA += lam_t delta_t a_t h_{t-1}   dB_t += lam_t delta_t x_t   dC_t += g_t h_t
//   dD += g_t x_t   dz_t = dout_t y_t SiLU'(z_t)   dh0 = a_0 lam_0
//
// A first pass (chain_scan_kernel in checkpoint mode) stores every lane's
// state after each 16-step tile, unless the forward call saved them (kOutSave,
// which also keeps y before the gate: then dz reads it instead of reading y
// out here).  This kernel walks the tiles backwards: a
// lane recomputes its tile's 16 states from the checkpoint into registers,
// then sweeps the tile backwards carrying a_{t+1} lam_{t+1} across tiles.
// Sums over n (dx, ddelta, and y for dz) are the row reduce-scatter of the
// forward read-out, landing on the lane that owns the step.  Sums over
// channels (dB, dC) fold the wavefront's four rows with permlane swaps, the
// four wavefronts through LDS, and leave one partial per block of 16
// channels for a separate reduction; dA and dD leave one partial per batch
// row.  Inputs and outputs move through LDS in 16 x 16 tiles as in the
// forward kernel.
#pragma once

#include "chain_scan.h"

namespace mssm {
namespace chain {

struct ChainBwdParams {
  const void* x;
  const void* delta;
  const void* B;
  const void* C;
  const void* z;            // or null
  const float* A;
  const float* Dskip;       // or null
  const float* h0;          // or null
  const float* dout;        // [batch, L, D]
  const float* ck;          // [batch, tiles, D, N]: state after each tile (the last unused)
  const float* y_pre;       // [batch, L, D] output before the gate (saved forward), or null
  float* dx;                // [batch, L, D]
  float* ddelta;
  float* dz;                // with z
  float* dh0;               // or null
  float* part_bc;           // [D / 16, batch * L, 2N]: dB | dC per block
  float* part_a;            // [batch, D, N]
  float* part_d;            // [batch, D], with Dskip
  int64_t L, D;
};

__device__ __forceinline__ float silu_grad(float v) {   // d/dv (v sigmoid(v))
  const float s = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-v * kLog2e));
  return s * (1.0f + v * (1.0f - s));
}

// a + b after permlane32_swap: lanes 0..31 get a summed with a of lanes
// 32..63, lanes 32..63 get b summed with b of lanes 0..31 (rows r and r + 2).
__device__ __forceinline__ float fold_rows2(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// the same with permlane16_swap: rows 0 and 2 get a summed with the next row's
// a, rows 1 and 3 get b summed with the previous row's b.
__device__ __forceinline__ float fold_rows1(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The row reduce-scatter of row_reduce_scatter16 in two parts, so that its
// first level can run as soon as both of its operands exist: rs_first(p[i],
// p[i + 8]) gives q8[i]; rs_rest(q8) finishes (lane n of the row returns the
// row total of p[n]).
__device__ __forceinline__ float rs_first(float lo, float hi) {
  float q;
  asm volatile(
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %0, %2, %2 row_ror:8 row_mask:0xf bank_mask:0xc"
      : "=&v"(q)
      : "v"(lo), "v"(hi));
  return q;
}
__device__ __forceinline__ float rs_rest(const float (&q8)[8], int n) {
  float q4[4];
  reduce_level2(q8, q4);
  return reduce_levels34(q4, n);
}

// acc += (value of lane s of the DPP row of v) * m in one instruction
// (v_fmac_f32 with a row_newbcast operand, which the compiler does not form by
// itself).  A DPP read needs two wait states after a VALU write of its
// source, which the compiler does not check inside asm: v must have been made
// ready with dpp_sources_ready (tests/test_isa_checks_cpu.py checks the built
// code for such hazards).
template <int s>
__device__ __forceinline__ void fmac_bcast(float& acc, float v, float m) {
  asm volatile(
      "v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "+v"(acc)
      : "v"(v), "v"(m), "i"(s));
}
// Two wait states after v and w are final, before fmac_bcast reads them
// through DPP: a tile's broadcast sources are computed once, so one s_nop
// before its sweep replaces one per instruction.
__device__ __forceinline__ void dpp_sources_ready(float v, float w) {
  asm volatile("s_nop 1" ::"v"(v), "v"(w));
}
__device__ __forceinline__ void fmac_bcast_dyn(float& acc, float v, float m, int s) {
  switch (s) {
    case 0: fmac_bcast<0>(acc, v, m); break;   case 1: fmac_bcast<1>(acc, v, m); break;
    case 2: fmac_bcast<2>(acc, v, m); break;   case 3: fmac_bcast<3>(acc, v, m); break;
    case 4: fmac_bcast<4>(acc, v, m); break;   case 5: fmac_bcast<5>(acc, v, m); break;
    case 6: fmac_bcast<6>(acc, v, m); break;   case 7: fmac_bcast<7>(acc, v, m); break;
    case 8: fmac_bcast<8>(acc, v, m); break;   case 9: fmac_bcast<9>(acc, v, m); break;
    case 10: fmac_bcast<10>(acc, v, m); break; case 11: fmac_bcast<11>(acc, v, m); break;
    case 12: fmac_bcast<12>(acc, v, m); break; case 13: fmac_bcast<13>(acc, v, m); break;
    case 14: fmac_bcast<14>(acc, v, m); break; default: fmac_bcast<15>(acc, v, m); break;
  }
}

constexpr int kBcRow = 48;   // floats per step row of the dB | dC partial tile

// grid: batch * D / 16 blocks of kBlock lanes.
// kSaved: the checkpoints come from the forward call, and with the gate so
// does y_pre, which then replaces this kernel's own read-out of y.
template <typename T, bool kSkip, bool kGate, bool kSaved>
__global__ __launch_bounds__(kBlock) void chain_bwd_kernel(ChainBwdParams prm) {
  constexpr bool kPre = kSaved && kGate;   // y_pre read, not recomputed
  // inputs [buffer][x, delta, B^T, C^T, dout, z]; outputs [buffer][dx, ddelta, dz];
  // dB/dC partials [buffer][wavefront][step][dB n | dC n]
  __shared__ __align__(16) float tin[2][kPre ? 7 : 6][kTile][kRow];
  __shared__ __align__(16) float tout[2][3][kTile][kRow];
  // (rows of kBcRow floats: the two steps a wavefront writes at once then
  // land 16 banks apart)
  __shared__ __align__(16) float tbc[2][kWaves][kTile][kBcRow];
  const int64_t L = prm.L, D = prm.D;
  const int64_t n_dgroups = D / kChannels;
  const int64_t blk = xcd_local_block(blockIdx.x, gridDim.x);
  const int64_t dg = blk % n_dgroups;
  const int64_t b = blk / n_dgroups;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int row = lane >> 4;
  const int ch = wave * 4 + row;
  const int64_t d0 = dg * kChannels;
  const int64_t chain_idx = (b * D + d0 + ch) * kStates + n;
  const float An = prm.A[(d0 + ch) * kStates + n];
  const float A2 = An * kLog2e;
  float Dd = 0.0f;
  if constexpr (kSkip) Dd = prm.Dskip[d0 + ch];
  const int64_t ntiles = (L + kTile - 1) / kTile;
  const int64_t last = ntiles - 1;
  const int tail_steps = static_cast<int>(L - last * kTile);

  // Loads: wavefront 0 x (and z), 1 delta and dout, 2 B (and y_pre), 3 C; 4
  // values per lane.
  const int ls = lane >> 2, lq = (lane & 3) * 4;
  const int ls_tail = ls < tail_steps ? ls : tail_steps - 1;
  const char* src;
  const char* src2 = nullptr;
  int esz = sizeof(T), esz2 = sizeof(T);
  int64_t rs = D;
  if (wave == 0) {
    src = static_cast<const char*>(prm.x) + (b * L * D + d0) * sizeof(T);
    if constexpr (kGate) src2 = static_cast<const char*>(prm.z) + (b * L * D + d0) * sizeof(T);
  } else if (wave == 1) {
    src = static_cast<const char*>(prm.delta) + (b * L * D + d0) * sizeof(T);
    src2 = reinterpret_cast<const char*>(prm.dout + b * L * D + d0);
    esz2 = 4;
  } else {
    src = static_cast<const char*>(wave == 2 ? prm.B : prm.C) + b * L * kStates * sizeof(T);
    rs = kStates;
    if (kPre && wave == 2) {
      src2 = reinterpret_cast<const char*>(prm.y_pre + b * L * D + d0);
      esz2 = 4;
    }
  }
  const int64_t rs_bytes = rs * esz;
  const uint32_t off_full = static_cast<uint32_t>(ls * rs_bytes + lq * esz);
  const uint32_t off_tail = static_cast<uint32_t>(ls_tail * rs_bytes + lq * esz);
  const uint32_t off2_full = static_cast<uint32_t>((ls * D + lq) * esz2);
  const uint32_t off2_tail = static_cast<uint32_t>((ls_tail * D + lq) * esz2);
  const int64_t tile_bytes = kTile * rs_bytes, tile_bytes2 = kTile * D * esz2;
  const bool has2 = wave == 1 || (kGate && wave == 0) || (kPre && wave == 2);

  struct Regs {
    uint4 v, v2 = make_uint4(0u, 0u, 0u, 0u);
  };
  auto tile_of = [&](int64_t i) {            // iteration i walks tile last - i (clamped at 0)
    return i <= last ? last - i : int64_t(0);
  };
  auto load = [&](Regs& r, int64_t i) {
    const int64_t kt = tile_of(i);
    r.v = load_raw(src + kt * tile_bytes + (kt == last ? off_tail : off_full), esz);
    if (has2) r.v2 = load_raw(src2 + kt * tile_bytes2 + (kt == last ? off2_tail : off2_full), esz2);
  };
  auto put = [&](const Regs& r, int buf, int64_t i) {
    float v[4], w[4];
    unpack_raw(r.v, esz, v);
    unpack_raw(r.v2, esz2, w);   // unused by the wavefronts without a second tile
    // steps past the end: delta and dout zero (the last tile only; a uniform
    // branch, so the other tiles pay nothing for it)
    if (wave == 1 && tile_of(i) == last) {
      if (ls >= tail_steps) v[0] = v[1] = v[2] = v[3] = w[0] = w[1] = w[2] = w[3] = 0.0f;
    }
    if (wave < 2) {
      lds_put4(&tin[buf][wave][ls][lq], v[0], v[1], v[2], v[3]);
      if (has2)
        lds_put4(&tin[buf][wave == 1 ? 4 : 5][ls][lq], w[0], w[1], w[2], w[3]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) tin[buf][wave][lq + q][ls] = v[q];
      if (kPre && wave == 2) lds_put4(&tin[buf][6][ls][lq], w[0], w[1], w[2], w[3]);
    }
  };

  // Stores of a finished tile (iteration i, buffer buf): wavefront 0 dx,
  // 1 ddelta, 2 dz; and each wavefront sums the four wavefronts' dB/dC
  // values of 4 of the tile's steps into the block's partial.
  auto store = [&](int64_t i) {
    const int buf = i & 1;
    const int64_t kt = tile_of(i);
    const int64_t t0 = kt * kTile;
    const int steps = kt == last ? tail_steps : kTile;
    if (wave < 2 || (kGate && wave == 2)) {
      float* dst = wave == 0 ? prm.dx : (wave == 1 ? prm.ddelta : prm.dz);
      const float4 v = lds_get4(&tout[buf][wave][ls][lq]);
      if (ls < steps) *reinterpret_cast<float4*>(dst + (b * L + t0 + ls) * D + d0 + lq) = v;
    }
    const int step = wave * 4 + (lane >> 4), col = (lane & 15) * 2;
    float2 sum = *reinterpret_cast<const float2*>(&tbc[buf][0][step][col]);
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const float2 v = *reinterpret_cast<const float2*>(&tbc[buf][w][step][col]);
      sum.x += v.x;
      sum.y += v.y;
    }
    if (step < steps)
      *reinterpret_cast<float2*>(prm.part_bc +
                                 ((dg * (gridDim.x / n_dgroups) + b) * L + t0 + step) *
                                     (2 * kStates) + col) = sum;
  };

  // state entering a tile: h0 (or 0) for tile 0, else the checkpoint
  auto state_in = [&](int64_t kt) {
    if (kt == 0) return prm.h0 ? prm.h0[chain_idx] : 0.0f;
    return prm.ck[((b * ntiles + kt - 1) * D + d0 + ch) * kStates + n];
  };

  float lamn = 0.0f;       // a_{t+1} lam_{t+1} entering the step being swept
  float dA = 0.0f, dDacc = 0.0f;
  auto compute = [&](int64_t i, float hin) {
    const int buf = i & 1;
    const int64_t kt = tile_of(i);
    const float xv = tin[buf][0][n][ch];
    const float dv = tin[buf][1][n][ch];
    const float go = tin[buf][4][n][ch];
    float zv = 0.0f;
    if constexpr (kGate) zv = tin[buf][5][n][ch];
    // B_t[n] and C_t[n] of the tile's steps, four at a time from LDS
    auto b4 = [&](int j) { return lds_get4(&tin[buf][2][n][4 * j]); };
    auto c4 = [&](int j) { return lds_get4(&tin[buf][3][n][4 * j]); };
    auto el = [](const float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; };
    const float gv = kGate ? go * silu(zv) : go;   // g of step n
    const float uv = dv * xv;
    // a separate copy for the reverse sweep's broadcasts of delta x (see opaque)
    const float uv_r = opaque(uv);
    // recompute: a_s and h_s
    float a[kTile], hs[kTile];
    float hp = hin;
#pragma unroll
    for (int j = 0; j < kTile / 4; ++j) {
      const float4 bq = b4(j);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = 4 * j + e;
        a[s] = fast_exp2(row_bcast_dyn(dv, s) * A2);
        hs[s] = __builtin_fmaf(a[s], hp, row_bcast_dyn(uv, s) * el(bq, e));
        hp = hs[s];
      }
    }
    // backwards through the tile; dB, dC over the wavefront's four channels
    // per pair of steps: rows 0 / 1 / 2 / 3 end with dB of step 2j / dB of
    // 2j + 1 / dC of 2j / dC of 2j + 1.
    // p1 = lam B, p2 = lam A a h_{s-1} (and py = C h for the gate's y) enter
    // sums over n: steps 8..15 wait for their partners 0..7, then both go
    // through the first reduce level
    constexpr int kH = kTile / 2;
    float p1h[kH], p2h[kH], q1[kH], q2[kH];
    float p3h[kGate ? kH : 1], q3[kGate ? kH : 1];
    float vb_odd = 0.0f, vc_odd = 0.0f;
    float4 bq = make_float4(0.0f, 0.0f, 0.0f, 0.0f), cq = bq;
    dpp_sources_ready(gv, dv);
#pragma unroll
    for (int s = kTile - 1; s >= 0; --s) {
      if (s % 4 == 3) {
        bq = b4(s / 4);
        cq = c4(s / 4);
      }
      const float Bs = el(bq, s % 4), Cs = el(cq, s % 4);
      float lam = lamn;
      fmac_bcast_dyn(lam, gv, Cs, s);        // lam = C_s g_s + a_{s+1} lam_{s+1}
      lamn = a[s] * lam;
      const float r = lamn * (s > 0 ? hs[s > 0 ? s - 1 : 0] : hin);   // lam a h_{s-1}
      fmac_bcast_dyn(dA, dv, r, s);
      const float p2 = r * An, p1 = lam * Bs;
      if (s >= kH) {
        p1h[s - kH] = p1;
        p2h[s - kH] = p2;
        if constexpr (kGate && !kPre) p3h[s - kH] = Cs * hs[s];
      } else {
        q1[s] = rs_first(p1, p1h[s]);
        q2[s] = rs_first(p2, p2h[s]);
        if constexpr (kGate && !kPre) q3[s] = rs_first(Cs * hs[s], p3h[s]);
      }
      const float vb = lam * row_bcast_dyn(uv_r, s);
      const float vc = row_bcast_dyn(gv, s) * hs[s];
      if (s & 1) {
        vb_odd = vb;
        vc_odd = vc;
      } else {
        const float lo = fold_rows2(vb, vc);
        const float hi = fold_rows2(vb_odd, vc_odd);
        tbc[buf][wave][s + (row & 1)][(row >> 1) * kStates + n] = fold_rows1(lo, hi);
      }
    }
    if constexpr (kPre) {    // dz = dout y SiLU'(z) with the forward's y = C.h + D x
      tout[buf][2][n][ch] = go * tin[buf][6][n][ch] * silu_grad(zv);
    } else if constexpr (kGate) {   // the same with y read out here
      float y = rs_rest(q3, n);
      if constexpr (kSkip) y = __builtin_fmaf(Dd, xv, y);
      tout[buf][2][n][ch] = go * y * silu_grad(zv);
    }
    const float s1 = rs_rest(q1, n);   // sum_n lam B of step n
    const float s2 = rs_rest(q2, n);   // sum_n lam A a h_{t-1} of step n
    float dxv = dv * s1;
    if constexpr (kSkip) {
      dxv = __builtin_fmaf(gv, Dd, dxv);
      if (kt != last || n < tail_steps) dDacc = __builtin_fmaf(gv, xv, dDacc);
    }
    tout[buf][0][n][ch] = dxv;
    tout[buf][1][n][ch] = __builtin_fmaf(xv, s1, s2);
  };

  // Pipeline (iterations walk the tiles backwards): iteration i: barrier;
  // stores of iteration i - 1; inputs of iteration i + 1 into LDS; loads for
  // iteration i + 3; the checkpoint for iteration i + 1; compute iteration i.
  Regs r0, r1;
  load(r0, 0);
  load(r1, 1);
  put(r0, 0, 0);
  load(r0, 2);
  float hin = state_in(tile_of(0));
  float hin_next = state_in(tile_of(1));
  int64_t i = 0;
  for (; i + 2 <= ntiles; i += 2) {
    block_sync();
    if (i >= 1) store(i - 1);
    put(r1, 1, i + 1);
    load(r1, i + 3);
    compute(i, hin);
    hin = hin_next;
    hin_next = state_in(tile_of(i + 2));
    block_sync();
    store(i);
    put(r0, 0, i + 2);
    load(r0, i + 4);
    compute(i + 1, hin);
    hin = hin_next;
    hin_next = state_in(tile_of(i + 3));
  }
  if (i < ntiles) {
    block_sync();
    if (i >= 1) store(i - 1);
    compute(i, hin);
  }
  block_sync();
  store(last);              // iteration last handles tile 0
  prm.part_a[chain_idx] = dA;
  if (prm.dh0) prm.dh0[chain_idx] = lamn;
  if constexpr (kSkip) {
    float t = dDacc;        // sum over the row's 16 lanes (one step each)
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) t += __shfl_xor(t, o, 16);
    if (n == 0) prm.part_d[b * D + d0 + ch] = t;
  }
}

template <typename T, bool kSkip, bool kGate, bool kSaved>
hipError_t launch_bwd_chain_t(const ChainBwdParams& p, int64_t batch, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(batch * (p.D / kChannels)));
  hipLaunchKernelGGL((chain_bwd_kernel<T, kSkip, kGate, kSaved>), grid, dim3(kBlock), 0, stream, p);
  return hipGetLastError();
}

}  // namespace chain
}  // namespace mssm
