// Single-pass selective scan with the state split across wavefronts (gfx950):
// the scan behind the selection projections when the channels are many
// (the fused selective SSM and the Mamba block at batch * D >= 32768).
//
// The per-element recurrence ("Understanding Mamba", eq. (2)-(3), first-order
// input term as "Selective State Space Models" states Mamba uses):
//   a = exp2(delta A[d,n] log2 e);  h[n] = a h[n] + (delta x) B_t[n];
//   y_t = sum_n C_t[n] h[n]
//
// Layout.  A block covers 64 adjacent channels of one batch row; lane l of
// every wavefront is channel d0 + l, and wavefront w owns state indices
// 4w .. 4w + 3 of those channels.  So:
//   * B_t and C_t are the same for all lanes of a wavefront (4 values each per
//     step): read through the scalar unit from a copy grouped by four state
//     indices (consecutive steps side by side, one wait per 2 steps) into
//     SGPRs, used directly as instruction operands;
//   * delta and u = delta x are per lane: the block stages 8-step tiles of
//     them in LDS once (u formed by the loader), every wavefront reads them;
//   * per element: one multiply for the exponent, v_exp_f32, one multiply for
//     the input term, one fma for the state and one fma for the partial
//     read-out, all plain VALU instructions (no cross-lane operands, which run
//     at half the rate of plain ones on gfx950);
//   * y_t is the sum of the four wavefronts' partial read-outs: each writes
//     its 8 partial sums per lane to LDS, and after the next barrier each
//     wavefront adds up two of the tile's steps (in wavefront order, so the
//     result does not depend on timing), applies the feedthrough and gate and
//     stores y (fp32, or the bf16 hi + lo pair of the block).
// Loads run two tiles ahead; LDS buffers alternate; one barrier per tile, the
// reduction of tile k - 1 runs right after the barrier of tile k.  Steps past
// the end of the sequence get delta = 0 (the state is left as it was) and
// store nothing.
#include <type_traits>

#include "chain_scan.h"

namespace mssm {
namespace split {

constexpr int kWaves = 4;
constexpr int kBlock = 64 * kWaves;
constexpr int kCh = 64;              // channels per block
constexpr int kTile = 8;             // steps per tile
constexpr int kSpw = 4;              // state indices per wavefront
constexpr int64_t kMinChannels = 32768;   // batch * D from which this layout is used

template <typename T>
__device__ __forceinline__ float elem(const T* p, int64_t i) {
  if constexpr (std::is_same_v<T, float>) return p[i];
  else return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// x: bf16 bits (uint16_t) or float32; kSkip: y += Dskip[d] x; kGate: y *=
// SiLU(z), z float32; kPair: y stored as bf16 hi / lo arrays with row stride
// ldy, else float32 rows of D.
template <typename TX, bool kSkip, bool kGate, bool kPair>
__global__ __launch_bounds__(kBlock) void split_scan_kernel(
    const TX* __restrict__ x, const float* __restrict__ delta,
    const float* __restrict__ bcg, int64_t bcg_rows, const float* __restrict__ z,
    const float* __restrict__ A, const float* __restrict__ Dskip, float* __restrict__ y,
    uint16_t* __restrict__ yhi, uint16_t* __restrict__ ylo, int64_t ldy, int64_t L, int64_t D) {
  __shared__ __align__(16) float s_del[2][kTile][kCh];
  __shared__ __align__(16) float s_u[2][kTile][kCh];
  __shared__ __align__(16) float s_part[2][kWaves][kTile][kCh];
  __shared__ __align__(16) float s_x[kSkip ? 2 : 1][kSkip ? kTile : 1][kCh];
  __shared__ __align__(16) float s_z[kGate ? 2 : 1][kGate ? kTile : 1][kCh];

  const int64_t n_dgroups = D / kCh;
  const int64_t blk = chain::xcd_local_block(blockIdx.x, gridDim.x);
  const int64_t b = blk / n_dgroups;
  const int64_t d0 = (blk % n_dgroups) * kCh;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = kSpw * wave;
  const int64_t d = d0 + lane;
  float a2[kSpw], h[kSpw];
#pragma unroll
  for (int i = 0; i < kSpw; ++i) {
    a2[i] = A[d * 16 + n0 + i] * kLog2e;
    h[i] = 0.0f;
  }
  float Dd = 0.0f;
  if constexpr (kSkip) Dd = Dskip[d];

  // loader: thread t stages step t / 32, channels 2 (t % 32) and 2 (t % 32) + 1
  const int ls = threadIdx.x >> 5;
  const int lc = (threadIdx.x & 31) * 2;
  const int64_t row0 = b * L;                      // first row of this batch row
  const int64_t ntiles = (L + kTile - 1) / kTile;
  struct Raw {
    float dl[2], xv[2], zv[2];
  };
  auto load = [&](Raw& r, int64_t k) {
    const int64_t t = k * kTile + ls;
    const int64_t tc = t < L ? t : L - 1;          // clamped: past the end reads the last row
    const int64_t off = (row0 + tc) * D + d0 + lc;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      r.dl[j] = t < L ? delta[off + j] : 0.0f;      // delta = 0 past the end: state kept
      r.xv[j] = elem(x, off + j);
      if constexpr (kGate) r.zv[j] = z[off + j];
    }
  };
  auto put = [&](const Raw& r, int buf) {
    *reinterpret_cast<float2*>(&s_del[buf][ls][lc]) = make_float2(r.dl[0], r.dl[1]);
    *reinterpret_cast<float2*>(&s_u[buf][ls][lc]) =
        make_float2(r.dl[0] * r.xv[0], r.dl[1] * r.xv[1]);
    if constexpr (kSkip)
      *reinterpret_cast<float2*>(&s_x[buf][ls][lc]) = make_float2(r.xv[0], r.xv[1]);
    if constexpr (kGate)
      *reinterpret_cast<float2*>(&s_z[buf][ls][lc]) = make_float2(r.zv[0], r.zv[1]);
  };

  // B_t and C_t of this wavefront's 4 state indices: 8 consecutive floats per
  // step in the grouped copy the projection writes, so consecutive steps are
  // one contiguous run, read through the scalar unit into SGPRs one group of
  // steps ahead (two alternating sets).  Steps past the end read rows of the
  // next batch row or the zero rows past the last token; their input term
  // is zero.
  const float* bcw = bcg + (static_cast<int64_t>(wave) * bcg_rows + row0) * 8;
  constexpr int kBcSteps = 2;              // steps per scalar load group
  float bc[2][kBcSteps * 8];
  auto load_bc = [&](int set, int64_t t) {
    const float* q = bcw + t * 8;
#pragma unroll
    for (int i = 0; i < kBcSteps * 8; ++i) bc[set][i] = q[i];
  };

  // x and z of the two steps this wavefront reduces, read with the tile's
  // inputs (the loader may overwrite that LDS buffer before the reduction)
  constexpr int kRs = kTile / kWaves;
  float xr[kRs] = {}, zr[kRs] = {};
  auto compute = [&](int64_t k, int buf) {
    float dv[kTile], uv[kTile];
#pragma unroll
    for (int s = 0; s < kTile; ++s) {
      dv[s] = s_del[buf][s][lane];
      uv[s] = s_u[buf][s][lane];
    }
#pragma unroll
    for (int j = 0; j < kRs; ++j) {
      if constexpr (kSkip) xr[j] = s_x[buf][wave * kRs + j][lane];
      if constexpr (kGate) zr[j] = s_z[buf][wave * kRs + j][lane];
    }
    float pt[kTile];
#pragma unroll
    for (int grp = 0; grp < kTile / kBcSteps; ++grp) {
      const int set = grp & 1;
      wait_scalar_loads();
      load_bc(set ^ 1, k * kTile + kBcSteps * (grp + 1));
      // Keep the next group's scalar loads here, a whole group ahead of
      // their use: left alone, the scheduler lifts this group's arithmetic
      // above the wait and the loads, and each group then starts by waiting
      // out the full latency of its own B and C.
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < kBcSteps; ++q) {
        const int s = kBcSteps * grp + q;
        const float* B = &bc[set][8 * q];
        float p = 0.0f;
#pragma unroll
        for (int i = 0; i < kSpw; ++i) {
          const float a = fast_exp2(dv[s] * a2[i]);
          h[i] = __builtin_fmaf(a, h[i], uv[s] * B[i]);
          p = __builtin_fmaf(B[4 + i], h[i], p);
        }
        pt[s] = p;
      }
    }
    // the partial read-outs leave after the last group, so the scalar-load
    // waits above (which count LDS accesses too) never wait for them
#pragma unroll
    for (int s = 0; s < kTile; ++s) s_part[buf][wave][s][lane] = pt[s];
  };

  // y of tile k (its partials in buffer buf): this wavefront's two steps
  auto reduce = [&](int64_t k, int buf) {
#pragma unroll
    for (int j = 0; j < kRs; ++j) {
      const int s = wave * kRs + j;
      const int64_t t = k * kTile + s;
      float v = s_part[buf][0][s][lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) v += s_part[buf][w][s][lane];
      if constexpr (kSkip) v = __builtin_fmaf(Dd, xr[j], v);
      if constexpr (kGate) v *= silu(zr[j]);
      if (t < L) {
        if constexpr (kPair) {
          const uint32_t hi = bf16_rne_bits(v);
          const int64_t o = (row0 + t) * ldy + d;
          yhi[o] = static_cast<uint16_t>(hi);
          ylo[o] = static_cast<uint16_t>(bf16_rne_bits(v - __uint_as_float(hi << 16)));
        } else {
          __builtin_nontemporal_store(v, &y[(row0 + t) * D + d]);
        }
      }
    }
  };

  // Pipeline, iteration k: barrier; reduce tile k - 1; tile k + 1 (loaded two
  // iterations earlier) into LDS; load tile k + 3; compute tile k.  Unrolled
  // by two so the register sets keep fixed names.
  Raw r0, r1;
  const int64_t last = ntiles - 1;
  load(r0, 0);
  load(r1, 1 < last ? 1 : last);
  put(r0, 0);
  load(r0, 2 < last ? 2 : last);
  load_bc(0, 0);
  int64_t k = 0;
  for (; k + 2 <= ntiles; k += 2) {
    block_sync();
    if (k >= 1) reduce(k - 1, 1);
    put(r1, 1);
    load(r1, k + 3 < last ? k + 3 : last);
    compute(k, 0);
    block_sync();
    reduce(k, 0);
    put(r0, 0);
    load(r0, k + 4 < last ? k + 4 : last);
    compute(k + 1, 1);
  }
  if (k < ntiles) {
    block_sync();
    if (k >= 1) reduce(k - 1, 1);
    compute(k, 0);
  }
  block_sync();
  reduce(last, static_cast<int>(last & 1));
}

template <typename TX, bool kSkip, bool kGate, bool kPair>
hipError_t launch_t(const ChainFusedArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.batch * (a.D / kCh)));
  const int64_t ldy = a.ld_y ? a.ld_y : a.D;
  hipLaunchKernelGGL((split_scan_kernel<TX, kSkip, kGate, kPair>), grid, dim3(kBlock), 0, stream,
                     static_cast<const TX*>(a.x), a.delta, a.bcg, xproj_bcg_rows(a.batch * a.L),
                     a.z, a.A, a.Dskip, static_cast<float*>(a.y), static_cast<uint16_t*>(a.y),
                     static_cast<uint16_t*>(a.y_lo), ldy, a.L, a.D);
  return hipGetLastError();
}

}  // namespace split

bool split_fused_applies(int64_t batch, int64_t D, int64_t N) {
  if (tuning(MSSM_TUNE_SCAN_ORDER) == MSSM_ORDER_CHUNKED) return false;
  return N == 16 && D % split::kCh == 0 && batch * D >= split::kMinChannels &&
         batch <= (int64_t(1) << 31) / (D / split::kCh);
}

hipError_t launch_split_fused(const ChainFusedArgs& a, hipStream_t stream) {
  if (!a.bcg) return hipErrorInvalidValue;   // needs the grouped B, C of launch_xproj
  if (!a.x_f32) {
    if (a.z || a.Dskip || a.y_bf16) return hipErrorInvalidValue;   // the fused SSM's form only
    return split::launch_t<uint16_t, false, false, false>(a, stream);
  }
  if (!a.z || !a.y_bf16 || !a.y_lo) return hipErrorInvalidValue;   // the block's form only
  if (a.Dskip) return split::launch_t<float, true, true, true>(a, stream);
  return split::launch_t<float, false, true, true>(a, stream);
}

}  // namespace mssm
