// Fused selective SSM for gfx950: selection projections + scan.
//
// The step size, input and output matrices are read off the tokens
// ("Understanding Mamba", section 5.1, eq. (6)): in the low-rank Mamba shape
// x_proj maps each token (D values) to [dt_low (R) | B_t (N) | C_t (N)], dt_proj
// maps dt_low back to D channels, a per-channel bias is added and softplus
// keeps the step size positive.  Here:
//
//   x_proj  : P = x @ W_x ([batch*L, D] x [D, R+2N], bf16 in, float32
//             accumulation) on the matrix cores (xproj.hip); its epilogue
//             stores dt_low as two bfloat16 parts, hi = bf16(dt_low) and
//             lo = bf16(dt_low - hi) (round to nearest even), so dt_proj's
//             matrix cores see dt_low to about 16 significant bits, and B, C
//             as float32 rows of P; W_dt is transposed to [D, R];
//   scan    : the same chunked two-pass scan as the plain path, except that
//             Delta never exists in memory: every 32-step tile of a wavefront's
//             channels is computed on the matrix cores (v_mfma_f32_32x32x16_bf16,
//             K = R in steps of 16, hi and lo parts accumulated into the same
//             float32 result), gets its bias and softplus on the vector
//             unit, and is parked in the wavefront's slice of LDS for the step
//             loop.  B_t and C_t are read as float32 rows of P (stride R + 2N)
//             through the scalar unit.
//
// The same scan kernels serve the Mamba block ("Understanding Mamba", section
// 8.1, eq. (9)): there x is the float32 output of the conv + SiLU prologue, the
// feedthrough D x and the SiLU(z) gate are applied per step, and the gated
// result is stored as bfloat16 for the output projection (FusedVariant).
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

// softplus(z) = ln(1 + e^z) as max(z, 0) + log1p(e), e = e^{-|z|} in (0, 1].
// u = 1 + e rounded, and c = e - (u - 1) is exactly (1 + e) - u (u - 1 is
// exact for u in [1, 2], Fast2Sum).  Then log1p(e) = log(u) + log(1 + c/u),
// and with |c| <= 2^-24 that is log(u) + c to within |c| e, a fraction of an
// ulp of the result: full relative accuracy down to the smallest e, with no
// division (v_log_f32 gives log2).
__device__ __forceinline__ float softplus_f(float z) {
  const float e = fast_exp2(-fabsf(z) * kLog2e);
  const float u = 1.0f + e;
  const float c = e - (u - 1.0f);
  return fmaxf(z, 0.0f) + __builtin_fmaf(__builtin_amdgcn_logf(u), 0.69314718055994531f, c);
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
  const int row = min(lane % 32, rows_valid - 1);
  const int khalf = 8 * (lane / 32);
  const uint16_t* arow = dtl + (int64_t)row * R + khalf;
  const uint16_t* arow_lo = dtl_lo + (int64_t)row * R + khalf;
  // one 32-column block at a time keeps a single 16-register accumulator live
#pragma unroll 1
  for (int nb = 0; nb < kBlocks; ++nb) {
    const int ch = min(nb * 32 + lane % 32, ch_valid - 1);
    const uint16_t* brow = wT + (int64_t)ch * R + khalf;
    f32x16 acc = f32x16{};
    for (int kk = 0; kk < R; kk += 16) {
      const bf16x8 a = load_bf16x8(arow + kk);
      const bf16x8 a_lo = load_bf16x8(arow_lo + kk);
      const bf16x8 b = load_bf16x8(brow + kk);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo, b, acc, 0, 0, 0);
    }
    const float bv = bias[ch];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // output element (row m, column n) of the 32x32 block held by this lane/register
      const int m = 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
      lds[m * stride + nb * 32 + lane % 32] = softplus_f(acc[r] + bv);
    }
  }
}

// What the fused scan reads and writes:
//   TX    : element type of x (bfloat16 bits or float32)
//   kSkip : y += Dskip[d] * x
//   kGate : y *= SiLU(z[b, t, d]), z float32 [batch, L, D]
//   TY    : element type of the stored y: float32, or bfloat16 bits, in which
//           case y is stored as a pair of arrays hi = bf16(y), lo = bf16(y - hi)
//           (round to nearest even; hi + lo keeps about 16 significant bits)
template <typename TX_, bool kSkip_, bool kGate_, typename TY_>
struct FusedVariant {
  using TX = TX_;
  using TY = TY_;
  static constexpr bool kSkip = kSkip_;
  static constexpr bool kGate = kGate_;
};
using FusedPlainVariant = FusedVariant<uint16_t, false, false, float>;

// The fused step loop: as scan_steps, with Delta from the LDS tile and B/C
// float32 rows of P (row stride ldbc floats).
template <int N, int CPL, bool kWithY, class FV>
__device__ __forceinline__ void fused_steps(const typename FV::TX* __restrict__ xb,
                                            const float* __restrict__ zb,
                                            const uint16_t* __restrict__ dtl,
                                            const uint16_t* __restrict__ dtl_lo,
                                            const uint16_t* __restrict__ wT,
                                            const float* __restrict__ bias, int R,
                                            const float* __restrict__ Bb, const float* __restrict__ Cb,
                                            int64_t ldbc, typename FV::TY* __restrict__ yb,
                                            typename FV::TY* __restrict__ ylo,
                                            const float (&A2)[CPL][N], const float (&Dd)[CPL],
                                            float (&h)[CPL][N], double (&S)[CPL], int wlane,
                                            int wave_ch0, int ch_valid, int64_t D, int nsteps,
                                            float* __restrict__ lds, int stride) {
  using TX = typename FV::TX;
  using TY = typename FV::TY;
  constexpr bool kGate = kWithY && FV::kGate;
  constexpr int kTile = (CPL == 1) ? 8 : 4;
  const uint32_t in_bytes = static_cast<uint32_t>((int64_t)nsteps * D * sizeof(TX));
  const buf_t xr = make_buf(xb, in_bytes);
  const int in_row = static_cast<int>(D * sizeof(TX));
  const int lane_blk = wave_ch0 + wlane * CPL;   // lane's first channel inside the block
  const int in_lane = lane_blk * static_cast<int>(sizeof(TX));
  buf_t zr;
  if constexpr (kGate) zr = make_buf(zb, static_cast<uint32_t>((int64_t)nsteps * D * sizeof(float)));
  const int z_row = static_cast<int>(D * sizeof(float));
  const int z_lane = lane_blk * static_cast<int>(sizeof(float));
  buf_t yr, ylr;
  int out_row = 0, out_lane = 0;
  if constexpr (kWithY) {
    yr = make_buf(yb, static_cast<uint32_t>((int64_t)nsteps * D * sizeof(TY)));
    if constexpr (sizeof(TY) == 2)
      ylr = make_buf(ylo, static_cast<uint32_t>((int64_t)nsteps * D * sizeof(TY)));
    out_row = static_cast<int>(D * sizeof(TY));
    out_lane = lane_blk * static_cast<int>(sizeof(TY));
  }
  const int last = nsteps > 0 ? nsteps - 1 : 0;
  float xc[kTile][CPL], zc[kGate ? kTile : 1][CPL];
#pragma unroll
  for (int j = 0; j < kTile; ++j) {
    const int r = min(j, last);
    buf_load_vals<TX, CPL>(xr, in_lane, __builtin_amdgcn_readfirstlane(r * in_row), xc[j]);
    if constexpr (kGate)
      buf_load_vals<float, CPL>(zr, z_lane, __builtin_amdgcn_readfirstlane(r * z_row), zc[j]);
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
    float xn[kTile][CPL], zn[kGate ? kTile : 1][CPL];
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      const int r = min(base + kTile + j, last);
      buf_load_vals<TX, CPL>(xr, in_lane, __builtin_amdgcn_readfirstlane(r * in_row), xn[j]);
      if constexpr (kGate)
        buf_load_vals<float, CPL>(zr, z_lane, __builtin_amdgcn_readfirstlane(r * z_row), zn[j]);
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
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            if constexpr (FV::kSkip) yv[c] = __builtin_fmaf(Dd[c], xc[j][c], yv[c]);
            if constexpr (kGate) yv[c] *= silu(zc[j][c]);
          }
          // lanes past the last channel repeat the last valid channel (clamped
          // addressing), so they store the same value to the same place
          if constexpr (sizeof(TY) == 2) {
            float hi[CPL], lo[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              hi[c] = __uint_as_float(bf16_rne_bits(yv[c]) << 16);
              lo[c] = yv[c] - hi[c];
            }
            buf_store_bf16<CPL>(yr, out_lane, s * out_row, hi);
            buf_store_bf16<CPL>(ylr, out_lane, s * out_row, lo);
          } else {
            buf_store_vals<CPL>(yr, out_lane, s * out_row, yv);
          }
        } else {
#pragma unroll
          for (int c = 0; c < CPL; ++c) S[c] += static_cast<double>(dt[c]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kTile; ++j)
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        xc[j][c] = xn[j][c];
        if constexpr (kGate) zc[j][c] = zn[j][c];
      }
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

template <int N, int CPL, typename TX>
__global__ __launch_bounds__(kFBlock) void fused_summary_kernel(
    const TX* __restrict__ x, const uint16_t* __restrict__ dtlow,
    const uint16_t* __restrict__ dtlow_lo,
    const uint16_t* __restrict__ wT, const float* __restrict__ bias,
    const float* __restrict__ A, const float* __restrict__ P, float* __restrict__ sum_h,
    double* __restrict__ sum_s, int64_t L, int64_t D, int R, int64_t chunk_len, int K,
    int64_t n_dtiles) {
  using FV = FusedVariant<TX, false, false, float>;
  __shared__ float lds_all[4][kDTile * lds_stride<CPL>()];
  const FusedCoord c = fused_coord<CPL>(n_dtiles, K - 1, D);
  if (c.d0 + c.wave_ch0 >= D) return;   // wavefront past the last channel (no barriers here)
  float* lds = lds_all[threadIdx.x / 64];
  const int64_t wave_d = c.d0 + c.wave_ch0;
  const int64_t dl = wave_d + (int64_t)c.wlane * CPL;
  float A2[CPL][N], h[CPL][N], Dd[CPL];
  double S[CPL];
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    S[q] = 0.0;
    Dd[q] = 0.0f;
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
  fused_steps<N, CPL, false, FV>(x + tok0 * D + c.d0, nullptr, dtlow + tok0 * R,
                                 dtlow_lo + tok0 * R, wT + wave_d * R, bias + wave_d, R,
                                 P + tok0 * ldbc + R, nullptr, ldbc, nullptr, nullptr, A2, Dd, h, S,
                                 c.wlane, c.wave_ch0, c.ch_valid, D, nsteps, lds,
                                 lds_stride<CPL>());
  if (c.active) {
    const int64_t row = c.b * (K - 1) + c.k;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
#pragma unroll
      for (int n = 0; n < N; ++n) sum_h[(row * N + n) * D + dl + q] = h[q][n];
      sum_s[row * D + dl + q] = S[q];
    }
  }
}

template <int N, int CPL, class FV>
__global__ __launch_bounds__(kFBlock) void fused_output_kernel(
    const typename FV::TX* __restrict__ x, const float* __restrict__ z,
    const float* __restrict__ Dskip, const uint16_t* __restrict__ dtlow,
    const uint16_t* __restrict__ dtlow_lo,
    const uint16_t* __restrict__ wT, const float* __restrict__ bias,
    const float* __restrict__ A, const float* __restrict__ P, const float* __restrict__ sum_h,
    typename FV::TY* __restrict__ y, typename FV::TY* __restrict__ y_lo, int64_t L, int64_t D,
    int R, int64_t chunk_len, int K, int64_t n_dtiles) {
  __shared__ float lds_all[4][kDTile * lds_stride<CPL>()];
  const FusedCoord c = fused_coord<CPL>(n_dtiles, K, D);
  if (c.d0 + c.wave_ch0 >= D) return;   // wavefront past the last channel (no barriers here)
  float* lds = lds_all[threadIdx.x / 64];
  const int64_t wave_d = c.d0 + c.wave_ch0;
  const int64_t dl = wave_d + (int64_t)c.wlane * CPL;
  float A2[CPL][N], h[CPL][N], Dd[CPL];
  double S_unused[CPL];
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    S_unused[q] = 0.0;
    Dd[q] = FV::kSkip ? Dskip[dl + q] : 0.0f;
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
  fused_steps<N, CPL, true, FV>(x + tok0 * D + c.d0, FV::kGate ? z + tok0 * D + c.d0 : nullptr,
                                dtlow + tok0 * R, dtlow_lo + tok0 * R, wT + wave_d * R,
                                bias + wave_d, R, P + tok0 * ldbc + R, P + tok0 * ldbc + R + N,
                                ldbc, y + tok0 * D + c.d0,
                                sizeof(typename FV::TY) == 2 ? y_lo + tok0 * D + c.d0 : nullptr,
                                A2, Dd, h, S_unused, c.wlane,
                                c.wave_ch0, c.ch_valid, D, nsteps, lds, lds_stride<CPL>());
}

// Delta[m, d] = softplus(sum_r (hi[m, r] + lo[m, r]) wT[d, r] + bias[d]) for the
// whole [M, D] matrix, float32: the step sizes of "Understanding Mamba",
// section 5.1 eq. (6) written out once for the single-pass scan.  Same
// arithmetic as delta_tile (v_mfma_f32_32x32x16_bf16, hi and lo parts
// accumulated into one float32 result, bias, softplus).  KS = R / 16 K steps.
// A block is 4 wavefronts over 128 channels (32 each) and kDtRowTiles tiles of
// 32 rows.  Each wavefront keeps its channels' W_dt^T operands in registers;
// each row tile's dt_low rows (one contiguous stretch of memory per part) are
// copied into LDS with 16-byte loads shared by the four wavefronts, the next
// tile's loads in flight while the current one computes.  Rows >= M and
// channels >= D read clamped operands and store nothing.
constexpr int kDtRowTiles = 8;               // 32-row tiles per block

template <int KS>
__global__ __launch_bounds__(kFBlock) __attribute__((amdgpu_waves_per_eu(3))) void dtproj_softplus_kernel(
    const uint16_t* __restrict__ dtl, const uint16_t* __restrict__ dtl_lo,
    const uint16_t* __restrict__ wT, const float* __restrict__ bias, float* __restrict__ delta,
    int64_t M, int64_t D, int64_t n_cblocks) {
  constexpr int R = 16 * KS;
  constexpr int kStride = R + 8;                    // LDS row stride (bf16): 16-byte rows, skewed banks
  constexpr int kRowChunks = R / 8;                 // 16-byte pieces per row
  constexpr int kChunks = 2 * 32 * kRowChunks;      // both parts of a 32-row tile
  constexpr int kPerThread = (kChunks + kFBlock - 1) / kFBlock;
  __shared__ __align__(16) uint16_t sa[2][32][kStride];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t rb = blockIdx.x / n_cblocks;
  const int64_t c0 = (blockIdx.x % n_cblocks) * 128 + wave * 32;
  const int khalf = 8 * (lane / 32);
  const int64_t ch = min(c0 + lane % 32, D - 1);
  bf16x8 bw[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) bw[k] = load_bf16x8(wT + ch * R + 16 * k + khalf);
  const float bias_c = bias[ch];
  const bool col_ok = c0 + lane % 32 < D;
  const uint32_t lane_off = static_cast<uint32_t>((4 * (lane / 32) * D + lane % 32) * 4);   // bytes

  // this thread's pieces of every tile: part, row, column (compile-time divisors)
  auto piece = [&](int q, int& arr, int& row, int& col) {
    const int c = threadIdx.x + kFBlock * q;
    arr = c / (32 * kRowChunks);
    row = (c % (32 * kRowChunks)) / kRowChunks;
    col = (c % kRowChunks) * 8;
  };
  u32x4 pre[kPerThread];
  auto fetch = [&](int64_t m0) {
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
      int arr, row, col;
      piece(q, arr, row, col);
      if (threadIdx.x + kFBlock * q < kChunks) {
        const int64_t m = min(m0 + row, M - 1);
        pre[q] = *reinterpret_cast<const u32x4*>((arr ? dtl_lo : dtl) + m * R + col);
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
      int arr, row, col;
      piece(q, arr, row, col);
      if (threadIdx.x + kFBlock * q < kChunks)
        *reinterpret_cast<u32x4*>(&sa[arr][row][col]) = pre[q];
    }
  };

  const int64_t first = rb * kDtRowTiles * 32;
  fetch(first);
  for (int t = 0; t < kDtRowTiles; ++t) {
    const int64_t m0 = first + 32 * t;
    if (m0 >= M) break;                        // uniform over the block
    block_sync();                           // the previous tile's LDS reads are done
    stash();
    block_sync();
    if (t + 1 < kDtRowTiles && m0 + 32 < M) fetch(m0 + 32);   // in flight during this tile
    if (c0 >= D) continue;                     // a wavefront past the last channel only copies
    f32x16 acc;                                // the bias enters as the accumulator's start
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = bias_c;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      bf16x8 a, a_lo;
      __builtin_memcpy(&a, &sa[0][lane % 32][16 * k + khalf], sizeof(a));
      __builtin_memcpy(&a_lo, &sa[1][lane % 32][16 * k + khalf], sizeof(a_lo));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bw[k], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo, bw[k], acc, 0, 0, 0);
    }
    // output element (row m0 + 8 (r / 4) + 4 (lane / 32) + r % 4, column c0 +
    // lane % 32): a wave-uniform row base per r and a small per-lane offset
    if (m0 + 32 <= M && c0 + 32 <= D) {        // uniform: every element in range
      // rows as SGPR offsets from the tile's corner, the lane's place as the
      // per-lane offset: no per-store vector address arithmetic
      const buf_t out = make_buf(delta + m0 * D + c0, 0x7fffffffu);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int soff = static_cast<int>((8 * (r / 4) + (r % 4)) * D * 4);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(softplus_f(acc[r])), out,
                                              static_cast<int>(lane_off), soff, kStoreNT);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
        if (col_ok && m < M) delta[m * D + c0 + lane % 32] = softplus_f(acc[r]);
      }
    }
  }
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// one rocBLAS handle per device, created on first use and kept until exit
std::mutex g_blas_mutex;
rocblas_handle g_blas[64] = {};

template <int N, int CPL, class FV>
hipError_t launch_fused_scan_t(const FusedScanArgs& a, const ScanPlan& p, hipStream_t stream) {
  using TX = typename FV::TX;
  using TY = typename FV::TY;
  const TX* x = static_cast<const TX*>(a.x);
  TY* y = static_cast<TY*>(a.y);
  const int64_t n_dtiles = (a.D + kFBlock * CPL - 1) / (kFBlock * CPL);
  const int R = static_cast<int>(a.R);
  if (p.K > 1) {
    const int64_t grid = n_dtiles * (p.K - 1) * a.batch;
    hipLaunchKernelGGL((fused_summary_kernel<N, CPL, TX>), dim3((unsigned)grid), dim3(kFBlock), 0,
                       stream, x, a.dtl, a.dtl_lo, a.wT, a.dt_bias, a.A, a.P, a.sum_h, a.sum_s,
                       a.L, a.D, R, p.chunk_len, p.K, n_dtiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_carry(a.sum_h, a.sum_s, a.A, nullptr, a.batch, a.D, a.N, p.K, stream);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = n_dtiles * p.K * a.batch;
  hipLaunchKernelGGL((fused_output_kernel<N, CPL, FV>), dim3((unsigned)grid), dim3(kFBlock), 0,
                     stream, x, a.z, a.Dskip, a.dtl, a.dtl_lo, a.wT, a.dt_bias, a.A, a.P, a.sum_h,
                     y, static_cast<TY*>(a.y_lo), a.L, a.D, R, p.chunk_len, p.K, n_dtiles);
  return hipGetLastError();
}

template <int N, class FV>
hipError_t launch_fused_scan_n(const FusedScanArgs& a, const ScanPlan& p, hipStream_t stream) {
  return p.cpl == 2 ? launch_fused_scan_t<N, 2, FV>(a, p, stream)
                    : launch_fused_scan_t<N, 1, FV>(a, p, stream);
}

template <class FV>
hipError_t launch_fused_scan_v(const FusedScanArgs& a, const ScanPlan& p, hipStream_t stream) {
  switch (a.N) {
    case 1: return launch_fused_scan_n<1, FV>(a, p, stream);
    case 2: return launch_fused_scan_n<2, FV>(a, p, stream);
    case 4: return launch_fused_scan_n<4, FV>(a, p, stream);
    case 8: return launch_fused_scan_n<8, FV>(a, p, stream);
    case 16: return launch_fused_scan_n<16, FV>(a, p, stream);
    case 32: return launch_fused_scan_n<32, FV>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

BlasLease::BlasLease(hipStream_t stream) : lock_(g_blas_mutex) {
  int dev = 0;
  hip_ = hipGetDevice(&dev);
  if (hip_ != hipSuccess) return;
  if (dev < 0 || dev >= 64) {
    hip_ = hipErrorInvalidDevice;
    return;
  }
  if (!g_blas[dev]) {
    if (rocblas_create_handle(&g_blas[dev]) != rocblas_status_success) {
      g_blas[dev] = nullptr;
      return;
    }
  }
  if (rocblas_set_stream(g_blas[dev], stream) != rocblas_status_success) return;
  handle_ = g_blas[dev];
  ok_ = true;
}

bool gemm_rm_bf16_bt(rocblas_handle h, int64_t M, int64_t n, int64_t k, const void* A,
                     int64_t lda, const void* BT, int64_t ldbt, float* C, int64_t ldc,
                     float beta) {
  // column-major C^T (n x M) = (BT stored k x n, transposed) (A^T, k x M)
  const float alpha = 1.0f;
  return rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, (rocblas_int)n,
                         (rocblas_int)M, (rocblas_int)k, &alpha, BT, rocblas_datatype_bf16_r,
                         (rocblas_int)ldbt, A, rocblas_datatype_bf16_r, (rocblas_int)lda, &beta,
                         C, rocblas_datatype_f32_r, (rocblas_int)ldc, C, rocblas_datatype_f32_r,
                         (rocblas_int)ldc, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0,
                         0) == rocblas_status_success;
}

namespace {

// One 64 x 64 tile per block.  With vec (both dimensions multiples of 8 and
// W 16-byte aligned) a thread moves 8 halves (16 bytes) per global access: it reads two 8-wide
// pieces of W's rows, and writes two 8-wide pieces of wT's rows gathered from
// a tile column in LDS (row pitch 72 halves keeps the 16-byte stores aligned
// and spreads the column reads over the banks).  Other shapes go one half at
// a time.
__global__ __launch_bounds__(256) void transpose_tiles_bf16_kernel(
    const uint16_t* __restrict__ W, uint16_t* __restrict__ wT, int64_t rows, int64_t cols,
    int64_t ldt, bool vec) {
  __shared__ __align__(16) uint16_t tile[64][72];
  const int64_t tiles_c = (cols + 63) / 64;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x / tiles_c) * 64;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x % tiles_c) * 64;
  const int t = threadIdx.x;
  if (vec) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int piece = t + 256 * h;              // 64 rows x 8 pieces
      const int i = piece >> 3, j = (piece & 7) * 8;
      const int64_t r = r0 + i, c = c0 + j;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (r < rows && c < cols) v = *reinterpret_cast<const uint4*>(W + r * cols + c);
      *reinterpret_cast<uint4*>(&tile[i][j]) = v;
    }
    block_sync();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int piece = t + 256 * h;              // 64 output rows (tile columns) x 8 pieces
      const int i = piece >> 3, j = (piece & 7) * 8;
      const int64_t c = c0 + i, r = r0 + j;
      if (c < cols && r < rows) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = static_cast<uint32_t>(tile[j + 2 * q][i]) |
                 (static_cast<uint32_t>(tile[j + 2 * q + 1][i]) << 16);
        *reinterpret_cast<uint4*>(wT + c * ldt + r) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    return;
  }
  const int tx = t & 63, ty = t >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < rows && c < cols) ? W[r * cols + c] : uint16_t(0);
  }
  block_sync();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) wT[c * ldt + r] = tile[tx][i];
  }
}

}  // namespace

hipError_t launch_transpose_bf16(const void* W, uint16_t* wT, int64_t rows, int64_t cols,
                                 hipStream_t stream, int64_t ldt) {
  const int64_t tiles = ((rows + 63) / 64) * ((cols + 63) / 64);
  if (tiles <= 0) return hipSuccess;
  if (ldt == 0) ldt = rows;
  if (ldt < rows) return hipErrorInvalidValue;
  // wT is workspace; W is the caller's
  const bool vec = rows % 8 == 0 && cols % 8 == 0 && ldt % 8 == 0 &&
                   reinterpret_cast<uintptr_t>(W) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(wT) % 16 == 0;
  hipLaunchKernelGGL(transpose_tiles_bf16_kernel, dim3(static_cast<unsigned>(tiles)), dim3(256), 0,
                     stream, static_cast<const uint16_t*>(W), wT, rows, cols, ldt, vec);
  return hipGetLastError();
}

hipError_t launch_wdt_transpose(const void* W_dt, int64_t R, int64_t D, uint16_t* wT,
                                hipStream_t stream) {
  return launch_transpose_bf16(W_dt, wT, R, D, stream, R);   // wT[d, r] = W_dt[r, d]
}

hipError_t launch_dtproj_softplus(const uint16_t* dtl, const uint16_t* dtl_lo, const uint16_t* wT,
                                  const float* bias, float* delta, int64_t M, int64_t D,
                                  int64_t R, hipStream_t stream) {
  const int64_t n_cblocks = (D + 127) / 128;
  const dim3 grid(static_cast<unsigned>((M + 32 * kDtRowTiles - 1) / (32 * kDtRowTiles) *
                                        n_cblocks));
#define MSSM_DTPROJ_CASE(KS)                                                                    \
  case KS:                                                                                     \
    hipLaunchKernelGGL((dtproj_softplus_kernel<KS>), grid, dim3(kFBlock), 0, stream, dtl,      \
                       dtl_lo, wT, bias, delta, M, D, n_cblocks);                              \
    break;
  switch (R / 16) {
    MSSM_DTPROJ_CASE(1) MSSM_DTPROJ_CASE(2) MSSM_DTPROJ_CASE(3) MSSM_DTPROJ_CASE(4)
    MSSM_DTPROJ_CASE(5) MSSM_DTPROJ_CASE(6) MSSM_DTPROJ_CASE(7) MSSM_DTPROJ_CASE(8)
    MSSM_DTPROJ_CASE(9) MSSM_DTPROJ_CASE(10) MSSM_DTPROJ_CASE(11) MSSM_DTPROJ_CASE(12)
    MSSM_DTPROJ_CASE(13) MSSM_DTPROJ_CASE(14) MSSM_DTPROJ_CASE(15) MSSM_DTPROJ_CASE(16)
    default: return hipErrorInvalidValue;     // R a multiple of 16 up to 256
  }
#undef MSSM_DTPROJ_CASE
  return hipGetLastError();
}

hipError_t launch_fused_scan(const FusedScanArgs& a, const ScanPlan& p, hipStream_t stream) {
  if (!a.x_f32) {
    if (a.z || a.Dskip || a.y_bf16) return hipErrorInvalidValue;
    return launch_fused_scan_v<FusedPlainVariant>(a, p, stream);
  }
  if (!a.z || !a.y_bf16 || !a.y_lo) return hipErrorInvalidValue;   // the block's form only
  if (a.Dskip) return launch_fused_scan_v<FusedVariant<float, true, true, uint16_t>>(a, p, stream);
  return launch_fused_scan_v<FusedVariant<float, false, true, uint16_t>>(a, p, stream);
}

FusedPlan plan_fused(int64_t batch, int64_t L, int64_t D, int64_t N, int64_t R, int cpl,
                     bool chain) {
  FusedPlan f;
  const int64_t M = batch * L;
  if (chain) {
    f.chain = true;
    f.scan.chain = true;
  } else {
    f.scan = plan_scan(batch, L, D, N, cpl);
  }
  f.p_bytes = align256(sizeof(float) * (size_t)M * (size_t)(R + 2 * N));
  f.dtl_offset = f.p_bytes;
  f.dtl_lo_offset = f.dtl_offset + align256(sizeof(uint16_t) * (size_t)M * (size_t)R);
  f.wt_offset = f.dtl_lo_offset + align256(sizeof(uint16_t) * (size_t)M * (size_t)R);
  f.wx_t_offset = f.wt_offset + align256(sizeof(uint16_t) * (size_t)D * (size_t)R);
  f.scan_offset = f.wx_t_offset +
                  align256(sizeof(uint16_t) * (size_t)(R + 2 * N) * (size_t)xproj_padded_k(D));
  if (chain) {
    f.delta_offset = f.scan_offset;
    f.workspace_bytes = f.delta_offset + align256(sizeof(float) * (size_t)M * (size_t)D);
    if (split_fused_applies(batch, D, N)) {
      f.bcg_offset = f.workspace_bytes;
      f.workspace_bytes += align256(sizeof(float) * 4 * 8 * (size_t)xproj_bcg_rows(M));
    }
  } else {
    f.workspace_bytes = f.scan_offset + f.scan.workspace_bytes;
  }
  return f;
}

size_t fused_workspace_bound(int64_t batch, int64_t L, int64_t D, int64_t N, int64_t R) {
  size_t w = plan_fused(batch, L, D, N, R, 1, false).workspace_bytes;
  if (D % 2 == 0) w = std::max(w, plan_fused(batch, L, D, N, R, 2, false).workspace_bytes);
  if (N == 16 && D % 16 == 0 && R <= 256)
    w = std::max(w, plan_fused(batch, L, D, N, R, 1, true).workspace_bytes);
  return w;
}

// One chain per lane: the Delta tile's matrix-core accumulators and operands
// already take many registers, and two chains per lane leave one wavefront
// per SIMD (218 VGPRs + 64 AGPRs); one chain keeps three, which measured 35%
// faster on MI355X for the fused workload (1.91 vs 2.94 ms).  The
// chains-per-lane setting 2 selects the other layout for tuning runs.
int choose_fused_cpl(int64_t D) {
  if (tuning(MSSM_TUNE_CHAINS_PER_LANE) == 2 && D % 2 == 0) return 2;   // tuning runs only
  return 1;
}

FusedStatus launch_fused(const FusedArgs& a, const FusedPlan& f, void* workspace,
                         hipStream_t stream) {
  FusedStatus st;
  char* ws = static_cast<char*>(workspace);
  float* P = reinterpret_cast<float*>(ws);
  const int64_t M = a.batch * a.L;
  const int64_t ldp = a.R + 2 * a.N;
  uint16_t* dtl = reinterpret_cast<uint16_t*>(ws + f.dtl_offset);
  uint16_t* dtl_lo = reinterpret_cast<uint16_t*>(ws + f.dtl_lo_offset);
  uint16_t* wT = reinterpret_cast<uint16_t*>(ws + f.wt_offset);
  // x_proj: dt_low (as its bf16 hi + lo pair) and the B, C columns of P (and
  // for the split-state scan B, C grouped by four state indices)
  uint16_t* WxT = reinterpret_cast<uint16_t*>(ws + f.wx_t_offset);
  float* bcg = (f.chain && split_fused_applies(a.batch, a.D, a.N))
                   ? reinterpret_cast<float*>(ws + f.bcg_offset)
                   : nullptr;
  st.hip = launch_xproj(static_cast<const uint16_t*>(a.x), nullptr, a.D, M, a.D, a.W_x, ldp,
                        a.R, WxT, dtl, dtl_lo, P, ldp, bcg, stream);
  if (st.hip != hipSuccess) return st;
  st.hip = launch_wdt_transpose(a.W_dt, a.R, a.D, wT, stream);
  if (st.hip != hipSuccess) return st;
  if (f.chain) {
    float* delta = reinterpret_cast<float*>(ws + f.delta_offset);
    st.hip = launch_dtproj_softplus(dtl, dtl_lo, wT, a.dt_bias, delta, M, a.D, a.R, stream);
    if (st.hip != hipSuccess) return st;
    ChainFusedArgs ca;
    ca.x = a.x;
    ca.delta = delta;
    ca.P = P;
    ca.ldp = ldp;
    ca.R = a.R;
    ca.A = a.A;
    ca.y = a.y;
    ca.batch = a.batch;
    ca.L = a.L;
    ca.D = a.D;
    ca.bcg = bcg;
    st.hip = launch_chain_fused(ca, stream);
    return st;
  }
  FusedScanArgs sa{};
  sa.x = a.x;
  sa.y = a.y;
  sa.P = P;
  sa.dtl = dtl;
  sa.dtl_lo = dtl_lo;
  sa.wT = wT;
  sa.dt_bias = a.dt_bias;
  sa.A = a.A;
  if (f.scan.K > 1) {
    sa.sum_h = reinterpret_cast<float*>(ws + f.scan_offset);
    sa.sum_s = reinterpret_cast<double*>(ws + f.scan_offset + f.scan.sum_s_offset);
  }
  sa.batch = a.batch;
  sa.L = a.L;
  sa.D = a.D;
  sa.N = a.N;
  sa.R = a.R;
  st.hip = launch_fused_scan(sa, f.scan, stream);
  return st;
}

}  // namespace mssm
