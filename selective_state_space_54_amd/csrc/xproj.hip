// The selection projection x_proj on the matrix cores (gfx950), one pass
// over x.
//
// Each token x_t (K = D values) is projected to [dt_low (R) | B_t (N) | C_t
// (N)] = x_t W_x ("Understanding Mamba", section 5.1, eq. (6), in the low-rank
// Mamba shape).  With batch * L = M tokens that is P[M, R + 2N] = x[M, K]
// W_x[K, R + 2N]: a tall, thin GEMM whose cost is reading x once (335 MB for
// the fused workload against 2 MB of weights), so the kernel is laid out for
// streaming x:
//
//   * a block owns 128 rows of x and all (up to 192) output columns, so every
//     element of x is read from memory exactly once (one block per compute
//     unit on the fused workload);
//   * 64-value slices along k of the block's x rows and of W^T (W_x
//     transposed, zero-padded along k to a multiple of 64, so the k tail needs
//     no test) are staged in LDS with 16-byte loads; the loads run two slices
//     ahead through two register sets, about 80 KB in flight per compute
//     unit, which is what streaming x near HBM speed needs; two LDS buffers,
//     one barrier per slice;
//   * the four wavefronts split the 128 x 192 tile 2 x 2: each owns 64 rows x
//     96 columns, 4 x 6 accumulator tiles of v_mfma_f32_16x16x32_bf16 with
//     float32 accumulation, reading its A and B fragments from LDS (each B
//     fragment serves four row tiles, each A fragment six column tiles);
//   * epilogue: columns below R (dt_low) are stored as the bf16 pair
//     hi = bf16(v), lo = bf16(v - hi) that dt_proj's matrix cores read (R is a
//     multiple of 16, so a 16-column fragment is all dt_low or all B/C); the
//     B and C columns are stored as float32 into P's rows (for N = 16 also,
//     on request, in four groups of four state indices: [4][M + 8][B 4 | C 4],
//     so that a wavefront owning four state indices finds consecutive steps'
//     B and C side by side, the layout the split-state scan reads).
//
// With two A operands (the Mamba block: x kept as a bf16 hi + lo pair) both
// tiles are multiplied into the same accumulators.
//
// For 16-byte aligned rows, K a multiple of 64 and 192 output columns (the
// fused selective SSM and the Mamba block with R = 160, N = 16; one A operand
// or the hi + lo pair) a second form takes over: the tiles are copied from
// memory straight into LDS (no register staging), x five stages deep and W^T
// three, with the pieces of a row permuted so that the fragment reads stay
// conflict-free (xproj_lds_kernel below).
//
// MFMA operand layout (v_mfma_f32_16x16x32_bf16): A fragment, lane l holds row
// l % 16 and 8 consecutive k values starting at 8 (l / 16); B fragment, lane l
// holds column l % 16 and the same 8 k values; both operands use the same k
// assignment, so the products pair up whatever order the hardware sums them
// in.  Result: lane l holds rows 4 (l / 16) + i, i = 0..3, of column l % 16.
#include <type_traits>

#include "mssm_internal.h"
#include "scan_device.h"

namespace mssm {

namespace {

constexpr int kXBlock = 256;          // 4 wavefronts: 2 x 2 over (rows, columns)
constexpr int kXRows = 128;           // rows of x per block
constexpr int kXK = 64;               // k values per LDS tile
constexpr int kXPitch = kXK + 8;      // LDS row pitch (bf16): 144 bytes, conflict-free 16-byte reads
constexpr int kXColsPerWave = 96;     // six 16-column fragments
constexpr int kXFrags = kXColsPerWave / 16;
constexpr int kXCols = 2 * kXColsPerWave;   // output columns per block

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  bf16x8 v;
  __builtin_memcpy(&v, &u, sizeof(v));
  return v;
}

// W^T[c, r] = W[r, c] for r < K, 0 for K <= r < Kp; W is [K, ncol] row-major,
// W^T [ncol, Kp].
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint16_t* __restrict__ W,
                                                            uint16_t* __restrict__ wT, int64_t K,
                                                            int64_t ncol, int64_t Kp,
                                                            float* __restrict__ bcg,
                                                            int64_t bcg_rows, int64_t M, bool vec) {
  // the grouped B/C rows past the last token (read by steps past the end of
  // the sequence, whose input term is zero) are set to zero here
  if (bcg && blockIdx.x == 0) {
    const int g = threadIdx.x >> 6, r = (threadIdx.x >> 3) & 7, j = threadIdx.x & 7;
    if (M + r < bcg_rows) bcg[(g * bcg_rows + M + r) * 8 + j] = 0.0f;
  }
  __shared__ __align__(16) uint16_t tile[64][72];
  const int64_t tiles_c = (ncol + 63) / 64;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x / tiles_c) * 64;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x % tiles_c) * 64;
  const int t = threadIdx.x;
  if (vec) {
    // 16-byte pieces: two 8-wide pieces of W's rows per thread in, two
    // 8-wide pieces of wT's rows (gathered from a tile column) out; the
    // 72-half pitch keeps the pieces aligned and the column reads spread
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int piece = t + 256 * h;
      const int i = piece >> 3, j = (piece & 7) * 8;
      const int64_t r = r0 + i, c = c0 + j;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (r < K && c < ncol) v = *reinterpret_cast<const uint4*>(W + r * ncol + c);
      *reinterpret_cast<uint4*>(&tile[i][j]) = v;
    }
    block_sync();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int piece = t + 256 * h;
      const int i = piece >> 3, j = (piece & 7) * 8;
      const int64_t c = c0 + i, r = r0 + j;
      if (c < ncol && r < Kp) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = static_cast<uint32_t>(tile[j + 2 * q][i]) |
                 (static_cast<uint32_t>(tile[j + 2 * q + 1][i]) << 16);
        *reinterpret_cast<uint4*>(wT + c * Kp + r) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    return;
  }
  const int tx = t & 63, ty = t >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < K && c < ncol) ? W[r * ncol + c] : uint16_t(0);
  }
  block_sync();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < ncol && r < Kp) wT[c * Kp + r] = tile[tx][i];
  }
}

// One 16-byte piece (8 bf16) of row m of an A operand at k0.  kVec: the row
// stride and base allow a 16-byte load, and K is a multiple of 8, so a piece
// is wholly inside or wholly past K.  Otherwise element loads, each tested.
template <bool kVec>
__device__ __forceinline__ uint4 load_piece(const uint16_t* __restrict__ A, int64_t lda,
                                            int64_t m, int64_t k0, int64_t K) {
  const uint16_t* p = A + m * lda + k0;
  if constexpr (kVec) {
    if (k0 >= K) return make_uint4(0u, 0u, 0u, 0u);
    return *reinterpret_cast<const uint4*>(p);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = k0 + 2 * j < K ? p[2 * j] : 0u;
      const uint32_t hi = k0 + 2 * j + 1 < K ? p[2 * j + 1] : 0u;
      w[j] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// This wavefront's part of the block's result (kRT 16-row tiles from row
// 16 kRT wr, columns c_wave): columns below R as the dt_low bf16 pair, the
// others as float32 into P and, with bcg, into the grouped B/C copy.
template <int kRT = 4>
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[4][kXFrags], int lane, int wr,
                                           int64_t m0, int c_wave, int nfrag, int64_t M,
                                           int ncol, int R, uint16_t* __restrict__ dtl,
                                           uint16_t* __restrict__ dtl_lo, float* __restrict__ P,
                                           int64_t ldp, float* __restrict__ bcg,
                                           int64_t bcg_rows) {
  const int col_in = lane & 15;
  const int row_in = 4 * (lane >> 4);
#pragma unroll
  for (int f = 0; f < kXFrags; ++f) {
    if (f >= nfrag) continue;
    const int c = c_wave + 16 * f + col_in;
    const bool dt_frag = c_wave + 16 * f < R;       // uniform: R is a multiple of 16
#pragma unroll
    for (int r = 0; r < kRT; ++r) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + 16 * kRT * wr + 16 * r + row_in + i;
        if (m >= M) continue;
        const float v = acc[r][f][i];
        if (dt_frag) {
          const uint32_t hi = bf16_rne_bits(v);
          dtl[m * R + c] = static_cast<uint16_t>(hi);
          dtl_lo[m * R + c] = static_cast<uint16_t>(bf16_rne_bits(v - __uint_as_float(hi << 16)));
        } else if (c < ncol) {
          P[m * ldp + c] = v;
          if (bcg) {   // N = 16: B and C also in four groups of four state indices
            const int n = c - R;
            const int g = (n & 15) >> 2, j = (n & 3) + (n >= 16 ? 4 : 0);
            bcg[(g * bcg_rows + m) * 8 + j] = v;
          }
        }
      }
    }
  }
}

// grid: (ceil(M / 128), ceil(ncol / 192)).  A0 (and A1 with kTwo) [M, K]
// bf16 with row stride lda; wT [ncol, Kp] bf16, Kp a multiple of 64, zero for
// k >= K.  Outputs: columns c < R to dtl / dtl_lo [M, R] (bf16 pair), columns
// R <= c < ncol to P[m * ldp + c] (float32) and, with bcg, to the grouped copy.
template <bool kTwo, bool kVec>
__global__ __launch_bounds__(kXBlock) void xproj_kernel(
    const uint16_t* __restrict__ A0, const uint16_t* __restrict__ A1, int64_t lda,
    const uint16_t* __restrict__ wT, int64_t Kp, int64_t K, int64_t M, int ncol, int R,
    uint16_t* __restrict__ dtl, uint16_t* __restrict__ dtl_lo, float* __restrict__ P,
    int64_t ldp, float* __restrict__ bcg, int64_t bcg_rows) {
  constexpr int kOps = kTwo ? 2 : 1;
  constexpr int kXPieces = kXRows * kXK / 8 / kXBlock;   // 16-byte x pieces per thread per tile
  constexpr int kWPieces = kXCols * kXK / 8 / kXBlock;   // 16-byte W pieces per thread per tile
  __shared__ __align__(16) uint16_t sa[2][kOps][kXRows][kXPitch];
  __shared__ __align__(16) uint16_t sb[2][kXCols][kXPitch];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave >> 1, wc = wave & 1;               // 64-row half, 96-column half
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * kXRows;
  const int c0 = static_cast<int>(blockIdx.y) * kXCols;
  const int c_wave = c0 + wc * kXColsPerWave;
  // 16-column fragments of this wavefront holding any column < ncol (uniform)
  int nfrag = (ncol - c_wave + 15) / 16;
  nfrag = nfrag < 0 ? 0 : (nfrag > kXFrags ? kXFrags : nfrag);

  struct Stage {
    uint4 x[kOps][kXPieces];
    uint4 w[kWPieces];
  };
  // piece q of this thread: tile row (q * 256 + tid) / 8, 8 k values at ((q * 256 + tid) % 8) * 8
  auto fetch = [&](Stage& st, int64_t t) {
    const int64_t k0 = t * kXK;
#pragma unroll
    for (int o = 0; o < kOps; ++o) {
      const uint16_t* A = o == 0 ? A0 : A1;
#pragma unroll
      for (int q = 0; q < kXPieces; ++q) {
        const int p = threadIdx.x + kXBlock * q;
        const int64_t m = min(m0 + (p >> 3), M - 1);
        st.x[o][q] = load_piece<kVec>(A, lda, m, k0 + (p & 7) * 8, K);
      }
    }
#pragma unroll
    for (int q = 0; q < kWPieces; ++q) {
      const int p = threadIdx.x + kXBlock * q;
      const int c = min(c0 + (p >> 3), ncol - 1);
      st.w[q] = *reinterpret_cast<const uint4*>(wT + static_cast<int64_t>(c) * Kp + k0 +
                                                (p & 7) * 8);
    }
  };
  auto stash = [&](const Stage& st, int buf) {
#pragma unroll
    for (int o = 0; o < kOps; ++o)
#pragma unroll
      for (int q = 0; q < kXPieces; ++q) {
        const int p = threadIdx.x + kXBlock * q;
        *reinterpret_cast<uint4*>(&sa[buf][o][p >> 3][(p & 7) * 8]) = st.x[o][q];
      }
#pragma unroll
    for (int q = 0; q < kWPieces; ++q) {
      const int p = threadIdx.x + kXBlock * q;
      *reinterpret_cast<uint4*>(&sb[buf][p >> 3][(p & 7) * 8]) = st.w[q];
    }
  };

  f32x4 acc[4][kXFrags];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int f = 0; f < kXFrags; ++f) acc[r][f] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int arow = lane & 15, bk = 8 * (lane >> 4);
  auto compute = [&](int buf) {
    if (nfrag == 0) return;
#pragma unroll
    for (int s = 0; s < kXK / 32; ++s) {
      bf16x8 b[kXFrags];
#pragma unroll
      for (int f = 0; f < kXFrags; ++f)
        b[f] = as_bf16x8(*reinterpret_cast<const uint4*>(
            &sb[buf][wc * kXColsPerWave + 16 * f + arow][32 * s + bk]));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int o = 0; o < kOps; ++o) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(
              &sa[buf][o][64 * wr + 16 * r + arow][32 * s + bk]));
#pragma unroll
          for (int f = 0; f < kXFrags; ++f)
            if (f < nfrag)
              acc[r][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[f], acc[r][f], 0, 0, 0);
        }
      }
    }
  };

  // Loads run two tiles ahead through two register sets; LDS buffers
  // alternate; one barrier per tile (buffer B was last read by the tile two
  // before, whose products every wavefront finished before this barrier).
  // Unrolled by two so the register sets keep fixed names; fetches past the
  // last tile repeat it and are never used.
  const int64_t ntiles = Kp / kXK;
  const int64_t last = ntiles - 1;
  Stage s0, s1;
  fetch(s0, 0);
  fetch(s1, 1 < last ? 1 : last);
  stash(s0, 0);
  fetch(s0, 2 < last ? 2 : last);
  int64_t t = 0;
  for (; t + 2 <= ntiles; t += 2) {
    block_sync();
    stash(s1, 1);
    fetch(s1, t + 3 < last ? t + 3 : last);
    compute(0);
    block_sync();
    stash(s0, 0);
    fetch(s0, t + 4 < last ? t + 4 : last);
    compute(1);
  }
  if (t < ntiles) {
    block_sync();
    compute(0);
  }

  store_tile(acc, lane, wr, m0, c_wave, nfrag, M, ncol, R, dtl, dtl_lo, P, ldp, bcg, bcg_rows);
}

// The same product with the tiles copied from memory straight into LDS
// (buffer_load_dwordx4 ... lds: each lane's 16 bytes land at the LDS address
// M0 + 16 lane), for 16-byte aligned rows, K a multiple of 64 and exactly 192
// output columns (every wavefront's six column fragments in range).  The x
// tile (128 rows of one A operand, or 64 rows of each of the bf16 pair: 16 KB)
// streams from memory; the W^T tile (192 rows, 24 KB) is the same for every
// block and mostly comes from L2.  So the two have rings of their own: five x
// stages, so that four x tiles of copies are in flight while one is
// multiplied, and three W^T stages (two in flight); 152 KB of LDS.  Each row
// is 8 16-byte pieces; piece q of row r sits at position r * 8 +
// (q ^ ((r >> 1) & 7)), so that the 16 rows a fragment read touches fall on
// 16 different 16-byte bank groups, and each copy instruction (64 consecutive
// positions) loads whatever pieces those positions hold.  Per tile: one wait
// for this thread's copies of the tile, one barrier (after it every thread's
// copies of the tile have landed, and every wavefront is done with the stages
// the next copies overwrite), the copies of x tile t + 4 and W^T tile t + 2,
// the products.
template <bool kTwo>
struct LdsTile {
  static constexpr int kOps = kTwo ? 2 : 1;
  static constexpr int kRows = kTwo ? 64 : 128;           // rows of each A operand
  static constexpr int kAPieces = kRows * 8;              // one A operand
  static constexpr int kXPieces = kOps * kAPieces;        // an x stage
  static constexpr int kWPieces = kXCols * 8;             // a W^T stage
  static constexpr int kXCopies = kXPieces / 256;         // copies per wavefront per tile
  static constexpr int kWCopies = kWPieces / 256;
  static constexpr int kRowTiles = kRows / 32;            // 16-row tiles per wavefront
  static constexpr int kXStages = 5, kWStages = 3;
  static_assert(kAPieces % 256 == 0 && kWPieces % 256 == 0, "whole copies per wavefront");
  static_assert((kXStages * kXPieces + kWStages * kWPieces) * 16 <= 160 * 1024,
                "the stages fit in LDS");
};

__device__ __forceinline__ int swz(int r, int q) { return r * 8 + (q ^ ((r >> 1) & 7)); }

template <bool kTwo>
__global__ __launch_bounds__(kXBlock) void xproj_lds_kernel(
    const uint16_t* __restrict__ A0, const uint16_t* __restrict__ A1, int64_t lda,
    const uint16_t* __restrict__ wT, int64_t Kp, int64_t M, int ncol, int R,
    uint16_t* __restrict__ dtl, uint16_t* __restrict__ dtl_lo, float* __restrict__ P,
    int64_t ldp, float* __restrict__ bcg, int64_t bcg_rows) {
  using T = LdsTile<kTwo>;
  constexpr int kOps = T::kOps;
  constexpr int kRows = T::kRows;
  // one array per stage, named by constant stage numbers (the lambdas below
  // are always inlined with literal stages), so the compiler can tell the
  // copies into one stage from the reads of another (else it makes every
  // LDS read wait for all copies in flight)
  __shared__ __align__(16) uint4 xs0[T::kXPieces];
  __shared__ __align__(16) uint4 xs1[T::kXPieces];
  __shared__ __align__(16) uint4 xs2[T::kXPieces];
  __shared__ __align__(16) uint4 xs3[T::kXPieces];
  __shared__ __align__(16) uint4 xs4[T::kXPieces];
  __shared__ __align__(16) uint4 ws0[T::kWPieces];
  __shared__ __align__(16) uint4 ws1[T::kWPieces];
  __shared__ __align__(16) uint4 ws2[T::kWPieces];
  // the stages are written only by the copies, which the compiler does not
  // count as stores to the arrays: their addresses go through an asm
  // statement so that it cannot take them for never written
  asm volatile("" ::"v"(xs0), "v"(xs1), "v"(xs2), "v"(xs3), "v"(xs4), "v"(ws0), "v"(ws1),
               "v"(ws2)
               : "memory");
  auto xring = [&](int S) __attribute__((always_inline)) -> uint4* {
    return S == 0 ? xs0 : S == 1 ? xs1 : S == 2 ? xs2 : S == 3 ? xs3 : xs4;
  };
  auto wring = [&](int S) __attribute__((always_inline)) -> uint4* {
    return S == 0 ? ws0 : S == 1 ? ws1 : ws2;
  };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * kRows;
  const int c0 = static_cast<int>(blockIdx.y) * kXCols;
  const int c_wave = c0 + wc * kXColsPerWave;

  // this thread's copy sources: copy i of wavefront w covers positions
  // 64 (4 i + w) .. 64 (4 i + w) + 63 of its stage; lane j fills position
  // 64 (4 i + w) + j.  x stage positions: A0 pieces (then A1 pieces); an
  // operand's pieces are whole multiples of four copies, so which operand
  // copy i reads does not depend on the wavefront.  Rows past M read the last
  // row (their results are not stored).  Byte offsets from the block's first
  // row / from wT.
  const buf_t xr0 = make_buf(A0 + m0 * lda, 0x7fffffffu);
  const buf_t xr1 = make_buf((kTwo ? A1 : A0) + m0 * lda, 0x7fffffffu);
  const buf_t wr_ = make_buf(wT, 0x7fffffffu);
  uint32_t xoff[T::kXCopies], woff[T::kWCopies];
#pragma unroll
  for (int i = 0; i < T::kXCopies; ++i) {
    const int pa = ((4 * i + wave) * 64 + lane) % T::kAPieces;
    const int r = pa >> 3, q = (pa & 7) ^ ((r >> 1) & 7);
    const int64_t rr = min(m0 + r, M - 1) - m0;
    xoff[i] = static_cast<uint32_t>(rr * lda * 2 + q * 16);
  }
#pragma unroll
  for (int i = 0; i < T::kWCopies; ++i) {
    const int pb = (4 * i + wave) * 64 + lane;
    const int c = pb >> 3, q = (pb & 7) ^ ((c >> 1) & 7);
    woff[i] = static_cast<uint32_t>((c0 + c) * Kp * 2 + q * 16);
  }
  using lds_ptr = __attribute__((address_space(3))) void*;
  const int64_t last = Kp / kXK - 1;
  auto issue_x = [&](int64_t t, int S) __attribute__((always_inline)) {
    const int soff = static_cast<int>((t < last ? t : last) * kXK * 2);   // bytes along k
#pragma unroll
    for (int i = 0; i < T::kXCopies; ++i) {
      const lds_ptr dst = (lds_ptr)(xring(S) + (4 * i + wave) * 64);
      const buf_t src = 4 * i < T::kAPieces / 64 ? xr0 : xr1;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, dst, 16, static_cast<int>(xoff[i]), soff, 0,
                                               0);
    }
  };
  auto issue_w = [&](int64_t t, int S) __attribute__((always_inline)) {
    const int soff = static_cast<int>((t < last ? t : last) * kXK * 2);
#pragma unroll
    for (int i = 0; i < T::kWCopies; ++i) {
      const lds_ptr dst = (lds_ptr)(wring(S) + (4 * i + wave) * 64);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr_, dst, 16, static_cast<int>(woff[i]), soff, 0,
                                               0);
    }
  };

  f32x4 acc[4][kXFrags];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int f = 0; f < kXFrags; ++f) acc[r][f] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int arow = lane & 15, qoff = lane >> 4;
  auto compute = [&](int SX, int SW) __attribute__((always_inline)) {
    const uint4* sx = xring(SX);
    const uint4* sw = wring(SW);
#pragma unroll
    for (int s = 0; s < kXK / 32; ++s) {
      const int q = 4 * s + qoff;
      bf16x8 b[kXFrags];
#pragma unroll
      for (int f = 0; f < kXFrags; ++f) b[f] = as_bf16x8(sw[swz(wc * kXColsPerWave + 16 * f + arow, q)]);
#pragma unroll
      for (int r = 0; r < T::kRowTiles; ++r) {
#pragma unroll
        for (int o = 0; o < kOps; ++o) {
          const bf16x8 a = as_bf16x8(sx[o * T::kAPieces + swz((kRows / 2) * wr + 16 * r + arow, q)]);
#pragma unroll
          for (int f = 0; f < kXFrags; ++f)
            acc[r][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[f], acc[r][f], 0, 0, 0);
        }
      }
    }
  };

  // Copy order: the prologue issues x tiles 0-2, W^T tile 0, then x tile 3 and
  // W^T tile 1; the step of tile t issues x tile t + 4, then W^T tile t + 2.
  // When the step of tile t waits, the copies issued after this thread's
  // copies of x tile t and W^T tile t are at most those of x tile t + 3 and
  // W^T tile t + 1.  s_waitcnt vmcnt(those) lgkmcnt(0): tile t has landed,
  // and this thread's LDS reads of the stages the next copies overwrite are
  // done (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4 left alone,
  // lgkmcnt 11:8).  Copies past the last tile repeat it, unused.
  constexpr int kAhead = T::kXCopies + T::kWCopies;
  constexpr int kWait = (kAhead & 15) | ((kAhead >> 4) << 14) | (7 << 4) | (0 << 8);
  const int64_t ntiles = last + 1;
  // barrier with no memory fence: the copies' own wait is the one that
  // matters, and a fence would wait for every copy in flight
  auto step = [&](int64_t t, int j) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kWait);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue_x(t + 4, (j + 4) % 5);
    issue_w(t + 2, (j + 2) % 3);
    compute(j % 5, j % 3);
  };
  issue_x(0, 0);
  issue_x(1, 1);
  issue_x(2, 2);
  issue_w(0, 0);
  issue_x(3, 3);
  issue_w(1, 1);
  // 15 steps (the stage numbers' common period) per trip, then the rest
  // with exits only, no step that a branch can skip, so that the compiler
  // still tells the stages apart in every step
  int64_t t = 0;
  for (; t + 15 <= ntiles; t += 15) {
#pragma unroll
    for (int j = 0; j < 15; ++j) step(t + j, j);
  }
#pragma unroll
  for (int j = 0; j < 14; ++j) {
    if (t + j >= ntiles) break;
    step(t + j, j);
  }
  __builtin_amdgcn_s_waitcnt(0);             // no copy still in flight at the end
  store_tile<T::kRowTiles>(acc, lane, wr, m0, c_wave, kXFrags, M, ncol, R, dtl, dtl_lo, P, ldp,
                           bcg, bcg_rows);
}

}  // namespace

int64_t xproj_padded_k(int64_t K) { return (K + kXK - 1) / kXK * kXK; }

int64_t xproj_bcg_rows(int64_t M) { return M + 8; }

hipError_t launch_xproj(const uint16_t* x, const uint16_t* x_lo, int64_t lda, int64_t M,
                        int64_t K, const void* W_x, int64_t ncol, int64_t R, uint16_t* WxT,
                        uint16_t* dtl, uint16_t* dtl_lo, float* P, int64_t ldp, float* bcg,
                        hipStream_t stream) {
  if (bcg && ncol - R != 32) return hipErrorInvalidValue;   // grouped B/C: N = 16 only
  const int64_t bcg_rows = bcg ? xproj_bcg_rows(M) : 0;
  if (M <= 0 || ncol <= 0) return hipSuccess;
  const int64_t Kp = xproj_padded_k(K);
  const int64_t tiles = ((Kp + 63) / 64) * ((ncol + 63) / 64);
  const bool tvec = ncol % 8 == 0 && reinterpret_cast<uintptr_t>(W_x) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(WxT) % 16 == 0;   // Kp is a multiple of 64
  hipLaunchKernelGGL(transpose_pad_kernel, dim3(static_cast<unsigned>(tiles)), dim3(256), 0,
                     stream, static_cast<const uint16_t*>(W_x), WxT, K, ncol, Kp, bcg, bcg_rows,
                     M, tvec);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<unsigned>((M + kXRows - 1) / kXRows),
                  static_cast<unsigned>((ncol + kXCols - 1) / kXCols));
  const bool vec = K % 8 == 0 && lda % 8 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                   (x_lo == nullptr || reinterpret_cast<uintptr_t>(x_lo) % 16 == 0);
  const int nc = static_cast<int>(ncol), r = static_cast<int>(R);
#define MSSM_XPROJ(TWO, VEC)                                                                    \
  hipLaunchKernelGGL((xproj_kernel<TWO, VEC>), grid, dim3(kXBlock), 0, stream, x, x_lo, lda,   \
                     WxT, Kp, K, M, nc, r, dtl, dtl_lo, P, ldp, bcg, bcg_rows)
  const bool lds_form = vec && K > 0 && K % kXK == 0 && ncol == kXCols &&
                        M * lda * 2 < (int64_t(1) << 31) && ncol * Kp * 2 < (int64_t(1) << 31);
  if (lds_form) {
    if (x_lo) {
      const dim3 lgrid(static_cast<unsigned>((M + 63) / 64));
      hipLaunchKernelGGL((xproj_lds_kernel<true>), lgrid, dim3(kXBlock), 0, stream, x, x_lo, lda,
                         WxT, Kp, M, nc, r, dtl, dtl_lo, P, ldp, bcg, bcg_rows);
    } else {
      const dim3 lgrid(static_cast<unsigned>((M + 127) / 128));
      hipLaunchKernelGGL((xproj_lds_kernel<false>), lgrid, dim3(kXBlock), 0, stream, x, x, lda,
                         WxT, Kp, M, nc, r, dtl, dtl_lo, P, ldp, bcg, bcg_rows);
    }
  } else if (x_lo) {
    if (vec) MSSM_XPROJ(true, true); else MSSM_XPROJ(true, false);
  } else {
    if (vec) MSSM_XPROJ(false, true); else MSSM_XPROJ(false, false);
  }
#undef MSSM_XPROJ
  return hipGetLastError();
}

}  // namespace mssm
