// Host side of the chunked scan: the carry pass, the plan (chunk length and
// workspace), the chains-per-lane choice and the launch sequence.  The chunk
// kernels themselves are templates in scan_kernels.h, instantiated by the
// scan_summary_*.hip and scan_out_*.hip launchers.
#include "scan_kernels.h"


namespace mssm {

// Carry pass.  For every chain (batch row, state n, channel d) the states
// entering the chunks follow c_{j+1} = P_j c_j + hloc_j (c_0 = h0, or 0),
// with the chunk decay P_j = exp(A S_j) = exp2(A log2(e) S_j) formed from the
// chunk's step-size total S_j (accumulated in float64 by the summary kernels;
// the exponent is taken in float32, which moves P by at most ~5e-8 absolute:
// its rounding error is relative, and |arg| 2^arg peaks near 0.5).  hloc_j is
// overwritten with c_{j+1}, the state entering chunk j + 1.
//
// The recurrence is a first-order linear one, so it composes like the scan
// itself ("Understanding Mamba", section 7.1, eq. (8)): a run of chunks acts
// on its entering state as c -> P c + H, with P the product of the run's
// decays and H the run's result from a zero state.  A block takes 64
// channels of one (batch row, n); its 16 wavefronts take 16 consecutive runs
// of kRun chunks each (one pass; longer sequences take several passes).
// Each wavefront loads its run once (coalesced rows of 64 channels), forms
// the decays and (P, H) of its run in registers, and publishes (P, H) in LDS;
// after one barrier every wavefront folds the runs before its own onto the
// state entering the pass, then replays its run from that state and stores
// the carries.  The dependent chain per pass is kRun + 16 multiply-adds
// instead of one per chunk, and every wavefront's loads are in flight at once.
namespace {
constexpr int kCarryWaves = 16;
constexpr int kRun = 32;
}  // namespace

__global__ __launch_bounds__(64 * kCarryWaves) void chunk_carry_kernel(
    float* __restrict__ sum_h, const double* __restrict__ sum_s, const float* __restrict__ A,
    const float* __restrict__ h0, int64_t D, int N, int K, int64_t n_dtiles) {
  __shared__ float sP[kCarryWaves][64], sH[kCarryWaves][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t bid = blockIdx.x;
  const int64_t dtile = bid % n_dtiles;
  const int64_t rest = bid / n_dtiles;
  const int n = static_cast<int>(rest % N);
  const int64_t b = rest / N;
  const int64_t d_raw = dtile * 64 + lane;
  const bool live = d_raw < D;              // lanes past the last channel only keep step
  const int64_t d = live ? d_raw : D - 1;   // (every wavefront reaches every barrier)
  const int64_t stride = (int64_t)N * D;    // from chunk j to chunk j + 1
  float* hp = sum_h + (b * (K - 1) * N + n) * D + d;
  const double* sp = sum_s + b * (K - 1) * D + d;
  const float a2 = A[d * N + n] * kLog2e;
  float c_pass = h0 != nullptr ? h0[(b * D + d) * N + n] : 0.0f;   // state entering the pass
  const int nj = K - 1;
  for (int pass0 = 0; pass0 < nj; pass0 += kRun * kCarryWaves) {
    const int j0 = pass0 + wave * kRun;
    float hv[kRun], pv[kRun];
    // every load is issued (past the end: the last chunk's, then replaced),
    // so all of a run's loads are in flight together
    double sv[kRun];
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      const int64_t j = min(j0 + i, nj - 1);
      hv[i] = hp[j * stride];
      sv[i] = sp[j * D];
    }
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      const bool in = j0 + i < nj;             // a run past the end acts as c -> c
      pv[i] = in ? fast_exp2(a2 * static_cast<float>(sv[i])) : 1.0f;
      hv[i] = in ? hv[i] : 0.0f;
    }
    float P = 1.0f, H = 0.0f;
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      H = __builtin_fmaf(pv[i], H, hv[i]);
      P *= pv[i];
    }
    sP[wave][lane] = P;
    sH[wave][lane] = H;
    block_sync();
    float c = c_pass;
    for (int w = 0; w < wave; ++w) c = __builtin_fmaf(sP[w][lane], c, sH[w][lane]);
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      c = __builtin_fmaf(pv[i], c, hv[i]);
      if (live && j0 + i < nj) hp[(int64_t)(j0 + i) * stride] = c;
    }
#pragma unroll
    for (int w = 0; w < kCarryWaves; ++w) c_pass = __builtin_fmaf(sP[w][lane], c_pass, sH[w][lane]);
    block_sync();                           // sP / sH are rewritten by the next pass
  }
}

// Writes the final state for an empty sequence: h_last = h0, or zero.
__global__ __launch_bounds__(kBlock) void state_init_kernel(float* __restrict__ h_last,
                                                            const float* __restrict__ h0,
                                                            int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i < count) h_last[i] = h0 != nullptr ? h0[i] : 0.0f;
}

bool state_size_supported(int64_t N) {
  return N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32;
}

static size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

hipError_t launch_carry(float* sum_h, const double* sum_s, const float* A, const float* h0,
                        int64_t batch, int64_t D, int64_t N, int K, hipStream_t stream) {
  const int64_t carry_tiles = (D + 63) / 64;
  const int64_t cgrid = carry_tiles * N * batch;
  hipLaunchKernelGGL(chunk_carry_kernel, dim3((unsigned)cgrid), dim3(64 * kCarryWaves), 0, stream,
                     sum_h, sum_s, A, h0, D, static_cast<int>(N), K, carry_tiles);
  return hipGetLastError();
}

hipError_t launch_state_init(float* h_last, const float* h0, int64_t count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  const int64_t grid = (count + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(state_init_kernel, dim3((unsigned)grid), dim3(kBlock), 0, stream, h_last,
                     h0, count);
  return hipGetLastError();
}

// Two chains per lane pay off for bfloat16 inputs (one 32-bit load brings both
// channels' x and delta; MI355X sweeps: about 10-13% faster), not for float32
// (register pressure lowers occupancy more than the extra ILP gains).
int default_cpl(int64_t D, mssm_dtype dtype) {
  const int64_t v = tuning(MSSM_TUNE_CHAINS_PER_LANE);   // tuning experiments only
  if (v == 1 || v == 2) return (v == 2 && D % 2 == 0) ? 2 : 1;
  return (dtype == MSSM_BFLOAT16 && D % 2 == 0) ? 2 : 1;
}

ScanPlan plan_scan(int64_t batch, int64_t L, int64_t D, int64_t N, int cpl) {
  ScanPlan p;
  p.cpl = cpl;
  if (batch <= 0 || L <= 0 || D <= 0) return p;
  // Chunk count: about 2560 blocks (ten per compute unit over the kernel's
  // life), with chunks of at least 64 steps (128 with two chains per lane).
  // Chunk-length sweeps of the long-sequence bf16 workload on MI355X (K
  // from 100 to 1024 chunks): 256 steps (2560 blocks) fastest, 1.57 ms against
  // 1.66 at 320 steps (2050 blocks) and 1.70 at 128 (the per-chunk cost after
  // the carry pass is small, so more chunks help until chunks get short).  The
  // chunk-length setting overrides it (tuning sweeps and chunk-boundary tests).
  const int64_t blocks_per_chunk = batch * ((D + kBlock * cpl - 1) / (kBlock * cpl));
  const int64_t target_blocks = 2560;
  int64_t K = (target_blocks + blocks_per_chunk / 2) / blocks_per_chunk;
  const int64_t min_chunk = cpl == 1 ? 64 : 128;
  K = std::max<int64_t>(1, std::min<int64_t>(K, L / min_chunk));
  int64_t chunk = (L + K - 1) / K;
  if (const int64_t v = tuning(MSSM_TUNE_CHUNK_LEN); v > 0) chunk = v;
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
    p.sum_s_offset = p.sum_h_bytes;
    p.workspace_bytes =
        p.sum_h_bytes + round_up(sizeof(double) * (size_t)batch * (size_t)(K - 1) * (size_t)D, 256);
  }
  return p;
}

size_t workspace_bound(int64_t batch, int64_t L, int64_t D, int64_t N) {
  size_t w = plan_scan(batch, L, D, N, 1).workspace_bytes;
  if (D % 2 == 0) w = std::max(w, plan_scan(batch, L, D, N, 2).workspace_bytes);
  return w;
}

ScanPlan plan_for(const ScanArgs& a) {
  if (chain_scan_applies(a)) {
    ScanPlan p;
    p.chain = true;
    return p;
  }
  return plan_scan(a.batch, a.L, a.D, a.N, choose_cpl(a));
}

int choose_cpl(const ScanArgs& a) {
  int cpl = default_cpl(a.D, a.dtype);
  const size_t align = 2 * (a.dtype == MSSM_FLOAT32 ? 4 : 2);
  if (cpl == 2 && (reinterpret_cast<uintptr_t>(a.x) % align != 0 ||
                   reinterpret_cast<uintptr_t>(a.delta) % align != 0 ||
                   reinterpret_cast<uintptr_t>(a.z) % align != 0 ||
                   reinterpret_cast<uintptr_t>(a.y) % 8 != 0))
    cpl = 1;
  return cpl;
}

template <bool kZoh, bool kSkip, bool kGate>
static hipError_t launch_output_state(const ScanArgs& a, const ScanPlan& plan,
                                      const ScanParams& p, hipStream_t stream) {
  if (a.h_last != nullptr)
    return launch_output_variant<Variant<kZoh, kSkip, kGate, true>>(a, plan, p, stream);
  return launch_output_variant<Variant<kZoh, kSkip, kGate, false>>(a, plan, p, stream);
}

template <bool kZoh>
static hipError_t launch_output_zoh(const ScanArgs& a, const ScanPlan& plan, const ScanParams& p,
                                    hipStream_t stream) {
  const bool skip = a.Dskip != nullptr, gate = a.z != nullptr;
  if (skip && gate) return launch_output_state<kZoh, true, true>(a, plan, p, stream);
  if (skip) return launch_output_state<kZoh, true, false>(a, plan, p, stream);
  if (gate) return launch_output_state<kZoh, false, true>(a, plan, p, stream);
  return launch_output_state<kZoh, false, false>(a, plan, p, stream);
}

static hipError_t launch_output(const ScanArgs& a, const ScanPlan& plan, const ScanParams& p,
                                hipStream_t stream) {
  return a.bbar == MSSM_BBAR_ZOH ? launch_output_zoh<true>(a, plan, p, stream)
                                 : launch_output_zoh<false>(a, plan, p, stream);
}

hipError_t launch_scan(const ScanArgs& a, const ScanPlan& plan, void* ws, hipStream_t stream) {
  if (plan.chain) return launch_chain_scan(a, stream);
  ScanParams p{};
  p.x = a.x;
  p.delta = a.delta;
  p.A = a.A;
  p.B = a.B;
  p.C = a.C;
  p.Dskip = a.Dskip;
  p.z = a.z;
  p.h0 = a.h0;
  p.h_last = a.h_last;
  p.y = static_cast<float*>(a.y);
  p.L = a.L;
  p.D = a.D;
  p.chunk_len = plan.chunk_len;
  p.K = plan.K;
  p.n_dtiles = (a.D + kBlock * plan.cpl - 1) / (kBlock * plan.cpl);
  const bool zoh = a.bbar == MSSM_BBAR_ZOH;
  if (plan.K > 1) {
    p.sum_h = static_cast<float*>(ws);
    p.sum_s = reinterpret_cast<double*>(static_cast<char*>(ws) + plan.sum_s_offset);
    hipError_t e = zoh ? launch_summary_zoh(a, plan, p, stream)
                       : launch_summary_euler(a, plan, p, stream);
    if (e != hipSuccess) return e;
    e = launch_carry(p.sum_h, p.sum_s, a.A, a.h0, a.batch, a.D, a.N, plan.K, stream);
    if (e != hipSuccess) return e;
  }
  return launch_output(a, plan, p, stream);
}

}  // namespace mssm
