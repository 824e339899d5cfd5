// Choice between the chunked scan and the single-pass (one lane per channel
// and state) scan, and the single-pass kernel's variant dispatch.
#include <cstdint>

#include "chain_scan.h"

namespace mssm {

namespace {

// Fewest batch * D channels for which the single-pass design is chosen by
// itself.  Its lanes each carry one chain, so a SIMD needs about two of its
// wavefronts (8192 channels on 1024 SIMDs) before the chain's latency is
// hidden; below that the chunked design, which cuts time into chunks for
// parallelism, is faster.
constexpr int64_t kMinChannels = 8192;

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

enum class Design { kAuto, kChunked, kChain };

// The scan-order setting (mssm_set_tuning) pins the design for tests and
// tuning runs; the single pass still needs a supported shape.
Design design_setting() {
  switch (tuning(MSSM_TUNE_SCAN_ORDER)) {
    case MSSM_ORDER_CHUNKED: return Design::kChunked;
    case MSSM_ORDER_SINGLE_PASS: return Design::kChain;
    default: return Design::kAuto;
  }
}

template <bool kZoh, bool kSkip, bool kGate>
hipError_t launch_state(const ScanArgs& a, hipStream_t stream) {
  if (a.h_last) return chain::launch_variant<Variant<kZoh, kSkip, kGate, true>>(a, stream);
  return chain::launch_variant<Variant<kZoh, kSkip, kGate, false>>(a, stream);
}

template <bool kZoh>
hipError_t launch_parts(const ScanArgs& a, hipStream_t stream) {
  const bool skip = a.Dskip != nullptr, gate = a.z != nullptr;
  if (skip && gate) return launch_state<kZoh, true, true>(a, stream);
  if (skip) return launch_state<kZoh, true, false>(a, stream);
  if (gate) return launch_state<kZoh, false, true>(a, stream);
  return launch_state<kZoh, false, false>(a, stream);
}

}  // namespace

bool single_pass_chosen(int64_t channels) {
  const Design d = design_setting();
  if (d == Design::kChunked) return false;
  return d == Design::kChain || channels >= kMinChannels;
}

bool chain_layout_ok(const ScanArgs& a) {
  if (a.N != chain::kStates || a.D % chain::kChannels != 0 || a.L < 1 || a.batch < 1)
    return false;
  // 4-value loads of x, delta, z, B, C and 16-byte stores of y
  const size_t in_align = a.dtype == MSSM_FLOAT32 ? 16 : 8;
  if (!aligned(a.x, in_align) || !aligned(a.delta, in_align) || !aligned(a.B, in_align) ||
      !aligned(a.C, in_align) || (a.z && !aligned(a.z, in_align)) || !aligned(a.y, 16))
    return false;
  // 32-bit lane offsets within a 16-step tile; grid size
  if (a.D * chain::kTile * static_cast<int64_t>(sizeof(float)) >= (int64_t(1) << 31)) return false;
  return a.batch <= (int64_t(1) << 31) / (a.D / chain::kChannels);
}

// Forward only: from this many steps on the chunked order is taken even with
// enough channels for the single pass.  Measured on MI355X at 8192-16384
// channels with two input sets alternating (so the Infinity Cache cannot keep
// the second read of x and delta that the chunked order makes), chunked time /
// single-pass time: bfloat16 1.00-1.02 at L = 8192, 0.96 at 16384, 0.86 at
// 32768; float32 1.03 at L = 16384, 0.93 at 32768 (and about 1.4 at L = 2048).
// The backward keeps the single pass, which beats its chunked order at every
// length.
static int64_t long_sequence_steps(mssm_dtype dtype) {
  return dtype == MSSM_BFLOAT16 ? 16384 : 32768;
}

bool chain_scan_applies(const ScanArgs& a) {
  const Design d = design_setting();
  if (d == Design::kChunked || !chain_layout_ok(a)) return false;
  if (d == Design::kAuto && a.L >= long_sequence_steps(a.dtype)) return false;
  return single_pass_chosen(a.batch * a.D);
}

bool chain_fused_applies(int64_t batch, int64_t D, int64_t N, int64_t R, const void* x,
                         const void* y) {
  if (design_setting() == Design::kChunked) return false;
  if (N != chain::kStates || D % chain::kChannels != 0 || batch < 1) return false;
  if (R > 256) return false;   // the delta kernel keeps W_dt in registers for R <= 256
  if (!aligned(x, 16) || !aligned(y, 16)) return false;
  if (D * chain::kTile * static_cast<int64_t>(sizeof(float)) >= (int64_t(1) << 31)) return false;
  if (batch > (int64_t(1) << 31) / (D / chain::kChannels)) return false;
  return single_pass_chosen(batch * D);
}

namespace {
template <bool kSkip, bool kGate>
hipError_t launch_save_state(const ScanArgs& a, float* ck, float* y_pre, hipStream_t stream) {
  if (a.h_last) return chain::launch_save<Variant<false, kSkip, kGate, true>>(a, ck, y_pre, stream);
  return chain::launch_save<Variant<false, kSkip, kGate, false>>(a, ck, y_pre, stream);
}
}  // namespace

hipError_t launch_chain_save(const ScanArgs& a, float* ck, float* y_pre, hipStream_t stream) {
  const bool skip = a.Dskip != nullptr, gate = a.z != nullptr;
  if (skip && gate) return launch_save_state<true, true>(a, ck, y_pre, stream);
  if (skip) return launch_save_state<true, false>(a, ck, y_pre, stream);
  if (gate) return launch_save_state<false, true>(a, ck, y_pre, stream);
  return launch_save_state<false, false>(a, ck, y_pre, stream);
}

hipError_t launch_chain_scan(const ScanArgs& a, hipStream_t stream) {
  return a.bbar == MSSM_BBAR_ZOH ? launch_parts<true>(a, stream)
                                 : launch_parts<false>(a, stream);
}

}  // namespace mssm
