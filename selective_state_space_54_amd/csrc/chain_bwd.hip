// The single-pass backward: checkpoints (the forward kernel storing every
// tile's final state) and the reverse kernel, dispatched over the element type
// and the optional parts.
#include <cstdint>

#include "chain_bwd.h"

namespace mssm {

namespace {

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

template <typename T, bool kSaved>
hipError_t launch_parts(const chain::ChainBwdParams& p, const BwdArgs& a, hipStream_t stream) {
  const bool skip = a.Dskip != nullptr, gate = a.z != nullptr;
  if (skip && gate) return chain::launch_bwd_chain_t<T, true, true, kSaved>(p, a.batch, stream);
  if (skip) return chain::launch_bwd_chain_t<T, true, false, kSaved>(p, a.batch, stream);
  if (gate) return chain::launch_bwd_chain_t<T, false, true, kSaved>(p, a.batch, stream);
  return chain::launch_bwd_chain_t<T, false, false, kSaved>(p, a.batch, stream);
}

// saved: the checkpoints in ck (and y_pre with the gate) come from the
// forward call; else the checkpoint pass writes ck first.
template <typename T>
hipError_t launch_typed(const BwdArgs& a, float* ck, const float* y_pre, bool saved,
                        float* part_bc, float* part_a, float* part_d, hipStream_t stream) {
  if (!saved) {
    chain::ChainParams cp{a.x,     a.delta, a.B,     a.C,     nullptr, a.A, nullptr, a.h0,
                          nullptr, nullptr, nullptr, a.L,     a.D,     chain::kStates};
    cp.ck = ck;
    const hipError_t e =
        chain::launch_io<chain::ChainIO<T, T, T, float>, PlainVariant, chain::kCkOnly>(
            cp, a.batch, stream);
    if (e != hipSuccess) return e;
  }
  chain::ChainBwdParams p{};
  p.x = a.x;
  p.delta = a.delta;
  p.B = a.B;
  p.C = a.C;
  p.z = a.z;
  p.A = a.A;
  p.Dskip = a.Dskip;
  p.h0 = a.h0;
  p.dout = a.dout;
  p.ck = ck;
  p.y_pre = y_pre;
  p.dx = a.dx;
  p.ddelta = a.ddelta;
  p.dz = a.dz;
  p.dh0 = a.dh0;
  p.part_bc = part_bc;
  p.part_a = part_a;
  p.part_d = part_d;
  p.L = a.L;
  p.D = a.D;
  return saved ? launch_parts<T, true>(p, a, stream) : launch_parts<T, false>(p, a, stream);
}

}  // namespace

bool chain_bwd_layout_ok(const BwdArgs& a) {
  if (a.N != chain::kStates || a.D % chain::kChannels != 0 || a.L < 1 || a.batch < 1)
    return false;
  const size_t in_align = a.dtype == MSSM_FLOAT32 ? 16 : 8;
  if (!aligned(a.x, in_align) || !aligned(a.delta, in_align) || !aligned(a.B, in_align) ||
      !aligned(a.C, in_align) || (a.z && !aligned(a.z, in_align)) || !aligned(a.dout, 16) ||
      !aligned(a.dx, 16) || !aligned(a.ddelta, 16) || (a.dz && !aligned(a.dz, 16)))
    return false;
  if (a.D * chain::kTile * static_cast<int64_t>(sizeof(float)) >= (int64_t(1) << 31)) return false;
  if (a.batch > (int64_t(1) << 31) / (a.D / chain::kChannels)) return false;
  if (a.saved_ck && !aligned(a.saved_ck, 16)) return false;
  if (a.saved_y_pre && !aligned(a.saved_y_pre, 16)) return false;
  return true;
}

bool chain_bwd_applies(const BwdArgs& a) {
  return chain_bwd_layout_ok(a) && single_pass_chosen(a.batch * a.D);
}

hipError_t launch_chain_bwd(const BwdArgs& a, float* ck, const float* y_pre, bool saved,
                            float* part_bc, float* part_a, float* part_d, hipStream_t stream) {
  if (a.dtype == MSSM_FLOAT32)
    return launch_typed<float>(a, ck, y_pre, saved, part_bc, part_a, part_d, stream);
  return launch_typed<uint16_t>(a, ck, y_pre, saved, part_bc, part_a, part_d, stream);
}

}  // namespace mssm
