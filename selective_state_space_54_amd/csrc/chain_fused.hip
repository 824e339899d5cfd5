// Single-pass scan launchers behind the selection projections (one lane per
// channel and state; from 32768 channels on, the split-state kernel): the fused
// selective SSM (bfloat16 x, float32 y) and the Mamba block (float32 x, the
// feedthrough D x, the SiLU(z) gate, y stored as a bfloat16 hi + lo pair for
// the output projection).  delta is the float32 matrix written by the
// dt_proj + softplus kernel; B and C are read straight out of the projection
// P = [dt_low | B | C] (rows of R + 2N floats).
#include "chain_scan.h"

namespace mssm {

hipError_t launch_chain_fused(const ChainFusedArgs& a, hipStream_t stream) {
  // with enough channels the state is split over the wavefronts of a block
  // instead (split_scan.hip): no cross-lane operands in the step
  if (split_fused_applies(a.batch, a.D, chain::kStates)) return launch_split_fused(a, stream);
  chain::ChainParams p{a.x,     a.delta, a.P + a.R, a.P + a.R + chain::kStates,
                       a.z,     a.A,     a.Dskip,   nullptr,
                       nullptr, a.y,     a.y_lo,    a.L,
                       a.D,     a.ldp};
  if (!a.x_f32) {
    if (a.z || a.Dskip || a.y_bf16) return hipErrorInvalidValue;   // the fused SSM's form only
    return chain::launch_io<chain::ChainIO<uint16_t, float, float, float>, PlainVariant>(
        p, a.batch, stream);
  }
  if (!a.z || !a.y_bf16 || !a.y_lo) return hipErrorInvalidValue;   // the block's form only
  p.ld_y = a.ld_y ? a.ld_y : a.D;
  if (p.ld_y < a.D || p.ld_y % 8 != 0) return hipErrorInvalidValue;   // 16-byte rows
  using IO = chain::ChainIO<float, float, float, uint16_t>;
  if (a.Dskip) return chain::launch_io<IO, Variant<false, true, true>>(p, a.batch, stream);
  return chain::launch_io<IO, Variant<false, false, true>>(p, a.batch, stream);
}

}  // namespace mssm
