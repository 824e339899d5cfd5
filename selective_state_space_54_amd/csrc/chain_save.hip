// The single-pass forward that also saves the backward pass's checkpoints
// (and the output before the gate), one instantiation per set of parts.
#include "chain_scan.h"

namespace mssm {

MSSM_DEFINE_CHAIN_SAVE(false, false, false)
MSSM_DEFINE_CHAIN_SAVE(false, false, true)
MSSM_DEFINE_CHAIN_SAVE(false, true, false)
MSSM_DEFINE_CHAIN_SAVE(false, true, true)
MSSM_DEFINE_CHAIN_SAVE(true, false, false)
MSSM_DEFINE_CHAIN_SAVE(true, false, true)
MSSM_DEFINE_CHAIN_SAVE(true, true, false)
MSSM_DEFINE_CHAIN_SAVE(true, true, true)

}  // namespace mssm
