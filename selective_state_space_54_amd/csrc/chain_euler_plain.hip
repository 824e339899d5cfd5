// Single-pass (one lane per channel and state) scan launchers: first-order input term,
// without the final state; every feedthrough / gate combination.
#include "chain_scan.h"

namespace mssm {

MSSM_DEFINE_CHAIN_VARIANT(false, false, false, false)
MSSM_DEFINE_CHAIN_VARIANT(false, true, false, false)
MSSM_DEFINE_CHAIN_VARIANT(false, false, true, false)
MSSM_DEFINE_CHAIN_VARIANT(false, true, true, false)

}  // namespace mssm
