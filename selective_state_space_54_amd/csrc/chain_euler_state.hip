// Single-pass (one lane per channel and state) scan launchers: first-order input term,
// writing the final state; every feedthrough / gate combination.
#include "chain_scan.h"

namespace mssm {

MSSM_DEFINE_CHAIN_VARIANT(false, false, false, true)
MSSM_DEFINE_CHAIN_VARIANT(false, true, false, true)
MSSM_DEFINE_CHAIN_VARIANT(false, false, true, true)
MSSM_DEFINE_CHAIN_VARIANT(false, true, true, true)

}  // namespace mssm
