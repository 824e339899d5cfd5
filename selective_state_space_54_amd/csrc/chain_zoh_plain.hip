// Single-pass (one lane per channel and state) scan launchers: exact zero-order-hold input term,
// without the final state; every feedthrough / gate combination.
#include "chain_scan.h"

namespace mssm {

MSSM_DEFINE_CHAIN_VARIANT(true, false, false, false)
MSSM_DEFINE_CHAIN_VARIANT(true, true, false, false)
MSSM_DEFINE_CHAIN_VARIANT(true, false, true, false)
MSSM_DEFINE_CHAIN_VARIANT(true, true, true, false)

}  // namespace mssm
