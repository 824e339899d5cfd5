// Single-pass (one lane per channel and state) scan launchers: exact zero-order-hold input term,
// writing the final state; every feedthrough / gate combination.
#include "chain_scan.h"

namespace mssm {

MSSM_DEFINE_CHAIN_VARIANT(true, false, false, true)
MSSM_DEFINE_CHAIN_VARIANT(true, true, false, true)
MSSM_DEFINE_CHAIN_VARIANT(true, false, true, true)
MSSM_DEFINE_CHAIN_VARIANT(true, true, true, true)

}  // namespace mssm
