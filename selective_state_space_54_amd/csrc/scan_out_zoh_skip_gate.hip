// Output-pass launcher: zero-order hold input term, feedthrough D x and SiLU(z) gate.
#include "scan_kernels.h"

namespace mssm {

MSSM_DEFINE_OUTPUT_VARIANT(true, true, true)

}  // namespace mssm
