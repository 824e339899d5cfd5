// Output-pass launcher: first order input term, feedthrough D x and SiLU(z) gate.
#include "scan_kernels.h"

namespace mssm {

MSSM_DEFINE_OUTPUT_VARIANT(false, true, true)

}  // namespace mssm
