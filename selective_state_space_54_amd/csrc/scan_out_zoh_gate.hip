// Output-pass launcher: zero-order hold input term, SiLU(z) gate.
#include "scan_kernels.h"

namespace mssm {

MSSM_DEFINE_OUTPUT_VARIANT(true, false, true)

}  // namespace mssm
