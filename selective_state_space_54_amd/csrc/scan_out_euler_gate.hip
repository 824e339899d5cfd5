// Output-pass launcher: first order input term, SiLU(z) gate.
#include "scan_kernels.h"

namespace mssm {

MSSM_DEFINE_OUTPUT_VARIANT(false, false, true)

}  // namespace mssm
