// Output-pass launcher: first order input term, no feedthrough, no gate.
#include "scan_kernels.h"

namespace mssm {

MSSM_DEFINE_OUTPUT_VARIANT(false, false, false)

}  // namespace mssm
