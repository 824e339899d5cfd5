// Output-pass launcher: zero-order hold input term, no feedthrough, no gate.
#include "scan_kernels.h"

namespace mssm {

MSSM_DEFINE_OUTPUT_VARIANT(true, false, false)

}  // namespace mssm
