// Output-pass launcher: zero-order hold input term, feedthrough D x.
#include "scan_kernels.h"

namespace mssm {

MSSM_DEFINE_OUTPUT_VARIANT(true, true, false)

}  // namespace mssm
