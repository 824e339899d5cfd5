// Output-pass launcher: first order input term, feedthrough D x.
#include "scan_kernels.h"

namespace mssm {

MSSM_DEFINE_OUTPUT_VARIANT(false, true, false)

}  // namespace mssm
