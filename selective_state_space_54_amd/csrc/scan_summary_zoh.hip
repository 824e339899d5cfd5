// Summary-pass launcher, exact zero-order-hold input term.
#include "scan_kernels.h"

namespace mssm {

hipError_t launch_summary_zoh(const ScanArgs& a, const ScanPlan& plan, const ScanParams& p,
                             hipStream_t stream) {
  return dispatch_shape(a, plan.cpl, SummaryLaunch<true>{p, a.batch, stream});
}

}  // namespace mssm
