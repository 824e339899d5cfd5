// Summary-pass launcher, first-order input term.
#include "scan_kernels.h"

namespace mssm {

hipError_t launch_summary_euler(const ScanArgs& a, const ScanPlan& plan, const ScanParams& p,
                             hipStream_t stream) {
  return dispatch_shape(a, plan.cpl, SummaryLaunch<false>{p, a.batch, stream});
}

}  // namespace mssm
