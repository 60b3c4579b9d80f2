// The buffer-form build of the sequential scan kernel (scan_kernel.h): row
// loads relative to a stream's table, for tables of at most 2^31 bytes.  A
// translation unit of its own so that the two builds compile in parallel.
#include "scan_kernel.h"

namespace sdm {

hipError_t launch_scan_kernel_buf(const ScanArgs& a, const ScanPlan& p, bool vbf16,
                                  hipStream_t stream) {
  return launch_scan_kernel<true>(a, p, vbf16, stream);
}

}  // namespace sdm
