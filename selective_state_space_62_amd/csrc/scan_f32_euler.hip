// Instantiates the scan kernels for fp32 I/O with the first-order (Euler) discretisation of B.
#include "scan_kernel.h"

namespace ssscan {

hipError_t launch_scan_f32_euler(const ScanDims& dm, const ScanPtrs& p, bool aggregate, hipStream_t s) {
  return scan_detail::launch_scan_impl<dev::F32, false>(dm, p, aggregate, s);
}

}  // namespace ssscan
