// Instantiates the scan kernels for bf16 I/O with the zero-order-hold discretisation of B.
#include "scan_kernel.h"

namespace ssscan {

hipError_t launch_scan_bf16_zoh(const ScanDims& dm, const ScanPtrs& p, bool aggregate, hipStream_t s) {
  return scan_detail::launch_scan_impl<dev::BF16, true>(dm, p, aggregate, s);
}

}  // namespace ssscan
