// The zero-order-hold instantiation of the backward main kernel
// (scan_bwd_kernel.h), compiled on its own to keep builds parallel.
#include "scan_bwd_kernel.h"

namespace ssscan {

hipError_t launch_scan_bwd_zoh_main(const BwdDims& dm, const BwdPtrs& p, hipStream_t s) {
  return dm.io == kIoBf16 ? bwd_detail::launch_bwd_n<dev::BF16, true>(dm, p, s)
                          : bwd_detail::launch_bwd_n<dev::F32, true>(dm, p, s);
}

}  // namespace ssscan
