// scan_fwd_n16.hip -- instantiates the forward scan kernels for state size 16
// (split from the other sizes so that they compile in parallel).
#include "scan_fwd_impl.h"

namespace mssm {

hipError_t launch_scan_n16(const ScanParams& p, bool bf16, bool vec,
                          hipStream_t stream) {
  return fwd::launch_conv<16>(p, bf16, vec, stream);
}

}  // namespace mssm
