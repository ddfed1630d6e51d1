// scan_fwd_n128.hip -- instantiates the forward scan kernels for state size 128
// (split from the other sizes so that they compile in parallel).
#include "scan_fwd_impl.h"

namespace mssm {

hipError_t launch_scan_n128(const ScanParams& p, bool bf16, bool vec,
                          hipStream_t stream) {
  return fwd::launch_conv<128>(p, bf16, vec, stream);
}

}  // namespace mssm
