// scan_fwd_n32.hip -- instantiates the forward scan kernels for state size 32
// (split from the other sizes so that they compile in parallel).
#include "scan_fwd_impl.h"

namespace mssm {

hipError_t launch_scan_n32(const ScanParams& p, bool bf16, bool vec,
                          hipStream_t stream) {
  return fwd::launch_conv<32>(p, bf16, vec, stream);
}

}  // namespace mssm
