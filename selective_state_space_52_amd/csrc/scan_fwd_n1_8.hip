// scan_fwd_n1_8.hip -- instantiates the forward scan kernels for state sizes 1, 2, 4, 8
// (split from the other sizes so that they compile in parallel).
#include "scan_fwd_impl.h"

namespace mssm {

hipError_t launch_scan_n1(const ScanParams& p, bool bf16, bool vec,
                          hipStream_t stream) {
  return fwd::launch_conv<1>(p, bf16, vec, stream);
}

hipError_t launch_scan_n2(const ScanParams& p, bool bf16, bool vec,
                          hipStream_t stream) {
  return fwd::launch_conv<2>(p, bf16, vec, stream);
}

hipError_t launch_scan_n4(const ScanParams& p, bool bf16, bool vec,
                          hipStream_t stream) {
  return fwd::launch_conv<4>(p, bf16, vec, stream);
}

hipError_t launch_scan_n8(const ScanParams& p, bool bf16, bool vec,
                          hipStream_t stream) {
  return fwd::launch_conv<8>(p, bf16, vec, stream);
}

}  // namespace mssm
