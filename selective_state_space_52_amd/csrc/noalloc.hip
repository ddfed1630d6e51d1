// noalloc.hip -- the allocation-free forward scan.  Its workspace (the packed
// B/C runs and the summaries of rows split in time) is a scratch array in
// device memory that is part of the library's code object, so a call makes
// no allocation: for code under HIP graph capture, serving loops and
// harnesses that cannot call hipMalloc.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "mssm.h"
#include "mssm_internal.h"

namespace {

// One copy per device, held from the library's first use on that device
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not the device array: its device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[MSSM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device
std::mutex g_scratch_lock;

}  // namespace

namespace mssm {

void* noalloc_scratch(hipError_t* err) {
  *err = hipSuccess;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> guard(g_scratch_lock);
  if (!g_scratch_ptr[dev]) {
    // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace mssm

extern "C" int mssm_selective_scan_fwd_noalloc(const void* u, const void* delta,
                                               const float* A, const void* B,
                                               const void* C, const float* D,
                                               const void* z, const float* delta_bias,
                                               int softplus, void* out, float* last_state,
                                               const mssm_dims* dims, void* stream) {
  return mssm::scan_fwd_entry(u, delta, A, B, C, D, z, delta_bias, softplus, out,
                              last_state, nullptr, nullptr, nullptr, nullptr, nullptr,
                              MSSM_NOALLOC_SCRATCH_BYTES, mssm::WsMode::kScratch, dims,
                              stream);
}
