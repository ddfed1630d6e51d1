// state_update.hip -- single-token decode step for gfx950.
//
// The inference form of the recurrence: one token per sequence, with the
// fixed-size state carried between calls and updated in place (page "Mamba:
// Selective State Space Models", "Mathematical Foundation / Efficient Scan":
// sequential scan with constant memory).  Per (batch b, channel d) row:
//   Delta  = softplus(dt + bias[d])
//   h[n]  <- exp(Delta A[d,n]) h[n] + Delta B[b,n] x
//   out    = (sum_n C[b,n] h[n] + D[d] x) * silu(z)
//
// The step is bound by HBM: the fp32 state (64 B per row at N = 16) is read
// and written once and dominates the bytes.  One lane owns one row; the lanes
// of a wave own consecutive rows, so the state is streamed with 16-byte
// accesses that together cover contiguous memory.
#include "dev_math.h"
#include "mssm_internal.h"

namespace mssm {
namespace {

struct UpdateShape {
  int64_t batch, dim;
  int32_t softplus;
};

template <bool BF16>
__device__ __forceinline__ float load_io(const void* base, int64_t i) {
  if constexpr (BF16)
    return bf16_bits(static_cast<const uint16_t*>(base)[i]);
  else
    return static_cast<const float*>(base)[i];
}

template <int N, bool BF16, bool VEC, bool HAS_Z>
__global__ void __launch_bounds__(256)
    state_update_kernel(float* __restrict__ state, const void* __restrict__ x,
                        const void* __restrict__ dt,
                        const void* __restrict__ z,
                        const float* __restrict__ A,
                        const void* __restrict__ Bm,
                        const void* __restrict__ Cm,
                        const float* __restrict__ Dv,
                        const float* __restrict__ bias,
                        void* __restrict__ out, const UpdateShape s) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= s.batch * s.dim) return;
  const int64_t b = r / s.dim;
  const int64_t d = r - b * s.dim;

  const float xv = load_io<BF16>(x, r);
  const float xr = load_io<BF16>(dt, r) + (bias ? bias[d] : 0.0f);
  const float dl = s.softplus ? softplus_f32(xr) : xr;
  const float w = dl * xv;

  float h[N], a[N];
  if constexpr (VEC && N % 4 == 0) {
    const float4* sp = reinterpret_cast<const float4*>(state + r * N);
    const float4* ap = reinterpret_cast<const float4*>(A + d * N);
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const float4 hv = sp[q], av = ap[q];
      h[4 * q] = hv.x; h[4 * q + 1] = hv.y; h[4 * q + 2] = hv.z; h[4 * q + 3] = hv.w;
      a[4 * q] = av.x; a[4 * q + 1] = av.y; a[4 * q + 2] = av.z; a[4 * q + 3] = av.w;
    }
  } else {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      h[n] = state[r * N + n];
      a[n] = A[d * N + n];
    }
  }

  float y = 0.0f;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const float e = hw_exp2(dl * (a[n] * kLog2e));
    h[n] = fmaf(e, h[n], w * load_io<BF16>(Bm, b * N + n));
    y = fmaf(load_io<BF16>(Cm, b * N + n), h[n], y);
  }
  y = fmaf(Dv ? Dv[d] : 0.0f, xv, y);
  if (HAS_Z) y *= silu_f32(load_io<BF16>(z, r));

  if constexpr (VEC && N % 4 == 0) {
    float4* sp = reinterpret_cast<float4*>(state + r * N);
#pragma unroll
    for (int q = 0; q < N / 4; ++q)
      sp[q] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
  } else {
#pragma unroll
    for (int n = 0; n < N; ++n) state[r * N + n] = h[n];
  }
  if constexpr (BF16)
    static_cast<uint16_t*>(out)[r] = to_bf16(y);
  else
    static_cast<float*>(out)[r] = y;
}

template <int N, bool BF16, bool VEC>
hipError_t launch_u(const UpdateParams& p, hipStream_t stream) {
  UpdateShape s{p.batch, p.dim, p.softplus};
  const int64_t rows = p.batch * p.dim;
  const dim3 grid((unsigned)((rows + 255) / 256));
  if (p.z)
    hipLaunchKernelGGL((state_update_kernel<N, BF16, VEC, true>), grid,
                       dim3(256), 0, stream, p.state, p.x, p.dt, p.z, p.A,
                       p.B, p.C, p.D, p.bias, p.out, s);
  else
    hipLaunchKernelGGL((state_update_kernel<N, BF16, VEC, false>), grid,
                       dim3(256), 0, stream, p.state, p.x, p.dt, p.z, p.A,
                       p.B, p.C, p.D, p.bias, p.out, s);
  return hipGetLastError();
}

template <int N>
hipError_t launch_un(const UpdateParams& p, bool bf16, hipStream_t stream) {
  const bool vec = ((uintptr_t)p.state % 16 == 0) && ((uintptr_t)p.A % 16 == 0);
  if (bf16)
    return vec ? launch_u<N, true, true>(p, stream)
               : launch_u<N, true, false>(p, stream);
  return vec ? launch_u<N, false, true>(p, stream)
             : launch_u<N, false, false>(p, stream);
}

}  // namespace

hipError_t launch_state_update(const UpdateParams& p, int N, bool bf16,
                               hipStream_t stream) {
  switch (N) {
    case 1: return launch_un<1>(p, bf16, stream);
    case 2: return launch_un<2>(p, bf16, stream);
    case 4: return launch_un<4>(p, bf16, stream);
    case 8: return launch_un<8>(p, bf16, stream);
    case 16: return launch_un<16>(p, bf16, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mssm
