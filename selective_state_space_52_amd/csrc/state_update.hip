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
// and written once and dominates the bytes.  Rows go to consecutive lanes
// (N / 4 lanes per row from N = 8 on), so the state is streamed with 16-byte
// accesses that cover contiguous memory.
#include "dev_math.h"
#include "mssm_internal.h"
#include "scan_common.h"

namespace mssm {
namespace {

struct UpdateShape {
  int64_t batch, dim;
  int32_t softplus;
  int32_t ngroups;  // B, C are (batch, ngroups, N); channel d reads d / (dim / ngroups)
};

template <bool BF16>
__device__ __forceinline__ float load_io(const void* base, int64_t i) {
  if constexpr (BF16)
    return bf16_bits(static_cast<const uint16_t*>(base)[i]);
  else
    return static_cast<const float*>(base)[i];
}

// Lanes per row: from N = 8 on, N / 4 lanes each own 4 states of the row, so
// consecutive lanes read consecutive 16-byte pieces of the state and one
// load instruction of a wave covers 1 KB of contiguous memory; the partial
// readouts are summed across the row's lanes.  Below N = 8, one lane per row.
template <int N>
constexpr int kLanesPerRow = N >= 8 ? N / 4 : 1;

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
  constexpr int LPR = kLanesPerRow<N>;
  constexpr int NPL = N / LPR;  // states per lane
  const int64_t rows = s.batch * s.dim;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r_raw = tid / LPR;
  const int part = (int)(tid % LPR);
  // every lane of a row group takes part in the cross-lane sum, so lanes
  // past the last row compute on the last row and store nothing
  const bool active = r_raw < rows;
  if (LPR == 1 && !active) return;
  const int64_t r = active ? r_raw : rows - 1;
  const int64_t b = r / s.dim;
  const int64_t d = r - b * s.dim;
  const int n0 = part * NPL;
  const int64_t bc = (b * s.ngroups + d / (s.dim / s.ngroups)) * N;  // this row's B, C

  const float xv = load_io<BF16>(x, r);
  const float xr = load_io<BF16>(dt, r) + (bias ? bias[d] : 0.0f);
  const float dl = s.softplus ? softplus_f32(xr) : xr;
  const float w = dl * xv;

  float h[NPL], a[NPL];
  float* __restrict__ sp = state + r * N + n0;
  const float* __restrict__ ap = A + d * N + n0;
  if constexpr (VEC && NPL % 4 == 0) {
#pragma unroll
    for (int q = 0; q < NPL / 4; ++q) {
      const float4 hv = reinterpret_cast<const float4*>(sp)[q];
      const float4 av = reinterpret_cast<const float4*>(ap)[q];
      h[4 * q] = hv.x; h[4 * q + 1] = hv.y; h[4 * q + 2] = hv.z; h[4 * q + 3] = hv.w;
      a[4 * q] = av.x; a[4 * q + 1] = av.y; a[4 * q + 2] = av.z; a[4 * q + 3] = av.w;
    }
  } else {
#pragma unroll
    for (int n = 0; n < NPL; ++n) {
      h[n] = sp[n];
      a[n] = ap[n];
    }
  }

  // this lane's B and C values: the same for every row of a group, read as
  // 16-byte pieces where the layout allows (one load instead of 8 or 4)
  float bv[NPL], cvv[NPL];
  if constexpr (VEC && (BF16 ? NPL >= 2 : true)) {
    Raw<BF16, NPL> rb, rc;
    load_chunk<BF16, true, NPL>(rb, Bm, bc + n0, NPL);
    load_chunk<BF16, true, NPL>(rc, Cm, bc + n0, NPL);
#pragma unroll
    for (int n = 0; n < NPL; ++n) {
      bv[n] = raw_get(rb, n);
      cvv[n] = raw_get(rc, n);
    }
  } else {
#pragma unroll
    for (int n = 0; n < NPL; ++n) {
      bv[n] = load_io<BF16>(Bm, bc + n0 + n);
      cvv[n] = load_io<BF16>(Cm, bc + n0 + n);
    }
  }

  float y = 0.0f;
#pragma unroll
  for (int n = 0; n < NPL; ++n) {
    const float e = hw_exp2(dl * (a[n] * kLog2e));
    h[n] = fmaf(e, h[n], w * bv[n]);
    y = fmaf(cvv[n], h[n], y);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off /= 2) y += __shfl_xor(y, off);
  y = fmaf(Dv ? Dv[d] : 0.0f, xv, y);
  if (HAS_Z) y *= silu_f32(load_io<BF16>(z, r));

  if (!active) return;
  if constexpr (VEC && NPL % 4 == 0) {
#pragma unroll
    for (int q = 0; q < NPL / 4; ++q)
      reinterpret_cast<float4*>(sp)[q] =
          make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
  } else {
#pragma unroll
    for (int n = 0; n < NPL; ++n) sp[n] = h[n];
  }
  if (part == 0) {
    if constexpr (BF16)
      static_cast<uint16_t*>(out)[r] = to_bf16(y);
    else
      static_cast<float*>(out)[r] = y;
  }
}

template <int N, bool BF16, bool VEC>
hipError_t launch_u(const UpdateParams& p, hipStream_t stream) {
  UpdateShape s{p.batch, p.dim, p.softplus, p.ngroups > 1 ? p.ngroups : 1};
  const int64_t threads = p.batch * p.dim * kLanesPerRow<N>;
  const dim3 grid((unsigned)((threads + 255) / 256));
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
  // 16-byte pieces: the state and A rows, and the B / C rows (their starts
  // are multiples of N values, so 16-byte aligned bases keep them aligned)
  const bool vec = ((uintptr_t)p.state % 16 == 0) && ((uintptr_t)p.A % 16 == 0) &&
                   ((uintptr_t)p.B % 16 == 0) && ((uintptr_t)p.C % 16 == 0);
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
    case 32: return launch_un<32>(p, bf16, stream);
    case 64: return launch_un<64>(p, bf16, stream);
    case 128: return launch_un<128>(p, bf16, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mssm
