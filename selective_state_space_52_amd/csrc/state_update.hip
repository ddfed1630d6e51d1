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
  U32Div dim_div;  // row / dim on the 32-bit index path (rows below 2^31)
};

// Sum of y over the LPR lanes of a row (aligned groups of LPR lanes), with
// every lane of the row getting the sum.  Up to 16 lanes the steps are DPP
// moves within a row of 16 lanes (no trip through LDS): the lane two and one
// away inside a quad, then the mirrored lane inside each 8 and each 16; a
// 32-lane row adds the lane 16 away.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int LPR>
__device__ __forceinline__ float row_sum(float y) {
  if constexpr (LPR >= 32) y += __shfl_xor(y, 16);
  if constexpr (LPR >= 16) y += dpp_mov<0x140>(y);  // row_mirror
  if constexpr (LPR >= 8) y += dpp_mov<0x141>(y);   // row_half_mirror
  if constexpr (LPR >= 4) y += dpp_mov<0x4E>(y);    // quad_perm [2,3,0,1]
  if constexpr (LPR >= 2) y += dpp_mov<0xB1>(y);    // quad_perm [1,0,3,2]
  return y;
}

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

// Row pieces per thread: a wave owns kItems consecutive 64-piece spans and
// issues the loads of all of them before it waits.  One is enough once every
// load of the step is issued before the first use (the state's load used to
// wait behind the softplus of dt): 2, 4 and 8 pieces measured 3%, 7% and 18%
// slower at 256 x 5120 rows of 16 states.
constexpr int kItems = 1;
constexpr int kBlock = 256;

// Idx: uint32_t when every row, state and B/C index fits in 31 bits (the
// common case: cheap division by the channel count), else int64_t.
// The state's loads and stores, with non-temporal (streaming) hints when NT.
typedef float f32x4v __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ float4 state_load4(const float* p) {
  if constexpr (NT) {
    const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
  } else {
    return *reinterpret_cast<const float4*>(p);
  }
}
template <bool NT>
__device__ __forceinline__ void state_store4(float* p, float a, float b, float c, float d) {
  if constexpr (NT) {
    const f32x4v v = {a, b, c, d};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4v*>(p));
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
}
template <bool NT>
__device__ __forceinline__ float state_load1(const float* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT>
__device__ __forceinline__ void state_store1(float* p, float v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <int N, bool BF16, bool VEC, bool HAS_Z, bool NT, typename Idx>
__global__ void __launch_bounds__(kBlock)
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
  constexpr bool VEC_STATE = VEC && NPL % 4 == 0;
  constexpr bool VEC_BC = VEC && (BF16 ? NPL >= 2 : true);
  const Idx dim = (Idx)s.dim;
  const Idx rows = (Idx)s.batch * dim;
  // channels per B/C group (one group: no division)
  const Idx cpg = s.ngroups > 1 ? dim / (Idx)s.ngroups : dim;
  const Idx first = (Idx)blockIdx.x * (kBlock * kItems) +
                    (Idx)(threadIdx.x >> 6) * (kLanes * kItems) + (threadIdx.x & (kLanes - 1));

  // ---- loads of every item, issued before any use
  Idx r[kItems], d[kItems];
  int n0[kItems];
  bool active[kItems];
  float h[kItems][NPL], a[kItems][NPL], bv[kItems][NPL], cv[kItems][NPL];
  float xv[kItems], dtv[kItems], zv[kItems], Dd[kItems], bb[kItems];
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const Idx v = first + (Idx)it * kLanes;
    const Idx r_raw = v / LPR;
    active[it] = r_raw < rows;
    // lanes past the last row still take part in the cross-lane sum, on the
    // last row, and store nothing
    r[it] = active[it] ? r_raw : rows - 1;
    n0[it] = (int)(v % LPR) * NPL;
    Idx b;
    if constexpr (sizeof(Idx) == 4)
      b = udiv(r[it], s.dim_div);
    else
      b = r[it] / dim;
    d[it] = r[it] - b * dim;
    const Idx grp = s.ngroups > 1 ? d[it] / cpg : (Idx)0;
    const Idx bc = (b * (Idx)s.ngroups + grp) * N + n0[it];  // this lane's B, C
    const float* sp = state + r[it] * N + n0[it];
    const float* ap = A + d[it] * N + n0[it];
    if constexpr (VEC_STATE) {
#pragma unroll
      for (int q = 0; q < NPL / 4; ++q) {
        const float4 hv = state_load4<NT>(sp + 4 * q);
        const float4 av = reinterpret_cast<const float4*>(ap)[q];
        h[it][4 * q] = hv.x; h[it][4 * q + 1] = hv.y; h[it][4 * q + 2] = hv.z; h[it][4 * q + 3] = hv.w;
        a[it][4 * q] = av.x; a[it][4 * q + 1] = av.y; a[it][4 * q + 2] = av.z; a[it][4 * q + 3] = av.w;
      }
    } else {
#pragma unroll
      for (int n = 0; n < NPL; ++n) {
        h[it][n] = state_load1<NT>(sp + n);
        a[it][n] = ap[n];
      }
    }
    // B and C are the same for every row of a group; read as 16- or 8-byte
    // pieces where the layout allows
    if constexpr (VEC_BC) {
      Raw<BF16, NPL> rb, rc;
      load_chunk<BF16, true, NPL>(rb, Bm, (int64_t)bc, NPL);
      load_chunk<BF16, true, NPL>(rc, Cm, (int64_t)bc, NPL);
#pragma unroll
      for (int n = 0; n < NPL; ++n) {
        bv[it][n] = raw_get(rb, n);
        cv[it][n] = raw_get(rc, n);
      }
    } else {
#pragma unroll
      for (int n = 0; n < NPL; ++n) {
        bv[it][n] = load_io<BF16>(Bm, (int64_t)(bc + n));
        cv[it][n] = load_io<BF16>(Cm, (int64_t)(bc + n));
      }
    }
    xv[it] = load_io<BF16>(x, (int64_t)r[it]);
    dtv[it] = load_io<BF16>(dt, (int64_t)r[it]);
    zv[it] = HAS_Z ? load_io<BF16>(z, (int64_t)r[it]) : 0.0f;
    Dd[it] = Dv ? Dv[d[it]] : 0.0f;
    bb[it] = bias ? bias[d[it]] : 0.0f;
  }

  // ---- the step
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const float xr = dtv[it] + bb[it];
    const float dl = s.softplus ? softplus_f32(xr) : xr;
    const float w = dl * xv[it];
    float y = 0.0f;
#pragma unroll
    for (int n = 0; n < NPL; ++n) {
      const float e = hw_exp2(dl * (a[it][n] * kLog2e));
      h[it][n] = fmaf(e, h[it][n], w * bv[it][n]);
      y = fmaf(cv[it][n], h[it][n], y);
    }
    y = row_sum<LPR>(y);
    y = fmaf(Dd[it], xv[it], y);
    if (HAS_Z) y *= silu_f32(zv[it]);

    if (!active[it]) continue;
    float* sp = state + r[it] * N + n0[it];
    if constexpr (VEC_STATE) {
#pragma unroll
      for (int q = 0; q < NPL / 4; ++q)
        state_store4<NT>(sp + 4 * q, h[it][4 * q], h[it][4 * q + 1], h[it][4 * q + 2],
                         h[it][4 * q + 3]);
    } else {
#pragma unroll
      for (int n = 0; n < NPL; ++n) state_store1<NT>(sp + n, h[it][n]);
    }
    if (n0[it] == 0) {
      if constexpr (BF16)
        static_cast<uint16_t*>(out)[r[it]] = to_bf16(y);
      else
        static_cast<float*>(out)[r[it]] = y;
    }
  }
}

template <int N, bool BF16, bool VEC, typename Idx>
hipError_t launch_u(const UpdateParams& p, hipStream_t stream) {
  UpdateShape s{p.batch, p.dim, p.softplus, p.ngroups > 1 ? p.ngroups : 1, U32Div{1u, 0u}};
  if (sizeof(Idx) == 4) s.dim_div = make_u32div((uint32_t)p.dim);
  const int64_t threads = p.batch * p.dim * kLanesPerRow<N>;
  const int64_t per_block = (int64_t)kBlock * kItems;
  const dim3 grid((unsigned)((threads + per_block - 1) / per_block));
#define MSSM_UPDATE_LAUNCH(Z, NT)                                                 \
  hipLaunchKernelGGL((state_update_kernel<N, BF16, VEC, Z, NT, Idx>), grid, dim3(kBlock), \
                     0, stream, p.state, p.x, p.dt, p.z, p.A, p.B, p.C, p.D, p.bias,  \
                     p.out, s)
  if (p.z) {
    if (p.stream_state) MSSM_UPDATE_LAUNCH(true, true);
    else MSSM_UPDATE_LAUNCH(true, false);
  } else {
    if (p.stream_state) MSSM_UPDATE_LAUNCH(false, true);
    else MSSM_UPDATE_LAUNCH(false, false);
  }
#undef MSSM_UPDATE_LAUNCH
  return hipGetLastError();
}

template <int N, bool BF16, bool VEC>
hipError_t launch_ui(const UpdateParams& p, hipStream_t stream) {
  // 32-bit indices when the largest index (state elements, or lane slots of
  // the grid) stays below 2^31
  const int64_t rows = p.batch * p.dim;
  const int64_t slots = rows * kLanesPerRow<N> + kBlock * kItems;
  const bool small = rows * N < (int64_t(1) << 31) && slots < (int64_t(1) << 31);
  return small ? launch_u<N, BF16, VEC, uint32_t>(p, stream)
               : launch_u<N, BF16, VEC, int64_t>(p, stream);
}

template <int N>
hipError_t launch_un(const UpdateParams& p, bool bf16, hipStream_t stream) {
  // 16-byte pieces: the state and A rows, and the B / C rows (their starts
  // are multiples of N values, so 16-byte aligned bases keep them aligned)
  const bool vec = ((uintptr_t)p.state % 16 == 0) && ((uintptr_t)p.A % 16 == 0) &&
                   ((uintptr_t)p.B % 16 == 0) && ((uintptr_t)p.C % 16 == 0);
  if (bf16)
    return vec ? launch_ui<N, true, true>(p, stream)
               : launch_ui<N, true, false>(p, stream);
  return vec ? launch_ui<N, false, true>(p, stream)
             : launch_ui<N, false, false>(p, stream);
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
