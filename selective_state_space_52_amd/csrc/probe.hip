// probe.hip -- issue-rate probes of the vector ALU, for the scan's ALU
// roofline.  The selective scan spends one v_exp_f32 and four fp32 mul/fma
// per state element (exp(Delta A), Delta u B, the state update and the C
// readout); these kernels time those instructions alone and in the scan's
// mix, so that the ceiling the bench reports is measured on the chip rather
// than taken from a datasheet rate.
//
// Each thread runs `iters` iterations over independent chains, so issue,
// not latency, sets the rate (the launch gives every SIMD several waves):
//   kind 0: 8 v_fma_f32 per iteration (8 chains);
//   kind 1: 8 v_exp_f32 per iteration (8 chains, input -|x| so every value
//           stays in (0, 1]);
//   kind 3: the same 4 state elements per iteration as an inclusive
//           associative scan of (decay, drive) pairs over the wave's 64 lanes
//           (one timestep per lane, six DPP levels), the chunk carry and the
//           readout (see below);
//   kind 4: 8 v_fma_f32 and 2 v_exp_f32 per iteration on independent chains
//           (no value passes between the fma and the exp chains), so that its
//           rate against kinds 0 and 1 shows whether the exponentials overlap
//           the multiply-adds or take their issue slots;
//   kind 2: the state-element mix, 4 state elements per iteration, each
//           v_mul (Delta A) + v_exp + v_mul (Delta u B) + v_fma (state) +
//           a readout multiply-add (the first a v_mul), plus one v_mul that
//           derives the next iteration's Delta from the readout (Delta u is
//           half the readout, folded into the B constants): 21 instructions
//           per iteration, 4 of them v_exp_f32, for iters a multiple of 4
//           (the loop is unrolled by 4; a remainder adds a few moves).
// Every thread writes one value to sink, so nothing is optimised away.
#include "dev_math.h"
#include "mssm_internal.h"

namespace mssm {

// One level of an inclusive scan of (a, b) pairs across lanes: the pair of
// an earlier lane (DPP control CTRL, rows in ROW_MASK; other lanes see the
// identity (1, 0)) is combined in front of this lane's.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void scan_level(float& a, float& b) {
  const float ap = __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(a), CTRL, ROW_MASK, 0xF, false));
  const float bp = __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(b), CTRL, ROW_MASK, 0xF, false));
  b = fmaf(a, bp, b);
  a = a * ap;
}

template <int KIND>
__global__ void __launch_bounds__(256) valu_probe_kernel(float* __restrict__ sink, int iters,
                                                         float seed) {
  const float s0 = seed + 1e-3f * (float)(threadIdx.x & 63);
  float r = 0.0f;
  if constexpr (KIND == 0) {
    float c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = s0 + (float)j;
#pragma unroll 4
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = fmaf(c[j], 0.999f, 1e-3f);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) r += c[j];
  } else if constexpr (KIND == 1) {
    float c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = s0 + (float)j;
#pragma unroll 4
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = hw_exp2(-fabsf(c[j]));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) r += c[j];
  } else if constexpr (KIND == 4) {
    float c[8], x[2];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = s0 + (float)j;
    x[0] = s0;
    x[1] = s0 + 0.5f;
#pragma unroll 4
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j) x[j] = hw_exp2(-fabsf(x[j]));
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = fmaf(c[j], 0.999f, 1e-3f);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) r += c[j];
    r += x[0] + x[1];
  } else if constexpr (KIND == 3) {
    // The same recurrence as an inclusive associative scan over a wave's 64
    // timesteps (lane = timestep), per state: a = exp(Delta A), b = Delta u B,
    // six levels of (a, b) o (a', b') = (a a', a' b + b') combining each lane
    // with an earlier one through DPP (row shifts by 1, 2, 4, 8 within rows of
    // 16 lanes, then the last lane of a row broadcast to the next row(s)),
    // then the chunk's entering state and the readout:
    //   h = a_cum h_in + b_cum,  y += C h.
    float a0[4], bb[4], cc[4], hin[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a0[j] = -(float)(j + 1) * kLog2e;
      bb[j] = 0.25f * (float)(j + 1);
      cc[j] = 0.5f - 0.1f * (float)j;
      hin[j] = 0.01f * (float)j;
    }
    float x = 0.1f * s0, y = s0, acc = 0.0f;
    for (int i = 0; i < iters; ++i) {
      float yv = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float a = hw_exp2(x * a0[j]);
        float b = y * bb[j];
        scan_level<0x111, 0xF>(a, b);  // row_shr:1
        scan_level<0x112, 0xF>(a, b);  // row_shr:2
        scan_level<0x114, 0xF>(a, b);  // row_shr:4
        scan_level<0x118, 0xF>(a, b);  // row_shr:8
        scan_level<0x142, 0xA>(a, b);  // row_bcast:15 into rows 1 and 3
        scan_level<0x143, 0xC>(a, b);  // row_bcast:31 into rows 2 and 3
        const float h = fmaf(a, hin[j], b);
        yv = fmaf(cc[j], h, yv);
        // the chunk's end state (lane 63) enters the next chunk
        hin[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h), 63));
      }
      acc += yv;
      x = fabsf(yv) * 0.125f;
      y = yv * 0.5f;
    }
    r = acc;
  } else {
    // per-lane "A" and "B, C" of 4 states; x plays Delta, y plays Delta u
    float a[4], bb[4], cc[4], h[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[j] = -(float)(j + 1) * kLog2e;
      bb[j] = 0.25f * (float)(j + 1);
      cc[j] = 0.5f - 0.1f * (float)j;
      h[j] = 0.0f;
    }
    float x = 0.1f * s0, y = s0, acc = 0.0f;
#pragma unroll 4
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = hw_exp2(x * a[j]);
        h[j] = fmaf(e, h[j], y * bb[j]);
      }
      acc = cc[0] * h[0];
#pragma unroll
      for (int j = 1; j < 4; ++j) acc = fmaf(cc[j], h[j], acc);
      x = fabsf(acc) * 0.125f;
      y = acc * 0.5f;
    }
    r = acc;
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
}

hipError_t launch_valu_probe(int kind, int blocks, int iters, float* sink,
                             hipStream_t stream) {
  const dim3 grid((unsigned)blocks), block(256);
  switch (kind) {
    case 0: hipLaunchKernelGGL(valu_probe_kernel<0>, grid, block, 0, stream, sink, iters, 0.5f); break;
    case 1: hipLaunchKernelGGL(valu_probe_kernel<1>, grid, block, 0, stream, sink, iters, 0.5f); break;
    case 2: hipLaunchKernelGGL(valu_probe_kernel<2>, grid, block, 0, stream, sink, iters, 0.5f); break;
    case 3: hipLaunchKernelGGL(valu_probe_kernel<3>, grid, block, 0, stream, sink, iters, 0.5f); break;
    default: hipLaunchKernelGGL(valu_probe_kernel<4>, grid, block, 0, stream, sink, iters, 0.5f); break;
  }
  return hipGetLastError();
}

}  // namespace mssm
