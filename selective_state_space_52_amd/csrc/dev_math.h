// dev_math.h -- fp32 device helpers for gfx950: bf16 unpack/pack, softplus,
// silu, built on the hardware exp2 / log2 / reciprocal (v_exp_f32,
// v_log_f32, v_rcp_f32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_bits(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo;
  __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ uint16_t to_bf16(float f) {
  __bf16 a = (__bf16)f;
  return __builtin_bit_cast(uint16_t, a);
}

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^-|x|).
// With e = e^-|x| in (0, 1]: for e < 1/16 a five-term series of log1p
// (truncation below 2e-7 relative, from the e^6/6 term); otherwise
// log2(1 + e) * ln 2, where the rounding of 1 + e costs at most 1.5e-6
// relative because log1p(e) >= 0.06 there.  No threshold on large x is
// needed: e underflows smoothly and the series returns e.
__device__ __forceinline__ float softplus_f32(float x) {
  const float e = hw_exp2(-fabsf(x) * kLog2e);
  const float ser = e * (1.0f - e * (0.5f - e * (0.33333334f - e * (0.25f - e * 0.2f))));
  const float lg = hw_log2(1.0f + e) * kLn2;
  return fmaxf(x, 0.0f) + (e < 0.0625f ? ser : lg);
}

// silu(z) = z / (1 + e^-z); e^-z overflows to +inf for very negative z and
// the reciprocal then returns 0, which is the right limit.
__device__ __forceinline__ float silu_f32(float z) {
  return z * hw_rcp(1.0f + hw_exp2(-z * kLog2e));
}

}  // namespace mssm
