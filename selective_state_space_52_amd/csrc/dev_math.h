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

// Two fp32 -> packed bf16 pair, round to nearest even: converted as one
// two-element vector, so both halves go through a single v_cvt_pk_bf16_f32
// (element-wise conversions and a shift/or cost four instructions).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint16_t to_bf16(float f) {
  __bf16 a = (__bf16)f;
  return __builtin_bit_cast(uint16_t, a);
}

// n / d for n < 2^31 and 1 <= d < 2^31 as (n * magic) >> shift (division by
// an invariant integer, Granlund and Montgomery, 1994): with l = ceil(log2 d),
// shift = 31 + l and magic = ceil(2^shift / d), the error magic * d - 2^shift
// is below d <= 2^l, so n * magic / 2^shift overshoots n / d by less than
// 1 / d and its floor is exact.  magic < 2^32.  Set up on the host.
struct U32Div {
  uint32_t magic, shift;
};
inline U32Div make_u32div(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t p2 = uint64_t(1) << (31 + l);
  return U32Div{(uint32_t)((p2 + d - 1) / d), 31 + l};
}
__device__ __forceinline__ uint32_t udiv(uint32_t n, U32Div v) {
  return (uint32_t)(((uint64_t)n * v.magic) >> v.shift);
}

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^-|x|).
// With e = e^-|x| in (0, 1] and u = 1 + e rounded to fp32, c = e - (u - 1)
// is the rounding error of u, exactly (|e| <= 1, so the two subtractions are
// exact), and log1p(e) = log(u) + log(1 + c / u) = log(u) + c to within
// |c| e, i.e. below 6e-8 relative.  v_log_f32 measured at most 1.2e-7
// relative error on every u = 1 + k 2^-23 in [1, 2), so the form is accurate
// for tiny e as well, without a series branch.  No threshold on large x is
// needed: e underflows smoothly and log1p(e) = c = e there.
__device__ __forceinline__ float softplus_f32(float x) {
  const float e = hw_exp2(-fabsf(x) * kLog2e);
  const float u = 1.0f + e;
  const float c = e - (u - 1.0f);
  return fmaxf(x, 0.0f) + fmaf(hw_log2(u), kLn2, c);
}

// silu(z) = z / (1 + e^-z); e^-z overflows to +inf for very negative z and
// the reciprocal then returns 0, which is the right limit.
__device__ __forceinline__ float silu_f32(float z) {
  return z * hw_rcp(1.0f + hw_exp2(-z * kLog2e));
}

}  // namespace mssm
