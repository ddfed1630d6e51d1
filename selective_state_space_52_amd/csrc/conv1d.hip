// conv1d.hip -- causal depthwise convolution over time (the Mamba block's
// local convolution ahead of the scan) for gfx950.
//
// Per (batch b, channel d) row, width K (the pages' d_conv = 4; page "Mamba
// State Space Model", model construction, and page "Mamba: Selective State
// Space Models", "Quick Start"):
//   v[t] = bias[d] + sum_{k=0}^{K-1} w[d,k] x[t-(K-1)+k],  x[t<0] = init or 0
//   out[t] = silu(v[t])  (or v[t])
//
// The op moves 2 io values per element and does K fmas and a silu, so it is
// bound by HBM.  With rows stored time-fastest, (batch, dim, L), each thread
// owns 8 consecutive timesteps of one row (16 bytes of bf16), so a wave reads
// and writes 1 KB contiguous pieces of a row; the K-1 inputs before a
// thread's chunk are read again from the previous piece (an L2 hit).
#include "dev_math.h"
#include "mssm_internal.h"
#include "scan_common.h"

namespace mssm {
namespace {

constexpr int kChunk = 8;  // timesteps per thread
constexpr int kPrev = 4;   // inputs read before a chunk (>= K - 1)

template <bool BF16, bool VEC, int K>
__global__ void __launch_bounds__(256)
    causal_conv1d_kernel(const void* __restrict__ x, const float* __restrict__ w,
                         const float* __restrict__ bias,
                         const void* __restrict__ init, void* __restrict__ out,
                         int64_t rows, int64_t dim, int64_t L, int silu) {
  static_assert(K >= 1 && K - 1 <= kPrev, "width");
  const int64_t per_row = (L + kChunk - 1) / kChunk;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= rows * per_row) return;
  const int64_t row = id / per_row;
  const int64_t t0 = (id - row * per_row) * kChunk;
  const int64_t d = row % dim;
  const int64_t off = row * L;

  Raw<BF16, kChunk> rx;
  load_chunk<BF16, VEC, kChunk>(rx, x, off + t0, L - t0);
  float xs[kPrev + kChunk];
  if (t0 >= kPrev) {
    Raw<BF16, kPrev> rp;
    load_chunk<BF16, VEC, kPrev>(rp, x, off + t0 - kPrev, kPrev);
#pragma unroll
    for (int j = 0; j < kPrev; ++j) xs[j] = raw_get(rp, j);
  } else {
    // t0 == 0: x[-(K-1)..-1] from init, older slots unused
#pragma unroll
    for (int j = 0; j < kPrev; ++j) xs[j] = 0.0f;
    if (init) {
#pragma unroll
      for (int j = 0; j < K - 1; ++j) {
        const int64_t i = row * (K - 1) + j;
        xs[kPrev - (K - 1) + j] =
            BF16 ? bf16_bits(static_cast<const uint16_t*>(init)[i])
                 : static_cast<const float*>(init)[i];
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kChunk; ++k) xs[kPrev + k] = raw_get(rx, k);

  float wk[K];
#pragma unroll
  for (int j = 0; j < K; ++j) wk[j] = w[d * K + j];
  const float b = bias ? bias[d] : 0.0f;
  float o[kChunk];
#pragma unroll
  for (int k = 0; k < kChunk; ++k) {
    float v = b;
#pragma unroll
    for (int j = 0; j < K; ++j) v = fmaf(wk[j], xs[kPrev + k - (K - 1) + j], v);
    o[k] = silu ? silu_f32(v) : v;
  }
  store_chunk<BF16, VEC, kChunk>(out, off + t0, o, L - t0);
}

// The (batch, length, channel) layout: consecutive threads own consecutive
// channels of the same kChunk timesteps, so every load and store of a wave
// is one contiguous piece of a timestep's channels.
template <bool BF16, int K>
__global__ void __launch_bounds__(256)
    causal_conv1d_bld_kernel(const void* __restrict__ x, const float* __restrict__ w,
                             const float* __restrict__ bias,
                             const void* __restrict__ init, void* __restrict__ out,
                             int64_t batch, int64_t dim, int64_t L, int silu) {
  const int64_t chunks = (L + kChunk - 1) / kChunk;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= batch * chunks * dim) return;
  const int64_t d = id % dim;
  const int64_t r = id / dim;
  const int64_t c = r % chunks;
  const int64_t b = r / chunks;
  const int64_t t0 = c * kChunk;
  auto at = [&](int64_t t) -> float {  // x at step t of channel d, t >= -(K-1)
    if (t >= L) return 0.0f;
    if (t >= 0) {
      const int64_t i = (b * L + t) * dim + d;
      return BF16 ? bf16_bits(static_cast<const uint16_t*>(x)[i])
                  : static_cast<const float*>(x)[i];
    }
    if (!init) return 0.0f;
    const int64_t i = (b * dim + d) * (K - 1) + (K - 1) + t;
    return BF16 ? bf16_bits(static_cast<const uint16_t*>(init)[i])
                : static_cast<const float*>(init)[i];
  };
  float xs[kChunk + K - 1];
#pragma unroll
  for (int j = 0; j < kChunk + K - 1; ++j) xs[j] = at(t0 - (K - 1) + j);
  float wk[K];
#pragma unroll
  for (int j = 0; j < K; ++j) wk[j] = w[d * K + j];
  const float bb = bias ? bias[d] : 0.0f;
#pragma unroll
  for (int k = 0; k < kChunk; ++k) {
    if (t0 + k >= L) break;
    float v = bb;
#pragma unroll
    for (int j = 0; j < K; ++j) v = fmaf(wk[j], xs[k + j], v);
    v = silu ? silu_f32(v) : v;
    const int64_t i = (b * L + t0 + k) * dim + d;
    if constexpr (BF16)
      static_cast<uint16_t*>(out)[i] = to_bf16(v);
    else
      static_cast<float*>(out)[i] = v;
  }
}

template <bool BF16>
hipError_t launch_bld(const ConvParams& p, hipStream_t st) {
  const int64_t chunks = (p.L + kChunk - 1) / kChunk;
  const int64_t threads = p.batch * chunks * p.dim;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  switch (p.width) {
    case 2:
      hipLaunchKernelGGL((causal_conv1d_bld_kernel<BF16, 2>), grid, block, 0, st, p.x,
                         p.w, p.bias, p.init, p.out, p.batch, p.dim, p.L, p.silu);
      break;
    case 3:
      hipLaunchKernelGGL((causal_conv1d_bld_kernel<BF16, 3>), grid, block, 0, st, p.x,
                         p.w, p.bias, p.init, p.out, p.batch, p.dim, p.L, p.silu);
      break;
    case 4:
      hipLaunchKernelGGL((causal_conv1d_bld_kernel<BF16, 4>), grid, block, 0, st, p.x,
                         p.w, p.bias, p.init, p.out, p.batch, p.dim, p.L, p.silu);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16, bool VEC>
hipError_t launch_k(const ConvParams& p, hipStream_t st) {
  const int64_t per_row = (p.L + kChunk - 1) / kChunk;
  const int64_t threads = p.batch * p.dim * per_row;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  const int64_t rows = p.batch * p.dim;
  switch (p.width) {
    case 2:
      hipLaunchKernelGGL((causal_conv1d_kernel<BF16, VEC, 2>), grid, block, 0, st,
                         p.x, p.w, p.bias, p.init, p.out, rows, p.dim, p.L, p.silu);
      break;
    case 3:
      hipLaunchKernelGGL((causal_conv1d_kernel<BF16, VEC, 3>), grid, block, 0, st,
                         p.x, p.w, p.bias, p.init, p.out, rows, p.dim, p.L, p.silu);
      break;
    case 4:
      hipLaunchKernelGGL((causal_conv1d_kernel<BF16, VEC, 4>), grid, block, 0, st,
                         p.x, p.w, p.bias, p.init, p.out, rows, p.dim, p.L, p.silu);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_causal_conv1d(const ConvParams& p, bool bf16, bool vec,
                                hipStream_t st) {
  if (p.layout_bld) return bf16 ? launch_bld<true>(p, st) : launch_bld<false>(p, st);
  if (bf16) return vec ? launch_k<true, true>(p, st) : launch_k<true, false>(p, st);
  return vec ? launch_k<false, true>(p, st) : launch_k<false, false>(p, st);
}

}  // namespace mssm
