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
#include <type_traits>

#include "dev_math.h"
#include "mssm_internal.h"
#include "scan_common.h"

namespace mssm {
namespace {

constexpr int kChunk = 8;  // timesteps per thread
constexpr int kPrev = 4;   // inputs read before a chunk (>= K - 1)

// Idx: uint32_t when every element index fits in 31 bits (cheap division
// by the row length), else int64_t.  Every load of a thread is issued before
// the first use: the inputs before the chunk come from an address clamped
// into the row (unused at the row start, where init supplies them).
template <bool BF16, bool VEC, int K, typename Idx>
__global__ void __launch_bounds__(256)
    causal_conv1d_kernel(const void* __restrict__ x, const float* __restrict__ w,
                         const float* __restrict__ bias,
                         const void* __restrict__ init, void* __restrict__ out,
                         Idx rows, Idx dim, Idx L, int silu, U32Div per_row_div,
                         U32Div dim_div) {
  static_assert(K >= 1 && K - 1 <= kPrev, "width");
  const Idx per_row = (L + kChunk - 1) / kChunk;
  const Idx id = (Idx)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= rows * per_row) return;
  // 32-bit indices: the two divisions by kernel constants as multiplies
  Idx row, d;
  if constexpr (sizeof(Idx) == 4) {
    row = udiv(id, per_row_div);
    d = row - udiv(row, dim_div) * dim;
  } else {
    row = id / per_row;
    d = row % dim;
  }
  const Idx t0 = (id - row * per_row) * kChunk;
  const Idx off = row * L;

  Raw<BF16, kChunk> rx;
  Raw<BF16, kPrev> rp;
  load_chunk<BF16, VEC, kChunk>(rx, x, (int64_t)(off + t0), (int64_t)(L - t0));
  const Idx tp = t0 >= kPrev ? t0 - kPrev : 0;
  load_chunk<BF16, VEC, kPrev>(rp, x, (int64_t)(off + tp), (int64_t)(L - tp));
  float wk[K];
#pragma unroll
  for (int j = 0; j < K; ++j) wk[j] = w[d * K + j];
  const float b = bias ? bias[d] : 0.0f;

  float xs[kPrev + kChunk];
  if (t0 >= kPrev) {
#pragma unroll
    for (int j = 0; j < kPrev; ++j) xs[j] = raw_get(rp, j);
  } else {
    // t0 == 0: x[-(K-1)..-1] from init, older slots unused
#pragma unroll
    for (int j = 0; j < kPrev; ++j) xs[j] = 0.0f;
    if (init) {
#pragma unroll
      for (int j = 0; j < K - 1; ++j) {
        const Idx i = row * (K - 1) + j;
        xs[kPrev - (K - 1) + j] =
            BF16 ? bf16_bits(static_cast<const uint16_t*>(init)[i])
                 : static_cast<const float*>(init)[i];
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kChunk; ++k) xs[kPrev + k] = raw_get(rx, k);

  float o[kChunk];
#pragma unroll
  for (int k = 0; k < kChunk; ++k) {
    float v = b;
#pragma unroll
    for (int j = 0; j < K; ++j) v = fmaf(wk[j], xs[kPrev + k - (K - 1) + j], v);
    o[k] = silu ? silu_f32(v) : v;
  }
  store_chunk<BF16, VEC, kChunk>(out, (int64_t)(off + t0), o, (int64_t)(L - t0));
}

// The (batch, length, channel) layout: consecutive threads own consecutive
// channels of the same kChunk timesteps, so every load and store of a wave
// is one contiguous piece of a timestep's channels.
template <bool BF16, int K, typename Idx>
__global__ void __launch_bounds__(256)
    causal_conv1d_bld_kernel(const void* __restrict__ x, const float* __restrict__ w,
                             const float* __restrict__ bias,
                             const void* __restrict__ init, void* __restrict__ out,
                             Idx batch, Idx dim, Idx L, int silu) {
  using SIdx = typename std::make_signed<Idx>::type;
  const Idx chunks = (L + kChunk - 1) / kChunk;
  const Idx id = (Idx)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= batch * chunks * dim) return;
  const Idx d = id % dim;
  const Idx r = id / dim;
  const Idx c = r % chunks;
  const Idx b = r / chunks;
  const SIdx t0 = (SIdx)(c * kChunk);
  auto at = [&](SIdx t) -> float {  // x at step t of channel d, t >= -(K-1)
    if (t >= (SIdx)L) return 0.0f;
    if (t >= 0) {
      const Idx i = (b * L + (Idx)t) * dim + d;
      return BF16 ? bf16_bits(static_cast<const uint16_t*>(x)[i])
                  : static_cast<const float*>(x)[i];
    }
    if (!init) return 0.0f;
    const Idx i = (Idx)((SIdx)((b * dim + d) * (K - 1) + (K - 1)) + t);
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
    if (t0 + k >= (SIdx)L) break;
    float v = bb;
#pragma unroll
    for (int j = 0; j < K; ++j) v = fmaf(wk[j], xs[k + j], v);
    v = silu ? silu_f32(v) : v;
    const Idx i = (b * L + (Idx)t0 + k) * dim + d;
    if constexpr (BF16)
      static_cast<uint16_t*>(out)[i] = to_bf16(v);
    else
      static_cast<float*>(out)[i] = v;
  }
}

template <bool BF16, typename Idx>
hipError_t launch_bld(const ConvParams& p, hipStream_t st) {
  const int64_t chunks = (p.L + kChunk - 1) / kChunk;
  const int64_t threads = p.batch * chunks * p.dim;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  const Idx batch = (Idx)p.batch, dim = (Idx)p.dim, L = (Idx)p.L;
  switch (p.width) {
    case 2:
      hipLaunchKernelGGL((causal_conv1d_bld_kernel<BF16, 2, Idx>), grid, block, 0, st,
                         p.x, p.w, p.bias, p.init, p.out, batch, dim, L, p.silu);
      break;
    case 3:
      hipLaunchKernelGGL((causal_conv1d_bld_kernel<BF16, 3, Idx>), grid, block, 0, st,
                         p.x, p.w, p.bias, p.init, p.out, batch, dim, L, p.silu);
      break;
    case 4:
      hipLaunchKernelGGL((causal_conv1d_bld_kernel<BF16, 4, Idx>), grid, block, 0, st,
                         p.x, p.w, p.bias, p.init, p.out, batch, dim, L, p.silu);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16, bool VEC, typename Idx>
hipError_t launch_k(const ConvParams& p, hipStream_t st) {
  const int64_t per_row = (p.L + kChunk - 1) / kChunk;
  const int64_t threads = p.batch * p.dim * per_row;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  const Idx rows = (Idx)(p.batch * p.dim), dim = (Idx)p.dim, L = (Idx)p.L;
  const U32Div prd = sizeof(Idx) == 4 ? make_u32div((uint32_t)per_row) : U32Div{1u, 0u};
  const U32Div dd = sizeof(Idx) == 4 ? make_u32div((uint32_t)p.dim) : U32Div{1u, 0u};
  switch (p.width) {
    case 2:
      hipLaunchKernelGGL((causal_conv1d_kernel<BF16, VEC, 2, Idx>), grid, block, 0, st,
                         p.x, p.w, p.bias, p.init, p.out, rows, dim, L, p.silu, prd, dd);
      break;
    case 3:
      hipLaunchKernelGGL((causal_conv1d_kernel<BF16, VEC, 3, Idx>), grid, block, 0, st,
                         p.x, p.w, p.bias, p.init, p.out, rows, dim, L, p.silu, prd, dd);
      break;
    case 4:
      hipLaunchKernelGGL((causal_conv1d_kernel<BF16, VEC, 4, Idx>), grid, block, 0, st,
                         p.x, p.w, p.bias, p.init, p.out, rows, dim, L, p.silu, prd, dd);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Gradients of the convolution for dout = dLoss/dout (the training step of
// the conv-fed block: the scan's backward yields du, the gradient of this
// convolution's output).  With g[t] = dout[t] silu'(v[t]) (or dout[t]),
// silu'(v) = s (1 + v (1 - s)), s = sigmoid(v):
//   dx[s]    = sum_k w[d,k] g[s + (K-1) - k]     (over steps inside the row)
//   dinit[j] = sum_{k <= j} w[d,k] g[j - k]       (the values before t = 0)
//   dw[d,k]  = sum_{b,t} g[t] x[t-(K-1)+k],  dbias[d] = sum_{b,t} g[t].
// One workgroup per channel, so the channel sums need no second pass and
// are added in a fixed order (repeated calls give the same bits): each
// thread owns 8 consecutive steps of a row (16-byte pieces, as in the
// forward), walks the batch and the row in strides of 256 chunks, keeps its
// partial sums in registers, and the workgroup adds them in a tree.  A
// thread recomputes v (hence g) for its 8 steps and the K-1 after them, so
// it reads x from 4 steps before its chunk to 4 after, and dout to 4 after.
template <bool BF16, bool VEC, int K>
__global__ void __launch_bounds__(256)
    causal_conv1d_bwd_kernel(const void* __restrict__ x, const float* __restrict__ w,
                             const float* __restrict__ bias, const void* __restrict__ init,
                             const void* __restrict__ dout, void* __restrict__ dx,
                             float* __restrict__ dw, float* __restrict__ dbias,
                             void* __restrict__ dinit, int64_t batch, int64_t dim,
                             int64_t L, int silu) {
  static_assert(K >= 1 && K - 1 <= kPrev, "width");
  constexpr int kNext = 4;  // steps after a chunk (>= K - 1)
  const int64_t d = blockIdx.x;
  const int tid = threadIdx.x;
  float wk[K];
#pragma unroll
  for (int j = 0; j < K; ++j) wk[j] = w[d * K + j];
  const float bv = bias ? bias[d] : 0.0f;
  float pw[K], pb = 0.0f;
#pragma unroll
  for (int j = 0; j < K; ++j) pw[j] = 0.0f;

  for (int64_t b = 0; b < batch; ++b) {
    const int64_t row = b * dim + d;
    const int64_t off = row * L;
    for (int64_t t0 = (int64_t)tid * kChunk; t0 < L; t0 += 256 * kChunk) {
      Raw<BF16, kChunk> rx, rg;
      Raw<BF16, kPrev> rp;
      Raw<BF16, kNext> rxn, rgn;
      load_chunk<BF16, VEC, kChunk>(rx, x, off + t0, L - t0);
      load_chunk<BF16, VEC, kChunk>(rg, dout, off + t0, L - t0);
      load_chunk<BF16, VEC, kNext>(rxn, x, off + t0 + kChunk, L - t0 - kChunk);
      load_chunk<BF16, VEC, kNext>(rgn, dout, off + t0 + kChunk, L - t0 - kChunk);
      if (t0 >= kPrev) load_chunk<BF16, VEC, kPrev>(rp, x, off + t0 - kPrev, kPrev);
      // x over [t0 - 4, t0 + 12): before the row from init (or 0)
      float xs[kPrev + kChunk + kNext];
      if (t0 >= kPrev) {
#pragma unroll
        for (int j = 0; j < kPrev; ++j) xs[j] = raw_get(rp, j);
      } else {
#pragma unroll
        for (int j = 0; j < kPrev; ++j) xs[j] = 0.0f;
        if (init) {
#pragma unroll
          for (int j = 0; j < K - 1; ++j) {
            const int64_t i = row * (K - 1) + j;
            xs[kPrev - (K - 1) + j] = BF16 ? bf16_bits(static_cast<const uint16_t*>(init)[i])
                                           : static_cast<const float*>(init)[i];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kChunk; ++j) xs[kPrev + j] = raw_get(rx, j);
#pragma unroll
      for (int j = 0; j < kNext; ++j) xs[kPrev + kChunk + j] = raw_get(rxn, j);
      // g over [t0, t0 + 8 + K - 1); steps past the row have dout = 0
      constexpr int NG = kChunk + K - 1;
      float gs[NG];
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        const float go = j < kChunk ? raw_get(rg, j) : raw_get(rgn, j - kChunk);
        float v = bv;
#pragma unroll
        for (int k = 0; k < K; ++k) v = fmaf(wk[k], xs[kPrev + j - (K - 1) + k], v);
        float gv = go;
        if (silu) {
          const float sg = hw_rcp(1.0f + hw_exp2(-v * kLog2e));
          gv = go * (sg * fmaf(v, 1.0f - sg, 1.0f));
        }
        gs[j] = gv;
      }
      float o[kChunk];
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        float a = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) a = fmaf(wk[k], gs[i + (K - 1) - k], a);
        o[i] = a;
        pb += gs[i];
#pragma unroll
        for (int k = 0; k < K; ++k) pw[k] = fmaf(gs[i], xs[kPrev + i - (K - 1) + k], pw[k]);
      }
      store_chunk<BF16, VEC, kChunk>(dx, off + t0, o, L - t0);
      if (t0 == 0 && dinit) {
#pragma unroll
        for (int j = 0; j < K - 1; ++j) {
          float a = 0.0f;
#pragma unroll
          for (int k = 0; k <= j; ++k) a = fmaf(wk[k], gs[j - k], a);
          const int64_t i = row * (K - 1) + j;
          if constexpr (BF16)
            static_cast<uint16_t*>(dinit)[i] = to_bf16(a);
          else
            static_cast<float*>(dinit)[i] = a;
        }
      }
    }
  }

  // channel sums: the workgroup's partials added in a fixed tree
  __shared__ float red[K + 1][256];
#pragma unroll
  for (int k = 0; k < K; ++k) red[k][tid] = pw[k];
  red[K][tid] = pb;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) {
#pragma unroll
      for (int k = 0; k <= K; ++k) red[k][tid] += red[k][tid + st];
    }
    __syncthreads();
  }
  if (tid <= K) {
    if (tid < K)
      dw[d * K + tid] = red[tid][0];
    else if (dbias)
      dbias[d] = red[K][0];
  }
}

template <bool BF16, bool VEC>
hipError_t launch_bwd_k(const ConvBwdParams& p, hipStream_t st) {
  const dim3 grid((unsigned)p.dim), block(256);
#define MSSM_CONV_BWD(KW)                                                                   \
  hipLaunchKernelGGL((causal_conv1d_bwd_kernel<BF16, VEC, KW>), grid, block, 0, st, p.x, \
                     p.w, p.bias, p.init, p.dout, p.dx, p.dw, p.dbias, p.dinit, p.batch,  \
                     p.dim, p.L, p.silu)
  switch (p.width) {
    case 2: MSSM_CONV_BWD(2); break;
    case 3: MSSM_CONV_BWD(3); break;
    case 4: MSSM_CONV_BWD(4); break;
    default: return hipErrorInvalidValue;
  }
#undef MSSM_CONV_BWD
  return hipGetLastError();
}

// 32-bit indices when every element index (and the grid's thread index, a
// chunk of kChunk elements per thread) stays below 2^31.
bool small_indices(const ConvParams& p) {
  const int64_t elems = p.batch * p.dim * (p.L + kChunk);
  return elems + 256 * kChunk < (int64_t(1) << 31);
}

}  // namespace

hipError_t launch_causal_conv1d_bwd(const ConvBwdParams& p, bool bf16, bool vec,
                                    hipStream_t st) {
  if (bf16) return vec ? launch_bwd_k<true, true>(p, st) : launch_bwd_k<true, false>(p, st);
  return vec ? launch_bwd_k<false, true>(p, st) : launch_bwd_k<false, false>(p, st);
}

hipError_t launch_causal_conv1d(const ConvParams& p, bool bf16, bool vec,
                                hipStream_t st) {
  if (small_indices(p)) {
    if (p.layout_bld)
      return bf16 ? launch_bld<true, uint32_t>(p, st) : launch_bld<false, uint32_t>(p, st);
    if (bf16)
      return vec ? launch_k<true, true, uint32_t>(p, st) : launch_k<true, false, uint32_t>(p, st);
    return vec ? launch_k<false, true, uint32_t>(p, st) : launch_k<false, false, uint32_t>(p, st);
  }
  if (p.layout_bld)
    return bf16 ? launch_bld<true, int64_t>(p, st) : launch_bld<false, int64_t>(p, st);
  if (bf16)
    return vec ? launch_k<true, true, int64_t>(p, st) : launch_k<true, false, int64_t>(p, st);
  return vec ? launch_k<false, true, int64_t>(p, st) : launch_k<false, false, int64_t>(p, st);
}

}  // namespace mssm
