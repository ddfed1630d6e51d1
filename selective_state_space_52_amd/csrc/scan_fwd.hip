// scan_fwd.hip -- the forward scan's non-template parts: the B/C pack, the
// work split helpers and the dispatch over state sizes (whose kernels are
// instantiated in scan_fwd_n*.hip).
#include "scan_fwd_impl.h"

namespace mssm {
namespace fwd {

// Writes the packed runs of `steps` timesteps per wave (steps >= L; the
// timesteps from L on are written as zeros) with `run_words` words per run.
// The source is bf16 or fp32 (src_bf16); the runs keep bf16 (dst_bf16) or
// hold fp32.  B and C are (batch, L, groups, N), or with state_major
// (batch, groups, N, L).  Threads i < nflags also zero flags[i]: the scan
// launch that follows on the same stream finds its summary flags cleared,
// with no separate fill.
__global__ void __launch_bounds__(256)
    bc_pack_kernel(const void* __restrict__ Bm, const void* __restrict__ Cm,
                   void* __restrict__ packed, int64_t batch, int64_t groups,
                   int64_t L, int64_t steps, int N, int NG, int src_bf16,
                   int dst_bf16, int64_t run_words, uint32_t* __restrict__ flags,
                   int64_t nflags, int state_major) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nflags) flags[i] = 0u;
  const int64_t total = batch * groups * steps * 2 * N;
  if (i >= total) return;
  const int npw = N / NG;
  // i indexes the values in order [b][group][wave][t][j], j < 2*npw
  const int j = (int)(i % (2 * npw));
  const int64_t r = i / (2 * npw);
  const int64_t t = r % steps;
  const int64_t bg = r / steps;           // run: (b * groups + group) * NG + wave
  const int g = (int)(bg % NG);
  const int64_t bgrp = bg / NG;
  const int64_t grp = bgrp % groups;
  const int64_t b = bgrp / groups;
  const int n = g * npw + (j < npw ? j : j - npw);
  const int64_t src = state_major ? ((b * groups + grp) * N + n) * L + t
                                  : ((b * L + t) * groups + grp) * N + n;
  const void* m = j < npw ? Bm : Cm;
  const int64_t vals_per_word = dst_bf16 ? 2 : 1;
  const int64_t dst = bg * run_words * vals_per_word + t * 2 * npw + j;
  if (dst_bf16) {
    static_cast<uint16_t*>(packed)[dst] =
        t < L ? static_cast<const uint16_t*>(m)[src] : (uint16_t)0;
  } else {
    float v = 0.0f;
    if (t < L)
      v = src_bf16 ? bf16_bits(static_cast<const uint16_t*>(m)[src])
                   : static_cast<const float*>(m)[src];
    static_cast<float*>(packed)[dst] = v;
  }
}


// The same runs for bf16 token-major B and C, NPW (even) states per wave:
// one thread per (run, token), in run-major order, so a wave's stores are
// one contiguous stretch of a run.  It reads the NPW / 2 words of its wave's
// states from the token's B row and from its C row and writes them as one
// piece of NPW words.  32-bit indices (the host checks the sizes); the
// divisions by the token count and the group count are multiplies by
// precomputed reciprocals.
template <int NPW>
__global__ void __launch_bounds__(256)
    bc_pack_tokens_kernel(const uint32_t* __restrict__ Bw, const uint32_t* __restrict__ Cw,
                          uint32_t* __restrict__ packed, uint32_t total, uint32_t steps,
                          U32Div steps_div, uint32_t L, uint32_t groups, U32Div groups_div,
                          uint32_t ng_log2, uint32_t run_words, uint32_t* __restrict__ flags,
                          uint32_t nflags) {
  static_assert(NPW % 2 == 0 && NPW <= 16, "whole bf16 pairs, at most a 64-byte piece");
  constexpr int H = NPW / 2;  // words of B (and of C) per wave and token
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nflags) flags[i] = 0u;
  if (i >= total) return;
  const uint32_t run = udiv(i, steps_div);
  const uint32_t t = i - run * steps;
  const uint32_t g = run & ((1u << ng_log2) - 1u);
  const uint32_t bgrp = run >> ng_log2;
  const uint32_t b = udiv(bgrp, groups_div);
  const uint32_t grp = bgrp - b * groups;
  const uint32_t ng = 1u << ng_log2;
  uint32_t v[NPW];
  if (t < L) {
    // words of the token's row: (b, t, grp) rows of N = NPW * ng values
    const uint32_t src = ((b * L + t) * groups + grp) * (H * ng) + g * H;
#pragma unroll
    for (int j = 0; j < H; ++j) {
      v[j] = Bw[src + j];
      v[H + j] = Cw[src + j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < NPW; ++j) v[j] = 0u;
  }
  uint32_t* dst = packed + run * run_words + t * NPW;
  if constexpr (NPW == 2) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(v[0], v[1]);
  } else {
#pragma unroll
    for (int j = 0; j < NPW; j += 4)
      *reinterpret_cast<uint4*>(dst + j) = make_uint4(v[j], v[j + 1], v[j + 2], v[j + 3]);
  }
}

}  // namespace fwd

hipError_t launch_bc_pack(const void* B, const void* C, void* packed,
                          int64_t batch, int64_t groups, int64_t L, int64_t steps,
                          int N, int waves, bool src_bf16, bool dst_bf16,
                          int64_t run_words, uint32_t* flags, int64_t nflags,
                          bool state_major, hipStream_t stream) {
  const int npw = N / waves;
  const int64_t tokens = batch * groups * steps * waves;  // (run, token) pairs
  const bool pow2 = waves > 0 && (waves & (waves - 1)) == 0;
  const bool aligned = ((reinterpret_cast<uintptr_t>(B) | reinterpret_cast<uintptr_t>(C)) % 4 |
                        reinterpret_cast<uintptr_t>(packed) % 16) == 0;
  // every index of the tokens kernel below 2^31: the source words, the
  // packed words and the thread count
  const int64_t top = std::max({batch * groups * L * N / 2, batch * groups * waves * run_words,
                                tokens + 256, nflags + 256});
  if (src_bf16 && dst_bf16 && !state_major && pow2 && aligned && top < (int64_t(1) << 31) &&
      (npw == 2 || npw == 4 || npw == 8 || npw == 16)) {
    uint32_t lg = 0;
    while ((1 << lg) < waves) ++lg;
    const int64_t threads = std::max<int64_t>(tokens, nflags);
    const dim3 grid((unsigned)((threads + 255) / 256));
    const auto Bw = static_cast<const uint32_t*>(B);
    const auto Cw = static_cast<const uint32_t*>(C);
    auto pk = static_cast<uint32_t*>(packed);
    const U32Div sd = make_u32div((uint32_t)steps), gd = make_u32div((uint32_t)groups);
    const uint32_t nf = flags ? (uint32_t)nflags : 0u;
#define MSSM_PACK_TOKENS(P)                                                                   \
  hipLaunchKernelGGL(fwd::bc_pack_tokens_kernel<P>, grid, dim3(256), 0, stream, Bw, Cw, pk, \
                     (uint32_t)tokens, (uint32_t)steps, sd, (uint32_t)L, (uint32_t)groups,  \
                     gd, lg, (uint32_t)run_words, flags, nf)
    switch (npw) {
      case 2: MSSM_PACK_TOKENS(2); break;
      case 4: MSSM_PACK_TOKENS(4); break;
      case 8: MSSM_PACK_TOKENS(8); break;
      default: MSSM_PACK_TOKENS(16); break;
    }
#undef MSSM_PACK_TOKENS
    return hipGetLastError();
  }
  const int64_t total = std::max<int64_t>(batch * groups * steps * 2 * N, nflags);
  hipLaunchKernelGGL(fwd::bc_pack_kernel, dim3((unsigned)((total + 255) / 256)),
                     dim3(256), 0, stream, B, C, packed, batch, groups, L, steps,
                     N, waves, src_bf16 ? 1 : 0, dst_bf16 ? 1 : 0, run_words, flags,
                     flags ? nflags : (int64_t)0, state_major ? 1 : 0);
  return hipGetLastError();
}

int64_t scan_bc_workspace_bytes(int64_t batch, int64_t L, int N, bool bf16) {
  const int NG = scan_waves_per_group(N);
  const int npw = N / NG;
  const int wps = bf16 ? npw : 2 * npw;
  return batch * NG * bc_run_words(L, wps) * 4;
}

int scan_waves_per_group(int N) {
  switch (N) {
    case 1: return fwd::kWaves<1>;
    case 2: return fwd::kWaves<2>;
    case 4: return fwd::kWaves<4>;
    case 8: return fwd::kWaves<8>;
    case 16: return fwd::kWaves<16>;
    case 32: return fwd::kWaves<32>;
    case 64: return fwd::kWaves<64>;
    default: return fwd::kWaves<128>;
  }
}

hipError_t launch_scan(const ScanParams& p, int N, bool bf16, bool vec,
                       hipStream_t stream) {
  switch (N) {
    case 1: return launch_scan_n1(p, bf16, vec, stream);
    case 2: return launch_scan_n2(p, bf16, vec, stream);
    case 4: return launch_scan_n4(p, bf16, vec, stream);
    case 8: return launch_scan_n8(p, bf16, vec, stream);
    case 16: return launch_scan_n16(p, bf16, vec, stream);
    case 32: return launch_scan_n32(p, bf16, vec, stream);
    case 64: return launch_scan_n64(p, bf16, vec, stream);
    case 128: return launch_scan_n128(p, bf16, vec, stream);
    default: return hipErrorInvalidValue;
  }
}


}  // namespace mssm
