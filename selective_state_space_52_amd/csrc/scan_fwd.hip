// scan_fwd.hip -- the forward scan's non-template parts: the B/C pack, the
// combine of segment summaries, the work split helpers and the dispatch over
// state sizes (whose kernels are instantiated in scan_fwd_n*.hip).
#include "scan_fwd_impl.h"

namespace mssm {
namespace fwd {

// Writes the packed runs of `steps` timesteps per wave (steps >= L; the
// timesteps from L on are written as zeros) with `run_words` words per run.
// The source is bf16 or fp32 (src_bf16); the runs keep bf16 (dst_bf16) or
// hold fp32.
__global__ void __launch_bounds__(256)
    bc_pack_kernel(const void* __restrict__ Bm, const void* __restrict__ Cm,
                   void* __restrict__ packed, int64_t batch, int64_t groups,
                   int64_t L, int64_t steps, int N, int NG, int src_bf16,
                   int dst_bf16, int64_t run_words) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
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
  const int64_t src = ((b * L + t) * groups + grp) * N + n;
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


// Initial state of every segment of the split groups, from the segment
// summaries: h_in[0] = h0, h_in[s+1] = exp(A * sum_s Delta) h_in[s] + S_s.
__global__ void __launch_bounds__(256)
    combine_kernel(const float* __restrict__ A, const float* __restrict__ h0,
                   const float* __restrict__ ws_S,
                   const double* __restrict__ ws_sum,
                   float* __restrict__ ws_hin, const ScanShape s, int N,
                   int64_t split_rows) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= split_rows * N) return;
  const int64_t sr = tid / N;
  const int n = (int)(tid - sr * N);
  const int P = s.segments;
  const int64_t gi = s.whole_groups + sr / kLanes;
  const int64_t b = gi / s.groups_per_batch;
  const int64_t d = (gi % s.groups_per_batch) * kLanes + (sr % kLanes);
  if (d >= s.dim) {
    for (int q = 0; q < P; ++q) ws_hin[(sr * P + q) * N + n] = 0.0f;
    return;
  }
  const double a = A[d * N + n];
  double h = (s.load_state && h0) ? h0[(b * s.dim + d) * N + n] : 0.0;
  for (int q = 0; q < P; ++q) {
    ws_hin[(sr * P + q) * N + n] = (float)h;
    if (q < P - 1)
      h = exp(a * ws_sum[sr * (P - 1) + q]) * h +
          (double)ws_S[(sr * (P - 1) + q) * N + n];
  }
}

hipError_t launch_combine(const ScanParams& p, const ScanShape& s, int N,
                          hipStream_t stream) {
  const int64_t split_rows = (int64_t)p.split_groups * kLanes;
  const int64_t threads = split_rows * N;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, stream, p.A, p.last_state, p.ws_S, p.ws_sum,
                     p.ws_hin, s, N, split_rows);
  return hipGetLastError();
}


}  // namespace fwd

hipError_t launch_bc_pack(const void* B, const void* C, void* packed,
                          int64_t batch, int64_t groups, int64_t L, int64_t steps,
                          int N, int waves, bool src_bf16, bool dst_bf16,
                          int64_t run_words, hipStream_t stream) {
  const int64_t total = batch * groups * steps * 2 * N;
  hipLaunchKernelGGL(fwd::bc_pack_kernel, dim3((unsigned)((total + 255) / 256)),
                     dim3(256), 0, stream, B, C, packed, batch, groups, L, steps,
                     N, waves, src_bf16 ? 1 : 0, dst_bf16 ? 1 : 0, run_words);
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
