// scan_fwd.hip -- forward selective scan kernels for gfx950 (CDNA4, wave64).
//
// Recurrence per (batch b, channel d) row, with the state kept in fp32
// (page "Mamba: Selective State Space Models", "Mathematical Foundation":
// input-dependent B, C and step Delta; Delta drives the discretisation):
//   Delta_t = softplus(delta_t + bias[d])        (or without softplus)
//   h_t[n]  = exp(Delta_t A[d,n]) h_{t-1}[n] + Delta_t B_t[n] u_t
//   out_t   = (sum_n C_t[n] h_t[n] + D[d] u_t) * silu(z_t)
//
// Mapping onto the chip.  The scan is not a dense contraction and is bound by
// the vector ALU (one v_exp_f32 per state element, which issues at half rate,
// plus four fp32 mul/fma), so the layout minimises issued VALU instructions:
//   * one lane per channel: 64 channels of one batch entry per workgroup, so
//     B_t and C_t are the same for every lane -- they are read with scalar
//     loads into SGPRs and cost no vector instructions or LDS traffic;
//   * the N states of a channel are split over the NG waves of the
//     workgroup (NPW = N / NG each), which multiplies the parallelism by NG;
//   * per-element work (softplus of delta, Delta*u, the D skip, the silu
//     gate, the bf16 round trip) is done once: each wave prepares and emits
//     8 timesteps of every 8*NG-step tile, sharing (Delta, Delta*u) and the
//     per-wave partial readouts through LDS;
//   * each lane reads its row's u / delta / z in 16-byte pieces (8 bf16
//     timesteps), one tile ahead of use, and writes 8 outputs per store.
// Long rows can be cut into time segments (aggregate -> combine -> main):
// the recurrence is associative on (decay, offset) pairs, so a segment's
// effect on the state is (exp(A * sum Delta), local end state from zero).
#include "dev_math.h"
#include "mssm_internal.h"

namespace mssm {
namespace {

constexpr int kLanes = 64;
constexpr int kChunk = 8;  // timesteps a wave prepares and emits per tile

struct ScanShape {
  int64_t dim, L;
  int32_t softplus, load_state;
  int32_t groups_per_batch, whole_groups, segments;
  int64_t seg_len;
};

template <bool BF16>
struct Raw;  // 8 consecutive io values of one row, as loaded
template <>
struct Raw<true> {
  uint32_t w[4];
};
template <>
struct Raw<false> {
  uint32_t w[8];
};

template <bool BF16>
__device__ __forceinline__ float raw_get(const Raw<BF16>& r, int k) {
  if constexpr (BF16)
    return (k & 1) ? bf16_hi(r.w[k >> 1]) : bf16_lo(r.w[k >> 1]);
  else
    return __uint_as_float(r.w[k]);
}

template <bool BF16>
__device__ __forceinline__ void raw_zero(Raw<BF16>& r) {
#pragma unroll
  for (int i = 0; i < (BF16 ? 4 : 8); ++i) r.w[i] = 0u;
}

// Values [t, t + 8) of a row; `nvalid` of them exist (the rest read as 0).
// VEC: 16-byte aligned and every chunk is whole or absent.
template <bool BF16, bool VEC>
__device__ __forceinline__ void load_chunk(Raw<BF16>& r, const void* base,
                                           int64_t off, int64_t nvalid) {
  if constexpr (VEC) {
    if (nvalid > 0) {
      if constexpr (BF16) {
        const uint4 v = *reinterpret_cast<const uint4*>(
            static_cast<const uint16_t*>(base) + off);
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
      } else {
        const uint4* q = reinterpret_cast<const uint4*>(
            static_cast<const float*>(base) + off);
        const uint4 v0 = q[0], v1 = q[1];
        r.w[0] = v0.x; r.w[1] = v0.y; r.w[2] = v0.z; r.w[3] = v0.w;
        r.w[4] = v1.x; r.w[5] = v1.y; r.w[6] = v1.z; r.w[7] = v1.w;
      }
    } else {
      raw_zero(r);
    }
  } else {
    if constexpr (BF16) {
      const uint16_t* s = static_cast<const uint16_t*>(base) + off;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (2 * i < nvalid) ? s[2 * i] : 0u;
        const uint32_t hi = (2 * i + 1 < nvalid) ? s[2 * i + 1] : 0u;
        r.w[i] = lo | (hi << 16);
      }
    } else {
      const uint32_t* s = static_cast<const uint32_t*>(base) + off;
#pragma unroll
      for (int i = 0; i < 8; ++i) r.w[i] = (i < nvalid) ? s[i] : 0u;
    }
  }
}

template <bool BF16, bool VEC>
__device__ __forceinline__ void store_chunk(void* base, int64_t off,
                                            const float (&o)[kChunk],
                                            int64_t nvalid) {
  if constexpr (BF16) {
    uint16_t* dst = static_cast<uint16_t*>(base) + off;
    if (VEC && nvalid >= kChunk) {
      uint4 v;
      v.x = pack_bf16x2(o[0], o[1]);
      v.y = pack_bf16x2(o[2], o[3]);
      v.z = pack_bf16x2(o[4], o[5]);
      v.w = pack_bf16x2(o[6], o[7]);
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
#pragma unroll
      for (int k = 0; k < kChunk; ++k)
        if (k < nvalid) dst[k] = to_bf16(o[k]);
    }
  } else {
    float* dst = static_cast<float*>(base) + off;
    if (VEC && nvalid >= kChunk) {
      float4* q = reinterpret_cast<float4*>(dst);
      q[0] = make_float4(o[0], o[1], o[2], o[3]);
      q[1] = make_float4(o[4], o[5], o[6], o[7]);
    } else {
#pragma unroll
      for (int k = 0; k < kChunk; ++k)
        if (k < nvalid) dst[k] = o[k];
    }
  }
}

// NPW consecutive B (or C) values of one token, kept as the loaded 32-bit
// words (bf16 pairs or fp32) and unpacked only where they are used, so that
// prefetched words do not force a wait.  The address is the same for every
// lane, so these become scalar loads.
template <int NPW, bool BF16>
struct BCWords {
  static constexpr int W = BF16 ? (NPW + 1) / 2 : NPW;
  uint32_t w[W];
};

template <int NPW, bool BF16, bool VEC>
__device__ __forceinline__ void load_bc(BCWords<NPW, BF16>& v, const void* base,
                                        int64_t off) {
  if constexpr (BF16) {
    const uint16_t* s = static_cast<const uint16_t*>(base) + off;
    if constexpr (VEC && NPW >= 2) {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(s);
#pragma unroll
      for (int j = 0; j < NPW / 2; ++j) v.w[j] = w[j];
    } else {
#pragma unroll
      for (int j = 0; j < BCWords<NPW, BF16>::W; ++j) {
        const uint32_t lo = s[2 * j];
        const uint32_t hi = (2 * j + 1 < NPW) ? (uint32_t)s[2 * j + 1] : 0u;
        v.w[j] = lo | (hi << 16);
      }
    }
  } else {
    const uint32_t* s = static_cast<const uint32_t*>(base) + off;
#pragma unroll
    for (int j = 0; j < NPW; ++j) v.w[j] = s[j];
  }
}

template <int NPW, bool BF16>
__device__ __forceinline__ float bc_get(const BCWords<NPW, BF16>& v, int j) {
  if constexpr (BF16)
    return (j & 1) ? bf16_hi(v.w[j >> 1]) : bf16_lo(v.w[j >> 1]);
  else
    return __uint_as_float(v.w[j]);
}

// Main pass (AGG = false): scans each task's time range from its initial
// state and writes out (and last_state after the final segment).
// Aggregate pass (AGG = true): scans segments 0..P-2 of the split groups from
// a zero state and writes the end state and the sum of Delta.
//
// Latency.  Scalar loads (B, C) and LDS reads (Delta, Delta*u) share one
// wait counter and scalar loads return out of order, so every wait on them is
// a full drain.  The state phase therefore walks a tile in batches of KB
// timesteps: the first timestep of a batch takes the one wait, then the next
// batch's B/C scalar loads and Delta/Delta*u LDS reads are issued, and the
// rest of the batch computes while they are in flight.
template <int N, int NG, bool BF16, bool VEC, bool HAS_Z, bool AGG, bool SOFTPLUS>
__global__ void __launch_bounds__(kLanes* NG)
    scan_kernel(const void* __restrict__ u, const void* __restrict__ delta,
                const void* __restrict__ z, const float* __restrict__ A,
                const void* __restrict__ Bm, const void* __restrict__ Cm,
                const float* __restrict__ Dv, const float* __restrict__ bias,
                void* __restrict__ out, float* __restrict__ last_state,
                float* __restrict__ ws_S, double* __restrict__ ws_sum,
                const float* __restrict__ ws_hin, const ScanShape s) {
  constexpr int NPW = N / NG;
  constexpr int T = kChunk * NG;
  constexpr int KB = 4;          // timesteps per batch
  constexpr int NB = T / KB;     // batches per tile
  __shared__ float2 s_dw[T][kLanes];                              // (Delta, Delta*u)
  __shared__ float s_y[AGG ? 1 : NG][AGG ? 1 : T][kLanes];       // partial readouts

  const int lane = threadIdx.x & (kLanes - 1);
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = g * NPW;

  // task -> (group, segment)
  int gi, seg, nseg;
  const int task = blockIdx.x;
  if constexpr (AGG) {
    const int per = s.segments - 1;
    gi = s.whole_groups + task / per;
    seg = task % per;
    nseg = s.segments;
  } else if (task < s.whole_groups) {
    gi = task;
    seg = 0;
    nseg = 1;
  } else {
    const int j = task - s.whole_groups;
    gi = s.whole_groups + j / s.segments;
    seg = j % s.segments;
    nseg = s.segments;
  }
  const int64_t b = gi / s.groups_per_batch;
  const int64_t d = (int64_t)(gi % s.groups_per_batch) * kLanes + lane;
  const bool valid = d < s.dim;
  const int64_t dc = valid ? d : s.dim - 1;
  const int64_t row = b * s.dim + dc;
  const int64_t t_begin = nseg > 1 ? (int64_t)seg * s.seg_len : 0;
  const int64_t t_end = nseg > 1 ? min(s.L, t_begin + s.seg_len) : s.L;
  const int64_t sr = (int64_t)(gi - s.whole_groups) * kLanes + lane;

  float A2[NPW], h[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    A2[j] = A[dc * N + n0 + j] * kLog2e;
    if (AGG)
      h[j] = 0.0f;
    else if (nseg > 1)
      h[j] = ws_hin[(sr * nseg + seg) * N + n0 + j];
    else if (s.load_state)
      h[j] = last_state[row * N + n0 + j];
    else
      h[j] = 0.0f;
  }
  const float bv_d = bias ? bias[dc] : 0.0f;
  const float Dd = (!AGG && Dv) ? Dv[dc] : 0.0f;
  double dsum = 0.0;

  const int64_t bc_base = b * s.L * N + n0;  // this wave's slice of B_t, C_t
  const int64_t rowoff = row * s.L;

  Raw<BF16> ru, rd, rz, nu, nd, nz;
  raw_zero(rz);
  raw_zero(nz);

  auto prep = [&](const Raw<BF16>& pu, const Raw<BF16>& pd) {
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const float x = raw_get(pd, k) + bv_d;
      const float dl = SOFTPLUS ? softplus_f32(x) : x;
      s_dw[g * kChunk + k][lane] = make_float2(dl, dl * raw_get(pu, k));
    }
  };

  // one timestep of this wave's NPW states; returns the partial readout
  using Words = BCWords<NPW, BF16>;
  auto advance = [&](const float2 dw, const Words& bq, const Words& cq) -> float {
    float y = 0.0f;
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
      const float e = hw_exp2(dw.x * A2[j]);
      h[j] = fmaf(e, h[j], dw.y * bc_get(bq, j));
      if constexpr (!AGG) y = fmaf(bc_get(cq, j), h[j], y);
    }
    if constexpr (AGG) dsum += (double)dw.x;
    return y;
  };

  // prologue: this wave's chunk of the first tile
  {
    const int64_t tc = t_begin + g * kChunk;
    const int64_t nv = t_end - tc;
    load_chunk<BF16, VEC>(ru, u, rowoff + tc, nv);
    load_chunk<BF16, VEC>(rd, delta, rowoff + tc, nv);
    if (HAS_Z && !AGG) load_chunk<BF16, VEC>(rz, z, rowoff + tc, nv);
    prep(ru, rd);
  }
  __syncthreads();

  for (int64_t tb = t_begin; tb < t_end; tb += T) {
    // prefetch this wave's chunk of the next tile
    {
      const int64_t tc = tb + T + g * kChunk;
      const int64_t nv = t_end - tc;
      load_chunk<BF16, VEC>(nu, u, rowoff + tc, nv);
      load_chunk<BF16, VEC>(nd, delta, rowoff + tc, nv);
      if (HAS_Z && !AGG) load_chunk<BF16, VEC>(nz, z, rowoff + tc, nv);
    }

    // state phase: every wave advances its NPW states over the whole tile
    const int64_t nt = t_end - tb;
    if (nt >= T) {
      float2 dwn[KB];
      Words bn[KB], cn[KB];
      const int64_t off0 = bc_base + tb * N;
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        dwn[i] = s_dw[i][lane];
        load_bc<NPW, BF16, VEC>(bn[i], Bm, off0 + i * N);
        if constexpr (!AGG) load_bc<NPW, BF16, VEC>(cn[i], Cm, off0 + i * N);
        else cn[i] = bn[i];
      }
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        float2 dwc[KB];
        Words bc_[KB], cc_[KB];
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          dwc[i] = dwn[i];
          bc_[i] = bn[i];
          cc_[i] = cn[i];
        }
        float yb[KB];
        yb[0] = advance(dwc[0], bc_[0], cc_[0]);  // takes the batch's wait
        __builtin_amdgcn_sched_barrier(0);
        if (kb + 1 < NB) {
          const int64_t offn = off0 + (int64_t)(kb + 1) * KB * N;
#pragma unroll
          for (int i = 0; i < KB; ++i) {
            dwn[i] = s_dw[(kb + 1) * KB + i][lane];
            load_bc<NPW, BF16, VEC>(bn[i], Bm, offn + i * N);
            if constexpr (!AGG) load_bc<NPW, BF16, VEC>(cn[i], Cm, offn + i * N);
            else cn[i] = bn[i];
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 1; i < KB; ++i) yb[i] = advance(dwc[i], bc_[i], cc_[i]);
        if constexpr (!AGG) {
#pragma unroll
          for (int i = 0; i < KB; ++i) s_y[g][kb * KB + i][lane] = yb[i];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      for (int kk = 0; kk < nt; ++kk) {
        Words bq, cq;
        const int64_t off = bc_base + (tb + kk) * N;
        load_bc<NPW, BF16, VEC>(bq, Bm, off);
        if constexpr (!AGG) load_bc<NPW, BF16, VEC>(cq, Cm, off);
        else cq = bq;
        const float y = advance(s_dw[kk][lane], bq, cq);
        if constexpr (!AGG) s_y[g][kk][lane] = y;
      }
    }
    __syncthreads();

    if constexpr (!AGG) {
      // output phase: this wave's chunk of the tile
      const int64_t tc = tb + g * kChunk;
      float o[kChunk];
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        float y = 0.0f;
#pragma unroll
        for (int w = 0; w < NG; ++w) y += s_y[w][g * kChunk + k][lane];
        y = fmaf(Dd, raw_get(ru, k), y);
        if (HAS_Z) y *= silu_f32(raw_get(rz, k));
        o[k] = y;
      }
      if (valid) store_chunk<BF16, VEC>(out, rowoff + tc, o, t_end - tc);
    }

    ru = nu;
    rd = nd;
    rz = nz;
    prep(ru, rd);
    __syncthreads();
  }

  if constexpr (AGG) {
    const int per = nseg - 1;
#pragma unroll
    for (int j = 0; j < NPW; ++j) ws_S[(sr * per + seg) * N + n0 + j] = h[j];
    if (g == 0) ws_sum[sr * per + seg] = dsum;
  } else {
    if (last_state && valid && seg == nseg - 1) {
#pragma unroll
      for (int j = 0; j < NPW; ++j) last_state[row * N + n0 + j] = h[j];
    }
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

template <int N, int NG, bool BF16, bool VEC, bool HAS_Z, bool AGG>
hipError_t launch_one(const ScanParams& p, const ScanShape& s, int tasks,
                      hipStream_t stream) {
  if (!p.softplus) {
    hipLaunchKernelGGL((scan_kernel<N, NG, BF16, VEC, HAS_Z, AGG, false>),
                       dim3(tasks), dim3(kLanes * NG), 0, stream, p.u, p.delta,
                       p.z, p.A, p.B, p.C, p.D, p.bias, p.out, p.last_state,
                       p.ws_S, p.ws_sum, p.ws_hin, s);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((scan_kernel<N, NG, BF16, VEC, HAS_Z, AGG, true>), dim3(tasks),
                     dim3(kLanes * NG), 0, stream, p.u, p.delta, p.z, p.A, p.B,
                     p.C, p.D, p.bias, p.out, p.last_state, p.ws_S, p.ws_sum,
                     p.ws_hin, s);
  return hipGetLastError();
}

template <int N, bool BF16, bool VEC>
hipError_t launch_n(const ScanParams& p, hipStream_t stream) {
  constexpr int NG = (N >= 8) ? N / 4 : 1;
  ScanShape s;
  s.dim = p.dim;
  s.L = p.L;
  s.softplus = p.softplus;
  s.load_state = p.load_state;
  s.groups_per_batch = p.groups_per_batch;
  s.whole_groups = p.whole_groups;
  s.segments = p.segments;
  s.seg_len = p.seg_len;
  hipError_t e;
  if (p.split_groups > 0) {
    e = launch_one<N, NG, BF16, VEC, false, true>(
        p, s, p.split_groups * (p.segments - 1), stream);
    if (e != hipSuccess) return e;
    const int64_t split_rows = (int64_t)p.split_groups * kLanes;
    const int64_t threads = split_rows * N;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, stream, p.A, p.last_state, p.ws_S,
                       p.ws_sum, p.ws_hin, s, N, split_rows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int tasks = p.whole_groups + p.split_groups * p.segments;
  if (p.z)
    return launch_one<N, NG, BF16, VEC, true, false>(p, s, tasks, stream);
  return launch_one<N, NG, BF16, VEC, false, false>(p, s, tasks, stream);
}

template <int N>
hipError_t launch_dtype(const ScanParams& p, bool bf16, bool vec,
                        hipStream_t stream) {
  if (bf16)
    return vec ? launch_n<N, true, true>(p, stream)
               : launch_n<N, true, false>(p, stream);
  return vec ? launch_n<N, false, true>(p, stream)
             : launch_n<N, false, false>(p, stream);
}

}  // namespace

int scan_waves_per_group(int N) { return (N >= 8) ? N / 4 : 1; }

hipError_t launch_scan(const ScanParams& p, int N, bool bf16, bool vec,
                       hipStream_t stream) {
  switch (N) {
    case 1: return launch_dtype<1>(p, bf16, vec, stream);
    case 2: return launch_dtype<2>(p, bf16, vec, stream);
    case 4: return launch_dtype<4>(p, bf16, vec, stream);
    case 8: return launch_dtype<8>(p, bf16, vec, stream);
    case 16: return launch_dtype<16>(p, bf16, vec, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mssm
