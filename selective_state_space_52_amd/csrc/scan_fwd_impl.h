// scan_fwd_impl.h -- forward selective scan kernels for gfx950 (CDNA4, wave64),
// as templates; scan_fwd_n*.hip instantiate them per state size.
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
//     workgroup (NPW = N / NG each), which multiplies the parallelism by NG
//     and gives each SIMD two waves of one workgroup at N = 16;
//   * per-element work (softplus of delta, Delta*u, the D skip, the silu
//     gate, the bf16 round trip) is done once: each wave prepares and emits
//     32 / NG timesteps of every 32-step tile, sharing (Delta, Delta*u) and
//     the per-wave partial readouts through LDS;
//   * B_t and C_t are repacked once per call into fp32 runs per wave, read
//     with 64-byte scalar loads;
//   * each lane reads its row's u / delta / z in 8- or 16-byte pieces, one
//     tile ahead of use, and writes its outputs with the same width.
// Long rows can be cut into time segments (aggregate -> combine -> main):
// the recurrence is associative on (decay, offset) pairs, so a segment's
// effect on the state is (exp(A * sum Delta), local end state from zero).
#pragma once

#include <algorithm>

#include "dev_math.h"
#include "mssm_internal.h"
#include "scan_common.h"

namespace mssm {
namespace fwd {

constexpr int kTile = 32;  // timesteps per tile
constexpr bool kWarmScalarCache = true;

// Waves per 64-channel workgroup: two states per wave up to N = 16 (one for
// N = 1), so a group of N = 16 runs 8 waves, two per SIMD; larger states keep
// 8 waves and give each wave N / 8 states.
template <int N>
constexpr int kWaves = N >= 16 ? 8 : (N >= 2 ? N / 2 : 1);

// The causal depthwise conv (width 4) that can feed the scan: u = silu(bias +
// sum_k w[k] x[t-3+k]), x at t < 0 from init (or 0).
struct ConvArgs {
  const float* w;      // (dim, 4) fp32
  const float* b;      // (dim) fp32 or null
  const void* init;    // (batch, dim, 3) io dtype (x at t = -3..-1) or null
  void* u_out;         // (batch, dim, L) io dtype: the conv output, or null
};
constexpr int kConvK = 4;

struct ScanShape {
  int64_t dim, L;
  int64_t ts;  // elements between consecutive timesteps of a row: 1, or dim
               // for the (batch, length, channel) layout
  int32_t ngroups, groups_per_bc;  // B/C groups; channel groups per B/C group
  int32_t softplus, load_state;
  int32_t groups_per_batch, whole_groups, segments;
  int64_t seg_len;
};


// Initial states of the split groups' segments (scan_fwd.hip).
hipError_t launch_combine(const ScanParams& p, const ScanShape& s, int N,
                          hipStream_t stream);

// Main pass (AGG = false): scans each task's time range from its initial
// state and writes out (and last_state after the final segment).
// Aggregate pass (AGG = true): scans segments 0..P-2 of the split groups from
// a zero state and writes the end state and the sum of Delta.
//
// A tile of kTile timesteps is done in three phases:
//   prep   : each wave turns KC = kTile / NG of the tile's timesteps into
//            (Delta, Delta*u) for its 64 channels and writes them to LDS;
//   state  : each wave advances its NPW states over all kTile timesteps and
//            writes its partial readouts to LDS;
//   output : each wave sums the NG partials of its KC timesteps, adds the D
//            skip, applies the gate and stores.
// Latency.  Scalar loads (B, C) and LDS reads (Delta, Delta*u) share one
// wait counter and scalar loads return out of order, so every wait on them is
// a full drain.  The state phase therefore walks a tile in batches of KB
// timesteps: the first timestep of a batch takes the one wait, then the next
// batch's B/C scalar loads and Delta/Delta*u LDS reads are issued, and the
// rest of the batch computes while they are in flight.
template <int N, int NG, bool BF16, bool VEC, bool HAS_Z, bool AGG, bool SOFTPLUS,
          bool CONV>
__device__ __forceinline__ void scan_body(
    const void* __restrict__ u, const void* __restrict__ delta,
    const void* __restrict__ z, const float* __restrict__ A,
    const float* __restrict__ Dv, const float* __restrict__ bias,
    void* __restrict__ out, float* __restrict__ last_state,
    float* __restrict__ ws_S, double* __restrict__ ws_sum,
    const float* __restrict__ ws_hin, const uint32_t* __restrict__ bcp,
    const ScanShape& s, float2 (&s_dw)[kTile][kLanes],
    float (&s_y)[NG][kTile][kLanes], const int task, const ConvArgs& cv) {
  constexpr int NPW = N / NG;
  constexpr int T = kTile;
  constexpr int KC = T / NG;     // timesteps a wave prepares and emits
  constexpr int WPS = BCLayout<NPW, BF16>::kWordsPerStep;
  constexpr int KB = BCLayout<NPW, BF16>::kSteps;  // timesteps per batch
  constexpr int NB = T / KB;     // batches per tile

  const int lane = threadIdx.x & (kLanes - 1);
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = g * NPW;

  // task -> (group, segment)
  int gi, seg, nseg;
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
  // first element of the row in u / delta / z / out
  const int64_t rowoff = s.ts == 1 ? row * s.L : b * s.L * s.dim + dc;
  // Time indices are 32-bit (the host keeps L below 2^31 - 64), so their
  // compares run on the scalar unit.
  const int Lr = (int)s.L;
  const int t_begin = nseg > 1 ? seg * (int)s.seg_len : 0;
  const int t_end = nseg > 1 ? (int)min(s.L, (int64_t)t_begin + s.seg_len) : Lr;
  const int64_t sr = (int64_t)(gi - s.whole_groups) * kLanes + lane;
  // Vector path with chunks of at most 8 steps (N >= 8): each lane keeps
  // pointers to its own rows, and the next tile's chunk start is clamped to
  // the task's last chunk (t_end is L, a multiple of 8, or a segment end, a
  // multiple of the tile, so t_end >= KC), so the loads need neither a
  // branch nor 64-bit index work.  A clamped chunk past the end re-reads
  // values of the task that nothing uses.
  constexpr bool kRowPtr = VEC && KC <= 8;
  constexpr int64_t kEs = BF16 ? 2 : 4;
  const char* const pu = static_cast<const char*>(u) + rowoff * kEs;
  const char* const pdl = static_cast<const char*>(delta) + rowoff * kEs;
  const char* const pz = HAS_Z ? static_cast<const char*>(z) + rowoff * kEs : nullptr;
  char* const po = AGG ? nullptr : static_cast<char*>(out) + rowoff * kEs;

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

  // With CONV, `u` holds the conv input x; each chunk also reads the 4 x
  // values before it (row start: the init values) and turns x into u.
  float cw[kConvK], cbias = 0.0f;
  Raw<BF16, kConvK> rp, np_;  // x[tc-4 .. tc-1] of the current / next chunk
  float uc[KC], un[KC];       // u of the current / next chunk, as fp32
  if constexpr (CONV) {
#pragma unroll
    for (int j = 0; j < kConvK; ++j) cw[j] = cv.w[dc * kConvK + j];
    cbias = cv.b ? cv.b[dc] : 0.0f;
  }
  auto load_prev = [&](Raw<BF16, kConvK>& r, int tc) {
    if (tc >= kConvK) {
      load_chunk<BF16, VEC, kConvK>(r, u, rowoff + (tc - kConvK) * s.ts,
                                    s.L - (tc - kConvK), s.ts);
    } else {
      // tc == 0 (chunks start at multiples of 4): slots 1..3 hold x[-3..-1]
      // from init, slot 0 is never used
      raw_zero(r);
      if (cv.init) {
        if constexpr (BF16) {
          const uint16_t* ip = static_cast<const uint16_t*>(cv.init) + row * (kConvK - 1);
          r.w[0] = (uint32_t)ip[0] << 16;
          r.w[1] = (uint32_t)ip[1] | ((uint32_t)ip[2] << 16);
        } else {
          const uint32_t* ip = static_cast<const uint32_t*>(cv.init) + row * (kConvK - 1);
          r.w[1] = ip[0];
          r.w[2] = ip[1];
          r.w[3] = ip[2];
        }
      }
    }
  };
  auto conv_u = [&](const Raw<BF16, KC>& px, const Raw<BF16, kConvK>& pp,
                    float (&uo)[KC]) {
    float xs[KC + kConvK];
#pragma unroll
    for (int j = 0; j < kConvK; ++j) xs[j] = raw_get(pp, j);
#pragma unroll
    for (int k = 0; k < KC; ++k) xs[kConvK + k] = raw_get(px, k);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      float v = cbias;
#pragma unroll
      for (int j = 0; j < kConvK; ++j) v = fmaf(cw[j], xs[k + 1 + j], v);
      uo[k] = silu_f32(v);
    }
  };

  // this wave's packed B/C run
  const int64_t bcg = b * s.ngroups + (gi % s.groups_per_batch) / s.groups_per_bc;
  const uint32_t* __restrict__ bcw = bcp + (bcg * NG + g) * bc_run_words(s.L, WPS);
  using Batch = BCBatch<NPW, BF16>;
  Raw<BF16, KC> ru, rd, rz, nu, nd, nz;
  raw_zero(rz);
  raw_zero(nz);

  // (Delta, Delta*u) of this wave's chunk into LDS; without the conv, u is
  // unpacked here once and kept (uv) for the chunk's D skip.  The aggregate
  // pass also sums Delta over the wave's own steps of the segment (dsum);
  // the waves' sums are added at the end.
  auto prep = [&](const Raw<BF16, KC>& pu, const Raw<BF16, KC>& pd, float (&uv)[KC],
                  int tile) {
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const float x = raw_get(pd, k) + bv_d;
      const float dl = SOFTPLUS ? softplus_f32(x) : x;
      if constexpr (!CONV) uv[k] = raw_get(pu, k);
      s_dw[g * KC + k][lane] = make_float2(dl, dl * uv[k]);
      if constexpr (AGG) {
        if (tile + g * KC + k < t_end) dsum += (double)dl;
      }
    }
  };

  // one timestep of this wave's NPW states; token i of the packed words w
  auto advance = [&](const float2 dw, const uint32_t* w, int i) -> float {
    float y = 0.0f;
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
      const float e = hw_exp2(dw.x * A2[j]);
      h[j] = fmaf(e, h[j], dw.y * bc_val<NPW, BF16>(w, i, j));
      if constexpr (!AGG) y = fmaf(bc_val<NPW, BF16>(w, i, NPW + j), h[j], y);
    }
    return y;
  };

  // prologue: this wave's chunk of the first tile
  {
    const int tc = t_begin + g * KC;
    const int nv = t_end - tc;
    load_chunk<BF16, VEC, KC>(ru, u, rowoff + tc * s.ts, nv, s.ts);
    load_chunk<BF16, VEC, KC>(rd, delta, rowoff + tc * s.ts, nv, s.ts);
    if (HAS_Z && !AGG) load_chunk<BF16, VEC, KC>(rz, z, rowoff + tc * s.ts, nv, s.ts);
    if constexpr (CONV) {
      load_prev(rp, tc);
      conv_u(ru, rp, uc);
    }
    prep(ru, rd, uc, t_begin);
  }
  __syncthreads();

  for (int tb = t_begin; tb < t_end; tb += T) {
    // prefetch this wave's chunk of the next tile
    if constexpr (kRowPtr) {
      const int tc = tb + T + g * KC;
      const int tl = min(tc, t_end - KC);
      // z first: loads complete in issue order, so the prep's wait for u and
      // delta also covers z, and nothing later waits behind the tile's stores
      if (HAS_Z && !AGG) load_chunk_row<BF16, KC>(nz, pz, tl);
      load_chunk_row<BF16, KC>(nu, pu, tl);
      load_chunk_row<BF16, KC>(nd, pdl, tl);
      // tc >= kTile here, so the 4 inputs before the chunk are in the row
      if constexpr (CONV) load_chunk_row<BF16, kConvK>(np_, pu, min(tc, t_end) - kConvK);
    } else {
      const int tc = tb + T + g * KC;
      const int nv = t_end - tc;
      load_chunk<BF16, VEC, KC>(nu, u, rowoff + tc * s.ts, nv, s.ts);
      load_chunk<BF16, VEC, KC>(nd, delta, rowoff + tc * s.ts, nv, s.ts);
      if (HAS_Z && !AGG) load_chunk<BF16, VEC, KC>(nz, z, rowoff + tc * s.ts, nv, s.ts);
      // tc >= kTile here, so the 4 inputs before the chunk are in the row.
      // On the vector path the load is unconditional (a conditional one
      // makes the compiler wait for the whole prefetch right after it): a
      // chunk past the end reads the row's last 4 inputs, which nothing uses.
      if constexpr (CONV) {
        if constexpr (VEC)
          load_chunk<BF16, true, kConvK>(np_, u, rowoff + min(tc, t_end) - kConvK, kConvK);
        else
          load_chunk<BF16, false, kConvK>(np_, u, rowoff + (tc - kConvK) * s.ts,
                                          nv + kConvK, s.ts);
      }
    }

    // state phase: every wave advances its NPW states over the whole tile
    const int nt = t_end - tb;
    if (nt >= T) {
      float2 dwn[KB];
      Batch bn = *reinterpret_cast<const Batch*>(bcw + (int64_t)tb * WPS);
#pragma unroll
      for (int i = 0; i < KB; ++i) dwn[i] = s_dw[i][lane];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        float2 dwc[KB];
#pragma unroll
        for (int i = 0; i < KB; ++i) dwc[i] = dwn[i];
        const Batch bc = bn;
        // pass 1: decays exp(Delta A) and drives Delta u B of the whole batch
        // (independent of the state, so the exponentials can run ahead of
        // the recurrence); token 0 takes the batch's wait
        float e[KB][NPW], bw[KB][NPW];
        auto decay_drive = [&](int i) {
#pragma unroll
          for (int j = 0; j < NPW; ++j) {
            e[i][j] = hw_exp2(dwc[i].x * A2[j]);
            bw[i][j] = dwc[i].y * bc_val<NPW, BF16>(bc.w, i, j);
          }
        };
        decay_drive(0);
        __builtin_amdgcn_sched_barrier(0);
        if (kb + 1 < NB) {
          bn = *reinterpret_cast<const Batch*>(bcw + ((int64_t)tb + (kb + 1) * KB) * WPS);
#pragma unroll
          for (int i = 0; i < KB; ++i) dwn[i] = s_dw[(kb + 1) * KB + i][lane];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 1; i < KB; ++i) decay_drive(i);
        // pass 2: the recurrence and the readout
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          float y = 0.0f;
#pragma unroll
          for (int j = 0; j < NPW; ++j) {
            h[j] = fmaf(e[i][j], h[j], bw[i][j]);
            if constexpr (!AGG) y = fmaf(bc_val<NPW, BF16>(bc.w, i, NPW + j), h[j], y);
          }
          if constexpr (!AGG) s_y[g][kb * KB + i][lane] = y;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      for (int kk = 0; kk < nt; ++kk) {
        uint32_t q[WPS];
#pragma unroll
        for (int j = 0; j < WPS; ++j) q[j] = bcw[((int64_t)tb + kk) * WPS + j];
        const float y = advance(s_dw[kk][lane], q, 0);
        if constexpr (!AGG) s_y[g][kk][lane] = y;
      }
    }
    __syncthreads();

    // Warm the scalar cache with the next tile's B/C run: one dword per
    // 64-byte line.  Scalar loads can only be waited on all together, so they
    // are issued here, where the first wait (the output phase's LDS reads)
    // comes after the whole prep phase.
    uint32_t touch = 0u;
    if (kWarmScalarCache) {
      const int64_t last = bc_run_words(s.L, WPS) - 1;  // last word of the run
      const int64_t f0 = ((int64_t)tb + T) * WPS;
#pragma unroll
      for (int f = 0; f < T * WPS; f += 16) touch += bcw[min(f0 + f, last)];
    }
    __builtin_amdgcn_sched_barrier(0);

    // prep of the next tile (its Delta/Delta*u slots are free: every wave is
    // past the state phase)
    if constexpr (CONV) conv_u(nu, np_, un);
    prep(nu, nd, un, tb + T);

    if constexpr (!AGG) {
      // output phase: this wave's chunk of the tile
      const int tc = tb + g * KC;
      float o[KC];
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        float y = s_y[0][g * KC + k][lane];
#pragma unroll
        for (int w = 1; w < NG; ++w) y += s_y[w][g * KC + k][lane];
        y = fmaf(Dd, uc[k], y);
        if (HAS_Z) y *= silu_f32(raw_get(rz, k));
        o[k] = y;
      }
      if constexpr (kRowPtr) {
        if (valid) store_chunk_row<BF16, KC>(po, tc, o, t_end - tc);
        if constexpr (CONV) {
          if (valid && cv.u_out)
            store_chunk_row<BF16, KC>(static_cast<char*>(cv.u_out) + rowoff * kEs, tc, uc,
                                      t_end - tc);
        }
      } else {
        if (valid) store_chunk<BF16, VEC, KC>(out, rowoff + tc * s.ts, o, t_end - tc, s.ts);
        if constexpr (CONV) {
          if (valid && cv.u_out)
            store_chunk<BF16, VEC, KC>(cv.u_out, rowoff + tc * s.ts, uc, t_end - tc, s.ts);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::"s"(touch));  // keeps the warming loads

    rz = nz;
#pragma unroll
    for (int k = 0; k < KC; ++k) uc[k] = un[k];
    __syncthreads();
  }

  if constexpr (AGG) {
    const int per = nseg - 1;
#pragma unroll
    for (int j = 0; j < NPW; ++j) ws_S[(sr * per + seg) * N + n0 + j] = h[j];
    // the segment's sum of Delta: the waves' sums over their own steps, added
    // in wave order (s_y is free: the loop ended on a barrier)
    double* part = reinterpret_cast<double*>(&s_y[0][0][0]);
    part[g * kLanes + lane] = dsum;
    __syncthreads();
    if (g == 0) {
      double tot = 0.0;
#pragma unroll
      for (int w = 0; w < NG; ++w) tot += part[w * kLanes + lane];
      ws_sum[sr * per + seg] = tot;
    }
  } else {
    if (last_state && valid && seg == nseg - 1) {
#pragma unroll
      for (int j = 0; j < NPW; ++j) last_state[row * N + n0 + j] = h[j];
    }
  }
}

// One launch runs `n_main` main-pass tasks (task = main_base + block) and,
// after them, aggregate-pass tasks (task = block - n_main).  Putting the
// aggregate pass of the time-split groups into the same launch as the main
// pass of the whole groups lets it run on the CUs' spare workgroup slots.
template <int N, int NG, bool BF16, bool VEC, bool HAS_Z, bool SOFTPLUS, bool CONV>
__global__ void __launch_bounds__(kLanes* NG)
    scan_kernel(const void* __restrict__ u, const void* __restrict__ delta,
                const void* __restrict__ z, const float* __restrict__ A,
                const float* __restrict__ Dv, const float* __restrict__ bias,
                void* __restrict__ out, float* __restrict__ last_state,
                float* __restrict__ ws_S, double* __restrict__ ws_sum,
                const float* __restrict__ ws_hin,
                const uint32_t* __restrict__ bcp, const ScanShape s,
                const int n_main, const int main_base, const ConvArgs cv) {
  __shared__ float2 s_dw[kTile][kLanes];        // (Delta, Delta*u) of a tile
  __shared__ float s_y[NG][kTile][kLanes];      // per-wave partial readouts
  const int blk = blockIdx.x;
  if (blk < n_main)
    scan_body<N, NG, BF16, VEC, HAS_Z, false, SOFTPLUS, CONV>(
        u, delta, z, A, Dv, bias, out, last_state, ws_S, ws_sum, ws_hin, bcp,
        s, s_dw, s_y, main_base + blk, cv);
  else
    scan_body<N, NG, BF16, VEC, HAS_Z, true, SOFTPLUS, CONV>(
        u, delta, z, A, Dv, bias, out, last_state, ws_S, ws_sum, ws_hin, bcp,
        s, s_dw, s_y, blk - n_main, cv);
}


template <int N, int NG, bool BF16, bool VEC, bool HAS_Z, bool CONV>
hipError_t launch_one(const ScanParams& p, const ScanShape& s, int n_main,
                      int main_base, int n_agg, hipStream_t stream) {
  const dim3 grid(n_main + n_agg), block(kLanes * NG);
  const ConvArgs cv{p.conv_w, p.conv_b, p.conv_init, p.u_out};
  if (p.softplus)
    hipLaunchKernelGGL((scan_kernel<N, NG, BF16, VEC, HAS_Z, true, CONV>), grid, block,
                       0, stream, p.u, p.delta, p.z, p.A, p.D, p.bias, p.out,
                       p.last_state, p.ws_S, p.ws_sum, p.ws_hin,
                       (const uint32_t*)p.ws_bc, s, n_main, main_base, cv);
  else
    hipLaunchKernelGGL((scan_kernel<N, NG, BF16, VEC, HAS_Z, false, CONV>), grid, block,
                       0, stream, p.u, p.delta, p.z, p.A, p.D, p.bias, p.out,
                       p.last_state, p.ws_S, p.ws_sum, p.ws_hin,
                       (const uint32_t*)p.ws_bc, s, n_main, main_base, cv);
  return hipGetLastError();
}

template <int N, int NG, bool BF16, bool VEC, bool CONV>
hipError_t launch_tasks(const ScanParams& p, const ScanShape& s, int n_main,
                        int main_base, int n_agg, hipStream_t stream) {
  if (p.z)
    return launch_one<N, NG, BF16, VEC, true, CONV>(p, s, n_main, main_base, n_agg, stream);
  return launch_one<N, NG, BF16, VEC, false, CONV>(p, s, n_main, main_base, n_agg, stream);
}

template <int N, bool BF16, bool VEC, bool CONV>
hipError_t launch_n(const ScanParams& p, hipStream_t stream) {
  constexpr int NG = kWaves<N>;
  ScanShape s;
  s.dim = p.dim;
  s.L = p.L;
  s.ts = p.layout_bld ? p.dim : 1;
  s.ngroups = p.ngroups > 1 ? p.ngroups : 1;
  s.groups_per_bc = p.groups_per_batch / s.ngroups;
  s.softplus = p.softplus;
  s.load_state = p.load_state;
  s.groups_per_batch = p.groups_per_batch;
  s.whole_groups = p.whole_groups;
  s.segments = p.segments;
  s.seg_len = p.seg_len;
  hipError_t e;
  {
    constexpr int WPS = BCLayout<N / NG, BF16>::kWordsPerStep;
    e = launch_bc_pack(p.B, p.C, p.ws_bc, p.batch, s.ngroups, p.L, p.L, N, NG, BF16,
                       BF16, bc_run_words(p.L, WPS), stream);
    if (e != hipSuccess) return e;
  }
  if (p.split_groups > 0 && p.whole_groups > 0 && p.side_stream) {
    // Two streams: the whole groups' main pass on the caller's stream, and
    // the split groups' chain (aggregate -> combine -> main) beside it on the
    // side stream, so that the chain runs on the CUs' spare workgroup slots.
    hipStream_t side = (hipStream_t)p.side_stream;
    e = hipEventRecord((hipEvent_t)p.ev_fork, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(side, (hipEvent_t)p.ev_fork, 0);
    if (e != hipSuccess) return e;
    e = launch_tasks<N, NG, BF16, VEC, CONV>(p, s, 0, 0, p.split_groups * (p.segments - 1), side);
    if (e != hipSuccess) return e;
    e = launch_combine(p, s, N, side);
    if (e != hipSuccess) return e;
    e = launch_tasks<N, NG, BF16, VEC, CONV>(p, s, p.split_groups * p.segments,
                                       p.whole_groups, 0, side);
    if (e != hipSuccess) return e;
    e = hipEventRecord((hipEvent_t)p.ev_join, side);
    if (e != hipSuccess) return e;
    if (p.ev_start) {
      e = hipEventRecord((hipEvent_t)p.ev_start, stream);
      if (e != hipSuccess) return e;
    }
    e = launch_tasks<N, NG, BF16, VEC, CONV>(p, s, p.whole_groups, 0, 0, stream);
    if (e == hipSuccess && p.ev_stop) e = hipEventRecord((hipEvent_t)p.ev_stop, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, (hipEvent_t)p.ev_join, 0);
    return e;
  }
  if (p.ev_start) {
    e = hipEventRecord((hipEvent_t)p.ev_start, stream);
    if (e != hipSuccess) return e;
  }
  if (p.split_groups > 0) {
    // one stream: whole groups' main pass + split groups' aggregate pass in
    // one launch, then the segment initial states, then the split groups'
    // main pass
    e = launch_tasks<N, NG, BF16, VEC, CONV>(p, s, p.whole_groups, 0,
                                       p.split_groups * (p.segments - 1), stream);
    if (e == hipSuccess) e = launch_combine(p, s, N, stream);
    if (e == hipSuccess)
      e = launch_tasks<N, NG, BF16, VEC, CONV>(p, s, p.split_groups * p.segments,
                                         p.whole_groups, 0, stream);
  } else {
    e = launch_tasks<N, NG, BF16, VEC, CONV>(p, s, p.whole_groups, 0, 0, stream);
  }
  if (e == hipSuccess && p.ev_stop) e = hipEventRecord((hipEvent_t)p.ev_stop, stream);
  return e;
}

template <int N, bool CONV>
hipError_t launch_dtype(const ScanParams& p, bool bf16, bool vec,
                        hipStream_t stream) {
  if (bf16)
    return vec ? launch_n<N, true, true, CONV>(p, stream)
               : launch_n<N, true, false, CONV>(p, stream);
  return vec ? launch_n<N, false, true, CONV>(p, stream)
             : launch_n<N, false, false, CONV>(p, stream);
}

template <int N>
hipError_t launch_conv(const ScanParams& p, bool bf16, bool vec,
                       hipStream_t stream) {
  return p.conv_w ? launch_dtype<N, true>(p, bf16, vec, stream)
                  : launch_dtype<N, false>(p, bf16, vec, stream);
}


}  // namespace fwd
}  // namespace mssm
