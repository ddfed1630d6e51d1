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
// the vector ALU (one v_exp_f32 per state element, which holds the VALU three to
// four times as long as an fma, plus four fp32 mul/fma), so the layout minimises
// issued VALU instructions:
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
//   * B_t and C_t are repacked once per call into one run per wave (the
//     wave's states of every token, in the io dtype), read with 64-byte
//     scalar loads;
//   * each lane reads its row's u / delta / z in 8- or 16-byte pieces, one
//     tile ahead of use, and writes its outputs with the same width; in the
//     (batch, length, channel) layout a lane instead takes 4 adjacent
//     channels of one step in the prep and output phases (kLdQuad).
// Long rows can be cut into time segments (aggregate tasks, then main tasks
// that fold the aggregates, in one launch): the recurrence is associative on
// (decay, offset) pairs, so a segment's effect on the state is
// (exp(A * sum Delta), local end state from zero).
#pragma once

#include <algorithm>

#include "dev_math.h"
#include "mssm_internal.h"
#include "scan_common.h"

namespace mssm {
namespace fwd {

constexpr int kTile = 32;  // timesteps per tile

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

// How a lane reaches a tile's u / delta / z / out in the prep and output
// phases:
//   kLdElem : one element at a time, any layout, length or alignment;
//   kLdRow  : (batch, dim, L) rows, L a multiple of 8, 16-byte aligned: 8- or
//             16-byte pieces of the lane's own row (lane = channel);
//   kLdQuad : (batch, L, dim), dim a multiple of 4, pointers aligned to 4
//             values: lane l takes channels 4 (l mod 16) .. +3 of the
//             workgroup's 64 at step l / 16 (+ 4 r), so one wave load is four
//             whole steps of the 64 channels, each one contiguous run.
// The state phase always has one channel per lane; the phases meet in LDS.
constexpr int kLdElem = 0;
constexpr int kLdRow = 1;
constexpr int kLdQuad = 2;
constexpr int kLdRowStaged = 3;  // kLdRow with the staged output store below
// With one channel per lane in the output phase (kLdElem, kLdRow), each
// wave's partial readouts sit in LDS as runs of 4 steps per lane
// ([wave][step / 4][lane] float4): the state phase writes a run once per 4
// steps and the output phase reads a wave's 4 steps with one 16-byte access.
constexpr bool kStepRunsY = true;
// kLdRowStaged (8 waves): the output phase computes a wave's 4 steps of the
// 64 channels (lane = channel), stages them in LDS and, after a barrier,
// stores them as wave g's 8 channels 8 g .. 8 g + 7 over the tile's 32 steps
// (lane l: channel 8 g + l / 8, steps 4 (l mod 8) ..), so that a store
// instruction writes 8 rows of 64 contiguous bytes (bf16) rather than 8 bytes
// of each of 64 rows; the scattered form makes about 6 times as many L2 write
// requests.  The extra barrier costs more than it saves when a CU holds one
// workgroup (nothing else runs while its waves meet), so the launch takes
// this mode only when it has more tasks than the device has CUs.

struct ScanShape {
  int64_t dim, L;
  int64_t ts;  // elements between consecutive timesteps of a row: 1, or dim
               // for the (batch, length, channel) layout
  int32_t ngroups, groups_per_bc;  // B/C groups; channel groups per B/C group
  int32_t softplus, load_state;
  int32_t groups_per_batch, whole_groups, split_groups, segments;
  int64_t seg_len;
};

// A main task waits for the aggregate tasks before it by polling their flags;
// each poll sleeps about 64 clocks.  The aggregates of its own launch are
// ahead of it in dispatch order and wait for nothing, so the wait ends; the
// limit (2^20 polls, well under a second) only bounds it should that ever
// fail, and the task then goes on with whatever the summaries hold.
constexpr uint32_t kFlagSpinLimit = 1u << 20;
// s_waitcnt operand waiting for every outstanding vector memory operation of
// the wave (vmcnt 0; the export and LDS/scalar counters left at their maxima)
constexpr int kWaitVmem0 = 0x0F70;

// kLdQuad: values 4 r .. 4 r + 3 of a chunk are the lane's 4 channels at its
// step of round r, read from byte offset off[r] of the lane's quad pointer
// (8 bytes in bf16, 16 in fp32).
template <bool BF16, int KC>
__device__ __forceinline__ void load_quads(Raw<BF16, KC>& r, const char* q,
                                           const int64_t (&off)[KC / 4]) {
#pragma unroll
  for (int i = 0; i < KC / 4; ++i) {
    if constexpr (BF16) {
      const uint2 v = *reinterpret_cast<const uint2*>(q + off[i]);
      r.w[2 * i] = v.x;
      r.w[2 * i + 1] = v.y;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(q + off[i]);
      r.w[4 * i] = v.x; r.w[4 * i + 1] = v.y; r.w[4 * i + 2] = v.z; r.w[4 * i + 3] = v.w;
    }
  }
}

template <bool BF16, int KC>
__device__ __forceinline__ void store_quads(char* q, const int64_t (&off)[KC / 4],
                                            const float (&o)[KC], const bool (&ok)[KC / 4]) {
#pragma unroll
  for (int i = 0; i < KC / 4; ++i) {
    if (!ok[i]) continue;
    if constexpr (BF16)
      *reinterpret_cast<uint2*>(q + off[i]) =
          make_uint2(pack_bf16x2(o[4 * i], o[4 * i + 1]), pack_bf16x2(o[4 * i + 2], o[4 * i + 3]));
    else
      *reinterpret_cast<uint4*>(q + off[i]) =
          make_uint4(__float_as_uint(o[4 * i]), __float_as_uint(o[4 * i + 1]),
                     __float_as_uint(o[4 * i + 2]), __float_as_uint(o[4 * i + 3]));
  }
}

// Main task (AGG = false): scans the task's time range from its initial
// state and writes out (and last_state after the final segment).  A task of
// segment k > 0 of a split group waits for the aggregates of segments
// 0..k-1 and folds them into its initial state, h = S_0 and then
// h = exp(A * sum_j Delta) h + S_j for j = 1..k-1, in fp64.
// Aggregate task (AGG = true): scans segment k < P-1 of a split group -- from
// the initial state for k = 0, from zero otherwise -- writes its end state
// S_k and its sum of Delta, then publishes them through the segment's flag:
// every wave waits for its own stores to complete, the workgroup meets at a
// barrier, and one thread stores the flag with an agent-scope release (one
// write-back of the XCD's L2 per aggregate rather than one per wave).
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
template <int N, int NG, bool BF16, int LD, bool HAS_Z, bool AGG, bool SOFTPLUS,
          bool CONV, bool WARM>
__device__ __forceinline__ void scan_body(
    const void* __restrict__ u, const void* __restrict__ delta,
    const void* __restrict__ z, const float* __restrict__ A,
    const float* __restrict__ Dv, const float* __restrict__ bias,
    void* __restrict__ out, float* __restrict__ last_state,
    float* __restrict__ ws_S, double* __restrict__ ws_sum,
    float* __restrict__ ws_h0, uint32_t* __restrict__ ws_flags,
    const uint32_t* __restrict__ bcp,
    const ScanShape& s, float2 (&s_dw)[kTile][kLanes],
    float (&s_y)[NG][kTile][kLanes], const int task, const ConvArgs& cv) {
  constexpr int NPW = N / NG;
  constexpr int T = kTile;
  constexpr int KC = T / NG;     // timesteps a wave prepares and emits
  constexpr int WPS = BCLayout<NPW, BF16>::kWordsPerStep;
  constexpr int KB = BCLayout<NPW, BF16>::kSteps;  // timesteps per batch
  constexpr int NB = T / KB;     // batches per tile
  constexpr bool VEC = LD == kLdRow || LD == kLdRowStaged;
  constexpr bool QUAD = LD == kLdQuad;
  constexpr int QR = KC / 4;     // kLdQuad: rounds of 4 steps per chunk
  static_assert(!(QUAD && CONV), "the conv-fed scan has no channel-quad path");
  constexpr bool Y4 = kStepRunsY && !QUAD;
  // s_y as runs of 4 steps: s_y4[wave][step / 4][lane]
  float4 (*const s_y4)[T / 4][kLanes] =
      reinterpret_cast<float4 (*)[T / 4][kLanes]>(&s_y[0][0][0]);

  const int lane = threadIdx.x & (kLanes - 1);
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = g * NPW;

  // task -> (group, segment); the split groups' tasks are segment-major, so
  // that the earliest segments' aggregates, and the main tasks that need the
  // fewest of them, come first in dispatch order
  int gi, seg, nseg, sg = 0;
  if constexpr (AGG) {
    seg = task / s.split_groups;
    sg = task % s.split_groups;
    gi = s.whole_groups + sg;
    nseg = s.segments;
  } else if (task < s.whole_groups) {
    gi = task;
    seg = 0;
    nseg = 1;
  } else {
    const int j = task - s.whole_groups;
    seg = j / s.split_groups;
    sg = j % s.split_groups;
    gi = s.whole_groups + sg;
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
  constexpr bool STAGE = LD == kLdRowStaged && kRowPtr && !AGG;
  static_assert(!STAGE || KC == 4, "the staged store takes 4 steps per lane");
  constexpr int64_t kEs = BF16 ? 2 : 4;
  // kLdQuad: the lane's channels cq .. cq + 3 (all in range or all out, as
  // dim is a multiple of 4; out of range reads the last 4 channels and stores
  // nothing), at step qs of each round of 4; steps sit qstride bytes apart
  const int qs = lane >> 4;
  const int64_t cq = (int64_t)(gi % s.groups_per_batch) * kLanes + 4 * (lane & 15);
  const bool qvalid = cq < s.dim;
  const uint32_t qstride = (uint32_t)(s.dim * kEs);
  const int64_t poff = QUAD ? b * s.L * s.dim + (qvalid ? cq : s.dim - 4) : rowoff;
  const char* const pu = static_cast<const char*>(u) + poff * kEs;
  const char* const pdl = static_cast<const char*>(delta) + poff * kEs;
  const char* const pz = HAS_Z ? static_cast<const char*>(z) + poff * kEs : nullptr;
  char* const po = AGG ? nullptr : static_cast<char*>(out) + poff * kEs;
  // STAGE: the staged store's channel and first step for this lane; wave g
  // stages its outputs in s_y4[g][g] (its own partials of its own steps,
  // which no other wave reads), at column lane ^ 2 g so that the store's
  // reads (8 step runs of 8 channels per 16 lanes) spread over the banks
  const int oa = lane & 7;
  const int64_t d_o = (int64_t)(gi % s.groups_per_batch) * kLanes + 8 * g + (lane >> 3);
  const bool valid_o = d_o < s.dim;
  char* const po_o =
      STAGE ? static_cast<char*>(out) +
                  ((b * s.dim + (valid_o ? d_o : s.dim - 1)) * s.L + 4 * oa) * kEs
            : nullptr;
  const uint32_t stg_w = (uint32_t)((9 * g * kLanes + (lane ^ (2 * g))) * 16);
  const uint32_t stg_r = (uint32_t)((9 * oa * kLanes + ((8 * g + (lane >> 3)) ^ (2 * oa))) * 16);
  // byte offsets of the rounds of the chunk at tc, the steps clamped into the
  // task (a clamped step re-reads values that nothing uses)
  auto quad_offsets = [&](int tc, int64_t (&off)[QR]) {
#pragma unroll
    for (int i = 0; i < QR; ++i)
      off[i] = (int64_t)((uint64_t)(uint32_t)min(tc + 4 * i + qs, t_end - 1) * qstride);
  };

  float A2[NPW], h[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    A2[j] = A[dc * N + n0 + j] * kLog2e;
    h[j] = 0.0f;
  }
  const int per = nseg - 1;  // aggregates of a split group
  if constexpr (AGG) {
    // segment 0 starts from the loaded state, and keeps it for its main task
    // (the final segment's main task overwrites last_state)
    if (seg == 0 && s.load_state) {
#pragma unroll
      for (int j = 0; j < NPW; ++j) {
        h[j] = last_state[row * N + n0 + j];
        ws_h0[sr * N + n0 + j] = h[j];
      }
    }
  } else if (nseg == 1) {
    if (s.load_state) {
#pragma unroll
      for (int j = 0; j < NPW; ++j) h[j] = last_state[row * N + n0 + j];
    }
  } else if (seg > 0 || s.load_state) {
    // wait for the summaries of the segments before this one (segment 0: the
    // kept initial state, published with segment 0's summary)
    if (threadIdx.x == 0) {
      const int nw = seg > 0 ? seg : 1;
      for (int q = 0; q < nw; ++q) {
        uint32_t it = 0;
        while (__hip_atomic_load(&ws_flags[q * s.split_groups + sg], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT) == 0u &&
               ++it < kFlagSpinLimit)
          __builtin_amdgcn_s_sleep(1);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    if (seg == 0) {
#pragma unroll
      for (int j = 0; j < NPW; ++j) h[j] = ws_h0[sr * N + n0 + j];
    } else {
      double hd[NPW];
#pragma unroll
      for (int j = 0; j < NPW; ++j) hd[j] = (double)ws_S[(sr * per + 0) * N + n0 + j];
      for (int q = 1; q < seg; ++q) {
        const double sum = ws_sum[sr * per + q];
#pragma unroll
        for (int j = 0; j < NPW; ++j)
          hd[j] = exp((double)A[dc * N + n0 + j] * sum) * hd[j] +
                  (double)ws_S[(sr * per + q) * N + n0 + j];
      }
#pragma unroll
      for (int j = 0; j < NPW; ++j) h[j] = (float)hd[j];
    }
  }
  const float bv_d = bias ? bias[dc] : 0.0f;
  const float Dd = (!AGG && Dv) ? Dv[dc] : 0.0f;
  double dsum = 0.0;
  // kLdQuad: bias and D of the lane's 4 channels; the aggregate's sums of
  // Delta per channel over the lane's steps
  float bq[4], Dq[4];
  double dq[4];
  if constexpr (QUAD) {
    const int64_t cqc = qvalid ? cq : s.dim - 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bq[j] = bias ? bias[cqc + j] : 0.0f;
      Dq[j] = (!AGG && Dv) ? Dv[cqc + j] : 0.0f;
      dq[j] = 0.0;
    }
  }

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
    if constexpr (QUAD) {
      // round i: the lane's 4 channels at tile step k, written as 4
      // consecutive (Delta, Delta*u) pairs of row k
#pragma unroll
      for (int i = 0; i < QR; ++i) {
        const int k = g * KC + 4 * i + qs;
        float dl[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = raw_get(pd, 4 * i + j) + bq[j];
          dl[j] = SOFTPLUS ? softplus_f32(x) : x;
          uv[4 * i + j] = raw_get(pu, 4 * i + j);
          if constexpr (AGG) {
            if (tile + k < t_end) dq[j] += (double)dl[j];
          }
        }
        float4* dst = reinterpret_cast<float4*>(&s_dw[k][4 * (lane & 15)]);
        dst[0] = make_float4(dl[0], dl[0] * uv[4 * i], dl[1], dl[1] * uv[4 * i + 1]);
        dst[1] = make_float4(dl[2], dl[2] * uv[4 * i + 2], dl[3], dl[3] * uv[4 * i + 3]);
      }
      return;
    }
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
  if constexpr (QUAD) {
    int64_t off[QR];
    quad_offsets(t_begin + g * KC, off);
    load_quads<BF16, KC>(ru, pu, off);
    load_quads<BF16, KC>(rd, pdl, off);
    if (HAS_Z && !AGG) load_quads<BF16, KC>(rz, pz, off);
    prep(ru, rd, uc, t_begin);
  } else {
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
    if constexpr (QUAD) {
      int64_t off[QR];
      quad_offsets(tb + T + g * KC, off);
      if (HAS_Z && !AGG) load_quads<BF16, KC>(nz, pz, off);
      load_quads<BF16, KC>(nu, pu, off);
      load_quads<BF16, KC>(nd, pdl, off);
    } else if constexpr (kRowPtr) {
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
      float yq[4];  // Y4: the readouts of the current run of 4 steps
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
          if constexpr (!AGG) {
            const int r = kb * KB + i;  // constant once unrolled
            if constexpr (Y4) {
              yq[r & 3] = y;
              if ((r & 3) == 3) s_y4[g][r >> 2][lane] = make_float4(yq[0], yq[1], yq[2], yq[3]);
            } else {
              s_y[g][r][lane] = y;
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      for (int kk = 0; kk < nt; ++kk) {
        uint32_t q[WPS];
#pragma unroll
        for (int j = 0; j < WPS; ++j) q[j] = bcw[((int64_t)tb + kk) * WPS + j];
        const float y = advance(s_dw[kk][lane], q, 0);
        if constexpr (!AGG) {
          if constexpr (Y4)
            reinterpret_cast<float*>(&s_y4[g][kk >> 2][lane])[kk & 3] = y;
          else
            s_y[g][kk][lane] = y;
        }
      }
    }
    __syncthreads();

    // Warm the scalar cache with the next tile's B/C run: one dword per
    // 64-byte line.  Scalar loads can only be waited on all together, so they
    // are issued here, where the first wait (the output phase's LDS reads)
    // comes after the whole prep phase.  WARM: plans whose groups all run
    // whole (one workgroup per CU) gain from it; with rows cut in time (two
    // workgroups per CU) it cost time, and so did a branch around it or the
    // same loads aimed at lines already cached, so the host picks a kernel
    // built with or without it.
    uint32_t touch = 0u;
    if constexpr (WARM) {
      // clamped to the row's steps in 32-bit arithmetic (L < 2^31 - 64): a
      // 64-bit clamp on word indices has no scalar compare and went to the VALU
      const int left = (int)s.L - (tb + T);  // steps of the next tile in the row
      const int tn = min(tb + T, (int)s.L - 1);
      const int fend = max(min(left, T) * WPS - 1, 0);
      const uint32_t* __restrict__ nb = bcw + (int64_t)tn * WPS;
#pragma unroll
      for (int f = 0; f < T * WPS; f += 16) touch += nb[min(f, fend)];
    }
    __builtin_amdgcn_sched_barrier(0);

    // prep of the next tile (its Delta/Delta*u slots are free: every wave is
    // past the state phase)
    if constexpr (CONV) conv_u(nu, np_, un);
    prep(nu, nd, un, tb + T);

    if constexpr (!AGG && QUAD) {
      // output phase, by channel quads: round i sums the partials of the
      // lane's 4 channels at tile step k
      float o[KC];
      int64_t off[QR];
      bool ok[QR];
      quad_offsets(tb + g * KC, off);
#pragma unroll
      for (int i = 0; i < QR; ++i) {
        const int k = g * KC + 4 * i + qs;
        ok[i] = qvalid && tb + k < t_end;
        float4 y = *reinterpret_cast<const float4*>(&s_y[0][k][4 * (lane & 15)]);
#pragma unroll
        for (int w = 1; w < NG; ++w) {
          const float4 p = *reinterpret_cast<const float4*>(&s_y[w][k][4 * (lane & 15)]);
          y.x += p.x; y.y += p.y; y.z += p.z; y.w += p.w;
        }
        const float ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float v = fmaf(Dq[j], uc[4 * i + j], ys[j]);
          if (HAS_Z) v *= silu_f32(raw_get(rz, 4 * i + j));
          o[4 * i + j] = v;
        }
      }
      store_quads<BF16, KC>(po, off, o, ok);
    } else if constexpr (!AGG) {
      // output phase: this wave's chunk of the tile
      const int tc = tb + g * KC;
      float o[KC], ys[KC];
      if constexpr (Y4) {
#pragma unroll
        for (int q = 0; q < KC / 4; ++q) {
          float4 v = s_y4[0][g * (KC / 4) + q][lane];
#pragma unroll
          for (int w = 1; w < NG; ++w) {
            const float4 p = s_y4[w][g * (KC / 4) + q][lane];
            v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
          }
          ys[4 * q] = v.x; ys[4 * q + 1] = v.y; ys[4 * q + 2] = v.z; ys[4 * q + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          ys[k] = s_y[0][g * KC + k][lane];
#pragma unroll
          for (int w = 1; w < NG; ++w) ys[k] += s_y[w][g * KC + k][lane];
        }
      }
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        float y = fmaf(Dd, uc[k], ys[k]);
        if (HAS_Z) y *= silu_f32(raw_get(rz, k));
        o[k] = y;
      }
      if constexpr (STAGE) {
        char* const lds_y = reinterpret_cast<char*>(&s_y[0][0][0]);
        *reinterpret_cast<float4*>(lds_y + stg_w) = make_float4(o[0], o[1], o[2], o[3]);
        __syncthreads();
        const float4 v = *reinterpret_cast<const float4*>(lds_y + stg_r);
        const float ov[4] = {v.x, v.y, v.z, v.w};
        if (valid_o) store_chunk_row<BF16, 4>(po_o, tb, ov, t_end - tb - 4 * oa);
        if constexpr (CONV) {
          if (valid && cv.u_out)
            store_chunk_row<BF16, KC>(static_cast<char*>(cv.u_out) + rowoff * kEs, tc, uc,
                                      t_end - tc);
        }
      } else if constexpr (kRowPtr) {
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
#pragma unroll
    for (int j = 0; j < NPW; ++j) ws_S[(sr * per + seg) * N + n0 + j] = h[j];
    // the segment's sum of Delta: the waves' sums over their own steps, added
    // in wave order (s_y is free: the loop ended on a barrier)
    double* part = reinterpret_cast<double*>(&s_y[0][0][0]);
    if constexpr (QUAD) {
      // per (wave, step of the round) and channel: NG * 4 * 64 doubles, within
      // s_y's NG * 32 * 64 floats
#pragma unroll
      for (int j = 0; j < 4; ++j) part[(g * 4 + qs) * kLanes + 4 * (lane & 15) + j] = dq[j];
      __syncthreads();
      if (g == 0) {
        double tot = 0.0;
#pragma unroll
        for (int w = 0; w < NG * 4; ++w) tot += part[w * kLanes + lane];
        ws_sum[sr * per + seg] = tot;
      }
    } else {
      part[g * kLanes + lane] = dsum;
      __syncthreads();
      if (g == 0) {
        double tot = 0.0;
#pragma unroll
        for (int w = 0; w < NG; ++w) tot += part[w * kLanes + lane];
        ws_sum[sr * per + seg] = tot;
      }
    }
    // publish: every wave waits for its own summary stores to complete, then
    // one release (write-back of this XCD's L2) ahead of the flag
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(&ws_flags[seg * s.split_groups + sg], 1u, __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_AGENT);
  } else {
    if (last_state && valid && seg == nseg - 1) {
#pragma unroll
      for (int j = 0; j < NPW; ++j) last_state[row * N + n0 + j] = h[j];
    }
  }
}

// One launch runs every task of a call: blocks [0, whole) are the whole
// groups' main tasks, the next n_agg blocks the split groups' aggregate
// tasks, the rest the split groups' main tasks.  The whole groups come first
// so that the dispatcher spreads them over the CUs, one each, ahead of the
// shorter split work; a main task only ever waits for aggregates, which are
// ahead of it in dispatch order and wait for nothing.
//
// The work plan counts on two workgroups per CU (16 waves, 4 per SIMD), so
// the kernel is held to 128 VGPRs.  At N = 128 that moves a few values of the
// fp64 fold in the prologue to scratch, once per task; the tile loop fits.
template <int N, int NG, bool BF16, int LD, bool HAS_Z, bool SOFTPLUS, bool CONV, bool WARM>
__global__ void __launch_bounds__(kLanes* NG) __attribute__((amdgpu_waves_per_eu(4)))
    scan_kernel(const void* __restrict__ u, const void* __restrict__ delta,
                const void* __restrict__ z, const float* __restrict__ A,
                const float* __restrict__ Dv, const float* __restrict__ bias,
                void* __restrict__ out, float* __restrict__ last_state,
                float* __restrict__ ws_S, double* __restrict__ ws_sum,
                float* __restrict__ ws_h0, uint32_t* __restrict__ ws_flags,
                const uint32_t* __restrict__ bcp, const ScanShape s,
                const int n_agg, const ConvArgs cv) {
  // 16-byte aligned: the channel-quad path moves 4 values per lane
  __shared__ __align__(16) float2 s_dw[kTile][kLanes];    // (Delta, Delta*u) of a tile
  __shared__ __align__(16) float s_y[NG][kTile][kLanes];  // per-wave partial readouts
  const int blk = blockIdx.x;
  const int a = blk - s.whole_groups;  // aggregate task, when in [0, n_agg)
  if (a >= 0 && a < n_agg)
    scan_body<N, NG, BF16, LD, HAS_Z, true, SOFTPLUS, CONV, WARM>(
        u, delta, z, A, Dv, bias, out, last_state, ws_S, ws_sum, ws_h0, ws_flags, bcp,
        s, s_dw, s_y, a, cv);
  else
    scan_body<N, NG, BF16, LD, HAS_Z, false, SOFTPLUS, CONV, WARM>(
        u, delta, z, A, Dv, bias, out, last_state, ws_S, ws_sum, ws_h0, ws_flags, bcp,
        s, s_dw, s_y, a < 0 ? blk : blk - n_agg, cv);
}


template <int N, int NG, bool BF16, int LD, bool HAS_Z, bool CONV>
hipError_t launch_one(const ScanParams& p, const ScanShape& s, int n_main, int n_agg,
                      hipStream_t stream) {
  const dim3 grid(n_main + n_agg), block(kLanes * NG);
  const ConvArgs cv{p.conv_w, p.conv_b, p.conv_init, p.u_out};
  // the scalar-cache warming pays only when no group is cut in time
  const bool warm = p.split_groups == 0;
#define MSSM_SCAN_LAUNCH(SP, WM)                                                            \
  hipLaunchKernelGGL((scan_kernel<N, NG, BF16, LD, HAS_Z, SP, CONV, WM>), grid, block, 0,  \
                     stream, p.u, p.delta, p.z, p.A, p.D, p.bias, p.out, p.last_state,     \
                     p.ws_S, p.ws_sum, p.ws_h0, p.ws_flags, (const uint32_t*)p.ws_bc, s,   \
                     n_agg, cv)
  if (p.softplus) {
    if (warm)
      MSSM_SCAN_LAUNCH(true, true);
    else
      MSSM_SCAN_LAUNCH(true, false);
  } else {
    if (warm)
      MSSM_SCAN_LAUNCH(false, true);
    else
      MSSM_SCAN_LAUNCH(false, false);
  }
#undef MSSM_SCAN_LAUNCH
  return hipGetLastError();
}

template <int N, int NG, bool BF16, int LD, bool CONV>
hipError_t launch_tasks(const ScanParams& p, const ScanShape& s, int n_main, int n_agg,
                        hipStream_t stream) {
  if (p.z)
    return launch_one<N, NG, BF16, LD, true, CONV>(p, s, n_main, n_agg, stream);
  return launch_one<N, NG, BF16, LD, false, CONV>(p, s, n_main, n_agg, stream);
}

template <int N, bool BF16, int LD, bool CONV>
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
  s.split_groups = p.split_groups;
  s.segments = p.segments;
  s.seg_len = p.seg_len;
  const int n_agg = p.split_groups > 0 ? p.split_groups * (p.segments - 1) : 0;
  const int n_main = p.whole_groups + p.split_groups * p.segments;
  hipError_t e;
  {
    // the pack also clears the aggregates' flags for the launch after it
    constexpr int WPS = BCLayout<N / NG, BF16>::kWordsPerStep;
    e = launch_bc_pack(p.B, p.C, p.ws_bc, p.batch, s.ngroups, p.L, p.L, N, NG, BF16,
                       BF16, bc_run_words(p.L, WPS), p.ws_flags, n_agg,
                       p.bc_state_major != 0, stream);
    if (e != hipSuccess) return e;
  }
  if (p.ev_start) {
    e = hipEventRecord((hipEvent_t)p.ev_start, stream);
    if (e != hipSuccess) return e;
  }
  e = launch_tasks<N, NG, BF16, LD, CONV>(p, s, n_main, n_agg, stream);
  if (e == hipSuccess && p.ev_stop) e = hipEventRecord((hipEvent_t)p.ev_stop, stream);
  return e;
}

// `vec`: the host found the vector path's conditions met for the call's
// layout (kLdRow for (batch, dim, L), kLdQuad for (batch, L, dim) without
// the conv)
template <int N, bool BF16, bool CONV>
hipError_t launch_ld(const ScanParams& p, bool vec, hipStream_t stream) {
  if (vec && !p.layout_bld) {
    if constexpr (kWaves<N> == 8) {
      const int64_t tasks = (int64_t)p.whole_groups + (int64_t)p.split_groups * (2 * p.segments - 1);
      if (tasks > p.cus) return launch_n<N, BF16, kLdRowStaged, CONV>(p, stream);
    }
    return launch_n<N, BF16, kLdRow, CONV>(p, stream);
  }
  if constexpr (!CONV) {
    if (vec) return launch_n<N, BF16, kLdQuad, CONV>(p, stream);
  }
  return launch_n<N, BF16, kLdElem, CONV>(p, stream);
}

template <int N, bool CONV>
hipError_t launch_dtype(const ScanParams& p, bool bf16, bool vec,
                        hipStream_t stream) {
  return bf16 ? launch_ld<N, true, CONV>(p, vec, stream)
              : launch_ld<N, false, CONV>(p, vec, stream);
}

template <int N>
hipError_t launch_conv(const ScanParams& p, bool bf16, bool vec,
                       hipStream_t stream) {
  return p.conv_w ? launch_dtype<N, true>(p, bf16, vec, stream)
                  : launch_dtype<N, false>(p, bf16, vec, stream);
}


}  // namespace fwd
}  // namespace mssm
