// scan_bwd.hip -- backward of the selective scan for gfx950 (CDNA4, wave64).
//
// Gradients of  sum_t dout_t out_t + sum_n dlast[n] h_{L-1}[n]  for one
// (batch b, channel d) row of the forward recurrence
//   Delta_t = softplus(x_t),  x_t = delta_t + bias[d]
//   e_t[n]  = exp(Delta_t A[d,n])
//   h_t[n]  = e_t[n] h_{t-1}[n] + Delta_t B_t[n] u_t
//   y_t     = sum_n C_t[n] h_t[n] + D[d] u_t,   out_t = y_t silu(z_t)
// (page "Mamba: Selective State Space Models", "Mathematical Foundation":
// the selective recurrence, trained through its parallel scan, section
// "Efficient Scan").  With g_t[n] = dLoss/dh_t[n], run backwards in time:
//   dy_t      = dout_t silu(z_t),     dz_t = dout_t y_t silu'(z_t)
//   g_t       = dy_t C_t + e_{t+1} g_{t+1}         (g_{L-1} adds dlast)
//   dC_t[n]  += dy_t h_t[n]            dB_t[n] += g_t[n] Delta_t u_t
//   du_t      = Delta_t sum_n g_t[n] B_t[n] + D dy_t
//   dDelta_t  = u_t sum_n g_t[n] B_t[n] + sum_n A[n] g_t[n] e_t[n] h_{t-1}[n]
//   ddelta_t  = dDelta_t sigmoid(x_t)    (softplus' = sigmoid)
//   dA[n]    += Delta_t g_t[n] e_t[n] h_{t-1}[n]
//   dD       += dy_t u_t,   dbias += ddelta_t,   dh0 = e_0 g_0
// dB, dC sum over channels and dA, dD, dbias over the batch.
//
// Time segments.  Both recurrences are linear, so a row cut into segments
// is joined by two carries per state: the state entering a segment and the
// gradient entering it from the end.  For a segment scanned from zero,
//   end state  S = h_end from h = 0,   decay over it  P = exp(A sum Delta)
//   reverse aggregate  R = sum_t E_t dy_t C_t,  E_t = exp(A sum_{start..t} Delta)
// (R is what the reverse recurrence carries to the segment start for a zero
// incoming gradient; E_t is a running product, so R is formed in the forward
// sweep and no extra reverse sweep is needed).  Then
//   h_in[s+1] = P_s h_in[s] + S_s,      g_in[s-1] = P_s g_in[s] + R_s
// and a state kept inside segment s at a point with running sum c is
// h = h(from zero) + exp(A c) h_in[s].
//
// Kernels (all rows and segments in parallel):
//   pass F   : scans each segment from zero with the recurrence above, keeping
//              the state and running sum of Delta at every 16-step tile, and
//              S, R, sum Delta of the segment;
//   combine  : h_in and g_in of every segment (fp64 decay);
//   pass R   : per segment, tiles in reverse: recompute e_t, h_t of the tile
//              into registers from its corrected checkpoint, run the reverse
//              recurrence, emit du, ddelta, dz and the partial sums;
//   reduce   : dB, dC over channel groups; dA, dD, dbias over batch and
//              segments (fixed order: deterministic).
// Mapping: one lane per channel, 64 channels of one batch entry per
// workgroup, the N states split over NG waves (4 each).  B_t and C_t are
// wave-uniform and read with wide scalar loads from a per-wave packed run
// (zero-padded to whole tiles); the next tile's lines are touched one tile
// ahead so that those loads hit the scalar cache.  Sums over n of a channel
// (y, g.B, A g e h) go through LDS to the wave that owns the timestep; dB and
// dC need sums over the 64 channels of a wave: 16 values per lane are
// written to a per-wave LDS block and read back transposed, so each lane adds
// 16 values and two DPP steps finish the sum.
#include <algorithm>
#include <atomic>

#include "dev_math.h"
#include "mssm_internal.h"
#include "scan_common.h"

namespace mssm {
namespace {

constexpr int kT = 16;                 // timesteps per tile (and checkpoint)
constexpr int kRedItems = 16;          // values per lane per channel reduction
constexpr int kRedPitch = kLanes + 4;  // padded row: conflict-free b128 reads
constexpr int kMinSegTiles = 4;        // shortest segment the plan makes

// Waves per 64-channel workgroup: four states per wave.
template <int N>
constexpr int kBwdWaves = N >= 4 ? N / 4 : 1;

struct BwdShape {
  int64_t dim, L;
  int64_t ts;  // elements between consecutive timesteps of a row: 1, or dim
               // for the (batch, length, channel) layout
  int32_t ngroups, reserved;  // B/C groups
  int32_t groups_per_batch, tiles;
  int32_t segments, seg_tiles;
  int32_t softplus, batch;
};

// LDS traffic between lanes of one wave: the wave's LDS operations complete
// in order, so only the compiler has to be kept from moving them.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int CTRL>
__device__ __forceinline__ float dpp_quad(float v) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum of v[k] over the 64 lanes of the wave, for k < kRedItems, in two
// halves: red_put writes the items, red_take (any time later, before the
// next red_put) reads them back transposed and returns, in lanes 4k .. 4k+3,
// the sum of item k.  Work placed between the two hides the writes' latency.
__device__ __forceinline__ void red_put(float (&red)[kRedItems][kRedPitch],
                                        const float (&v)[kRedItems], int lane) {
#pragma unroll
  for (int k = 0; k < kRedItems; ++k) red[k][lane] = v[k];
}
__device__ __forceinline__ float red_take(float (&red)[kRedItems][kRedPitch], int lane) {
  wave_lds_sync();
  const float4* row = reinterpret_cast<const float4*>(&red[lane >> 2][16 * (lane & 3)]);
  const float4 a = row[0], b = row[1], c = row[2], d = row[3];
  float s = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w)) +
            (((c.x + c.y) + (c.z + c.w)) + ((d.x + d.y) + (d.z + d.w)));
  s += dpp_quad<0xB1>(s);  // quad_perm [1,0,3,2]
  s += dpp_quad<0x4E>(s);  // quad_perm [2,3,0,1]
  wave_lds_sync();
  return s;
}

// Touch one dword in each 64-byte line of a tile's packed B/C run so that the
// tile's wide scalar loads later hit the scalar cache.
template <int WPS>
__device__ __forceinline__ uint32_t warm_tile(const uint32_t* __restrict__ bcw,
                                              int64_t tile) {
  uint32_t touch = 0u;
  const int64_t f0 = tile * kT * WPS;
#pragma unroll
  for (int f = 0; f < kT * WPS; f += 16) touch += bcw[f0 + f];
  return touch;
}

// Per-task indices shared by both passes.
struct Task {
  int gi, seg;
  int64_t b, d, dc, row, rowoff;
  int64_t bcg;  // run of B/C: batch entry * groups + the channel group's B/C group
  bool valid;
  int tile_begin, tile_end;
};

__device__ __forceinline__ Task task_of(const BwdShape& s, int lane) {
  Task k;
  const int task = blockIdx.x;
  k.gi = task / s.segments;
  k.seg = task - k.gi * s.segments;
  k.b = k.gi / s.groups_per_batch;
  k.d = (int64_t)(k.gi % s.groups_per_batch) * kLanes + lane;
  k.valid = k.d < s.dim;
  k.dc = k.valid ? k.d : s.dim - 1;
  k.row = k.b * s.dim + k.dc;
  k.rowoff = s.ts == 1 ? k.row * s.L : k.b * s.L * s.dim + k.dc;
  k.bcg = k.b * s.ngroups + (k.gi % s.groups_per_batch) / (s.groups_per_batch / s.ngroups);
  k.tile_begin = k.seg * s.seg_tiles;
  k.tile_end = min(s.tiles, k.tile_begin + s.seg_tiles);
  return k;
}

// ---------------------------------------------------------------- pass F ---
template <int N, int NG, bool BF16, bool VEC, bool HAS_Z>
__global__ void __launch_bounds__(kLanes* NG)
    bwd_pass_f_kernel(const void* __restrict__ u, const void* __restrict__ delta,
                      const void* __restrict__ z, const void* __restrict__ dout,
                      const float* __restrict__ A, const float* __restrict__ bias,
                      float* __restrict__ ws_ck, float* __restrict__ ws_cd,
                      float* __restrict__ ws_S, float* __restrict__ ws_R,
                      double* __restrict__ ws_sum,
                      const uint32_t* __restrict__ bcp, const BwdShape s) {
  constexpr int NPW = N / NG;
  constexpr int T = kT;
  constexpr int KC = T / NG;
  constexpr int WPS = BCLayout<NPW, BF16>::kWordsPerStep;
  constexpr int KB = BCLayout<NPW, BF16>::kSteps;
  constexpr int NB = T / KB;
  using Batch = BCBatch<NPW, BF16>;
  __shared__ float2 s_dw[2][T][kLanes];  // (Delta, Delta*u), double-buffered
  __shared__ float s_dy[2][T][kLanes];   // dout * silu(z)
  __shared__ double s_ds[2][NG][kLanes];  // each wave's sum of its steps' Delta

  const int lane = threadIdx.x & (kLanes - 1);
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = g * NPW;
  const Task k = task_of(s, lane);
  const int64_t Lp = (int64_t)s.tiles * T;
  const uint32_t* __restrict__ bcw = bcp + (k.bcg * NG + g) * Lp * WPS;
  const bool sp = s.softplus != 0;

  float A2[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) A2[j] = A[k.dc * N + n0 + j] * kLog2e;
  const float bv = bias ? bias[k.dc] : 0.0f;

  Raw<BF16, KC> ru, rd, rz, ro;
  raw_zero(rz);
  // N = 16 with bf16 rows: the next tile's inputs are read by channel runs
  // (lane l of wave g: channel 16 g + l / 4 of the group, steps 4 (l mod 4)
  // .., so a load moves 16 rows of 32 contiguous bytes rather than 8 bytes of
  // each of 64 rows) and meet the lanes that own their channels in LDS; the
  // staging rows hold a channel's 16 steps as four 8-byte pieces, piece p at
  // slot p ^ ((channel / 8) mod 4), free of bank conflicts both ways.
  constexpr bool kStageIn = VEC && BF16 && NG == 4 && KC == 4;
  __shared__ __align__(16) char s_stg[kStageIn ? 4 * kLanes * 32 : 16];
  const int c_st = (kLanes / NG) * g + (lane >> 2);
  const int q_st = lane & 3;
  const int64_t d_st = (int64_t)(k.gi % s.groups_per_batch) * kLanes + c_st;
  const int64_t row_st = k.b * s.dim + (d_st < s.dim ? d_st : s.dim - 1);
  auto stg_at = [&](int tt, int c, int piece) -> uint2* {
    return reinterpret_cast<uint2*>(s_stg + (tt * kLanes + c) * 32 + 8 * (piece ^ ((c >> 3) & 3)));
  };
  auto load_staged = [&](int tile) {
    const int64_t t = (int64_t)tile * T + 4 * q_st;
    const int64_t nv = s.L - t;
    const int64_t off = row_st * s.L + t;
    load_chunk<BF16, true, KC>(ru, u, off, nv);
    load_chunk<BF16, true, KC>(rd, delta, off, nv);
    if constexpr (HAS_Z) load_chunk<BF16, true, KC>(rz, z, off, nv);
    load_chunk<BF16, true, KC>(ro, dout, off, nv);
  };
  // hand the staged pieces to their lanes (every wave, behind one barrier)
  auto unstage = [&]() {
    if constexpr (kStageIn) {
      *stg_at(0, c_st, q_st) = make_uint2(ru.w[0], ru.w[1]);
      *stg_at(1, c_st, q_st) = make_uint2(rd.w[0], rd.w[1]);
      if constexpr (HAS_Z) *stg_at(2, c_st, q_st) = make_uint2(rz.w[0], rz.w[1]);
      *stg_at(3, c_st, q_st) = make_uint2(ro.w[0], ro.w[1]);
      __syncthreads();
      uint2 v = *stg_at(0, lane, g);
      ru.w[0] = v.x; ru.w[1] = v.y;
      v = *stg_at(1, lane, g);
      rd.w[0] = v.x; rd.w[1] = v.y;
      if constexpr (HAS_Z) {
        v = *stg_at(2, lane, g);
        rz.w[0] = v.x; rz.w[1] = v.y;
      }
      v = *stg_at(3, lane, g);
      ro.w[0] = v.x; ro.w[1] = v.y;
    }
  };
  // Time indices are 32-bit (the host keeps L below 2^31 - 64).  On the
  // vector path with chunks of at most 8 steps (L a multiple of 8, so
  // L >= KC) each lane keeps pointers to its own rows and a chunk's start is
  // clamped to the row's last chunk: no branch or 64-bit compare per load;
  // prep zeroes the steps past L.
  constexpr bool kRowPtr = VEC && KC <= 8;
  const int Lr = (int)s.L;
  constexpr int64_t kEs = BF16 ? 2 : 4;
  const char* const pu = static_cast<const char*>(u) + k.rowoff * kEs;
  const char* const pdl = static_cast<const char*>(delta) + k.rowoff * kEs;
  const char* const pz = HAS_Z ? static_cast<const char*>(z) + k.rowoff * kEs : nullptr;
  const char* const pdo = static_cast<const char*>(dout) + k.rowoff * kEs;
  auto load = [&](int tile) {
    const int tc = tile * T + g * KC;
    if constexpr (kRowPtr) {
      const int tl = min(tc, Lr - KC);
      load_chunk_row<BF16, KC>(ru, pu, tl);
      load_chunk_row<BF16, KC>(rd, pdl, tl);
      if constexpr (HAS_Z) load_chunk_row<BF16, KC>(rz, pz, tl);
      load_chunk_row<BF16, KC>(ro, pdo, tl);
    } else {
      const int nv = Lr - tc;
      const int64_t off = k.rowoff + (int64_t)tc * s.ts;
      load_chunk<BF16, VEC, KC>(ru, u, off, nv, s.ts);
      load_chunk<BF16, VEC, KC>(rd, delta, off, nv, s.ts);
      if constexpr (HAS_Z) load_chunk<BF16, VEC, KC>(rz, z, off, nv, s.ts);
      load_chunk<BF16, VEC, KC>(ro, dout, off, nv, s.ts);
    }
  };
  // (Delta, Delta*u) and dout*silu(z) of this wave's chunk into LDS, and the
  // fp64 sum of the chunk's Delta (the waves' sums give the tile's sum)
  auto prep = [&](int tile, int buf) {
    const int nv = Lr - (tile * T + g * KC);
    double ds = 0.0;
#pragma unroll
    for (int q = 0; q < KC; ++q) {
      const bool ok = k.valid && q < nv;
      const float x = raw_get(rd, q) + bv;
      float dl = sp ? softplus_f32(x) : x;
      float dyv = raw_get(ro, q);
      if constexpr (HAS_Z) dyv *= silu_f32(raw_get(rz, q));
      dl = ok ? dl : 0.0f;
      dyv = ok ? dyv : 0.0f;
      s_dw[buf][g * KC + q][lane] = make_float2(dl, dl * raw_get(ru, q));
      s_dy[buf][g * KC + q][lane] = dyv;
      ds += (double)dl;
    }
    s_ds[buf][g][lane] = ds;
  };

  float h[NPW], E[NPW], Rg[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    h[j] = 0.0f;
    E[j] = 1.0f;
    Rg[j] = 0.0f;
  }
  double cum = 0.0;
  float* __restrict__ ck = ws_ck + (int64_t)k.gi * s.tiles * N * kLanes;
  float* __restrict__ cd = ws_cd + (int64_t)k.gi * s.tiles * kLanes;

  load(k.tile_begin);
  prep(k.tile_begin, 0);
  __syncthreads();
  for (int ti = k.tile_begin; ti < k.tile_end; ++ti) {
    const int cur = (ti - k.tile_begin) & 1;
    const bool more = ti + 1 < k.tile_end;
    if (more) {
      if constexpr (kStageIn)
        load_staged(ti + 1);
      else
        load(ti + 1);
    }
    const uint32_t touch = more ? warm_tile<WPS>(bcw, ti + 1) : 0u;
#pragma unroll
    for (int j = 0; j < NPW; ++j) ck[((int64_t)ti * N + n0 + j) * kLanes + lane] = h[j];
    if (g == 0) cd[(int64_t)ti * kLanes + lane] = (float)cum;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      const Batch bc = *reinterpret_cast<const Batch*>(bcw + ((int64_t)ti * T + kb * KB) * WPS);
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const float2 dw = s_dw[cur][kb * KB + i][lane];
        const float dyv = s_dy[cur][kb * KB + i][lane];
#pragma unroll
        for (int j = 0; j < NPW; ++j) {
          const float e = hw_exp2(dw.x * A2[j]);
          h[j] = fmaf(e, h[j], dw.y * bc_val<NPW, BF16>(bc.w, i, j));
          E[j] *= e;
          Rg[j] = fmaf(E[j], dyv * bc_val<NPW, BF16>(bc.w, i, NPW + j), Rg[j]);
        }
      }
    }
    // the tile's sum of Delta, the waves' chunk sums in wave order
#pragma unroll
    for (int w = 0; w < NG; ++w) cum += s_ds[cur][w][lane];
    if (more) {
      if constexpr (kStageIn) unstage();
      prep(ti + 1, cur ^ 1);
    }
    asm volatile("" ::"s"(touch));  // keeps the warming loads
    __syncthreads();
  }
  const int64_t task = blockIdx.x;
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    ws_S[(task * N + n0 + j) * kLanes + lane] = h[j];
    ws_R[(task * N + n0 + j) * kLanes + lane] = Rg[j];
  }
  if (g == 0) ws_sum[task * kLanes + lane] = cum;
}

// --------------------------------------------------------------- combine ---
// Initial state and incoming end gradient of every segment, per (task row,
// state); fp64 decay exp(A sum Delta).
__global__ void __launch_bounds__(256)
    bwd_combine_kernel(const float* __restrict__ A, const float* __restrict__ h0,
                       const float* __restrict__ dlast,
                       const float* __restrict__ ws_S,
                       const float* __restrict__ ws_R,
                       const double* __restrict__ ws_sum,
                       float* __restrict__ ws_hin, float* __restrict__ ws_gin,
                       const BwdShape s, int N, int64_t groups) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= groups * N * kLanes) return;
  const int lane = (int)(tid % kLanes);
  const int64_t r = tid / kLanes;
  const int n = (int)(r % N);
  const int64_t gi = r / N;
  const int P = s.segments;
  const int64_t b = gi / s.groups_per_batch;
  const int64_t d = (gi % s.groups_per_batch) * kLanes + lane;
  auto at = [&](int seg) { return ((gi * P + seg) * N + n) * kLanes + lane; };
  if (d >= s.dim) {
    for (int q = 0; q < P; ++q) ws_hin[at(q)] = ws_gin[at(q)] = 0.0f;
    return;
  }
  const double a = A[d * N + n];
  const int64_t si = (b * s.dim + d) * N + n;
  double h = h0 ? h0[si] : 0.0;
  for (int q = 0; q < P; ++q) {
    ws_hin[at(q)] = (float)h;
    h = exp(a * ws_sum[(gi * P + q) * kLanes + lane]) * h + (double)ws_S[at(q)];
  }
  double gr = dlast ? dlast[si] : 0.0;
  for (int q = P - 1; q >= 0; --q) {
    ws_gin[at(q)] = (float)gr;
    gr = exp(a * ws_sum[(gi * P + q) * kLanes + lane]) * gr + (double)ws_R[at(q)];
  }
}

// ---------------------------------------------------------------- pass R ---
template <int N, int NG>
struct alignas(16) BwdSmem {
  float2 dw[kT][kLanes];                // (Delta, Delta*u) of the tile
  float dy[kT][kLanes];                 // dout * silu(z)
  float y[NG][kT][kLanes];              // per-wave partial readouts
  float2 s[NG][kT][kLanes];             // per-wave (sum g B, sum A g e h_prev)
  float red[NG][kRedItems][kRedPitch];  // per-wave channel-sum transpose
  float dbc[kT][2 * N];                 // the tile's channel sums of dB, dC
};

// Two waves per SIMD (two 4-wave workgroups per CU at N <= 16) need at most
// 256 VGPRs per wave.
template <int N, int NG, bool BF16, bool VEC, bool HAS_Z>
__global__ void __launch_bounds__(kLanes* NG) __attribute__((amdgpu_waves_per_eu(2)))
    bwd_pass_r_kernel(const void* __restrict__ u, const void* __restrict__ delta,
                      const void* __restrict__ z, const void* __restrict__ dout,
                      const float* __restrict__ A, const float* __restrict__ Dv,
                      const float* __restrict__ bias, void* __restrict__ du,
                      void* __restrict__ ddelta, void* __restrict__ dz,
                      float* __restrict__ dh0, const float* __restrict__ ws_ck,
                      const float* __restrict__ ws_cd,
                      const float* __restrict__ ws_hin,
                      const float* __restrict__ ws_gin,
                      float* __restrict__ ws_dbc, float* __restrict__ ws_dA,
                      float* __restrict__ ws_dDb,
                      const uint32_t* __restrict__ bcp, const BwdShape s) {
  constexpr int NPW = N / NG;
  constexpr int T = kT;
  constexpr int KC = T / NG;  // timesteps a wave prepares and emits per tile
  constexpr int WPS = BCLayout<NPW, BF16>::kWordsPerStep;
  constexpr int KB = BCLayout<NPW, BF16>::kSteps;  // timesteps per B/C batch
  constexpr int NB = T / KB;
  constexpr int RS = kRedItems / (2 * NPW);  // timesteps per channel reduction
  static_assert(T % KB == 0 && KB % RS == 0, "tile, batch and reduction nest");
  using Batch = BCBatch<NPW, BF16>;
  __shared__ BwdSmem<N, NG> sm;
  // staged output stores: (batch, dim, L) rows of bf16, 4 waves of 4 steps
  constexpr bool kStageOut = VEC && BF16 && NG == 4 && KC == 4;
  // Staging rows: per tensor (du, ddelta, dz, then u, delta, z, dout) and
  // channel, the tile's 16 steps as four 8-byte pieces, piece p at slot
  // p ^ ((channel / 8) mod 4) so that both access patterns below are free
  // of bank conflicts.
  constexpr int kStgPitch = 32;
  static_assert(!kStageOut || 7 * kLanes * kStgPitch <= (int)sizeof(sm.red),
                "staging fits in the reduction blocks");
  char* const stg = reinterpret_cast<char*>(&sm.red[0][0][0]);
  auto stg_at = [&](int tt, int c, int piece) -> uint2* {
    return reinterpret_cast<uint2*>(stg + (tt * kLanes + c) * kStgPitch +
                                    8 * (piece ^ ((c >> 3) & 3)));
  };

  const int lane = threadIdx.x & (kLanes - 1);
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = g * NPW;
  // the staged accesses' lane mapping: channel 16 g + lane / 4 of the
  // group, steps 4 (lane mod 4) .. of the tile
  const int c_st = (kLanes / NG) * g + (lane >> 2);
  const int q_st = lane & 3;
  const Task k = task_of(s, lane);
  const int64_t task = blockIdx.x;
  const int64_t Lp = (int64_t)s.tiles * T;
  const uint32_t* __restrict__ bcw = bcp + (k.bcg * NG + g) * Lp * WPS;
  const float* __restrict__ ck = ws_ck + (int64_t)k.gi * s.tiles * N * kLanes;
  const float* __restrict__ cd = ws_cd + (int64_t)k.gi * s.tiles * kLanes;
  const bool sp = s.softplus != 0;

  float A2[NPW], Av[NPW], hin[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    Av[j] = A[k.dc * N + n0 + j];
    A2[j] = Av[j] * kLog2e;
    hin[j] = ws_hin[(task * N + n0 + j) * kLanes + lane];
  }
  const float bv = bias ? bias[k.dc] : 0.0f;
  const float Dd = Dv ? Dv[k.dc] : 0.0f;

  float gr[NPW], dA[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    gr[j] = ws_gin[(task * N + n0 + j) * kLanes + lane];
    dA[j] = 0.0f;
  }
  float dDacc = 0.0f, dbacc = 0.0f;
  // prepared values of this wave's chunk of the current tile
  float cD[KC], cS[KC], cU[KC], cDy[KC], cDz[KC];
  Raw<BF16, KC> nu, nd, nz, no;
  raw_zero(nz);

  auto prep_r = [&](int64_t tile_base) {
    const int64_t nv = s.L - (tile_base + g * KC);
#pragma unroll
    for (int q = 0; q < KC; ++q) {
      const bool ok = k.valid && q < nv;
      const float uu = raw_get(nu, q);
      const float x = raw_get(nd, q) + bv;
      float dl = x, sg = 1.0f;
      if (sp) {
        dl = softplus_f32(x);
        sg = hw_rcp(1.0f + hw_exp2(-x * kLog2e));
      }
      const float o = raw_get(no, q);
      float dyv = o, dzf = 0.0f;
      if constexpr (HAS_Z) {
        const float zz = raw_get(nz, q);
        const float sz = hw_rcp(1.0f + hw_exp2(-zz * kLog2e));
        dyv = o * (zz * sz);
        dzf = o * (sz * fmaf(zz, 1.0f - sz, 1.0f));
      }
      if (!ok) {
        dl = 0.0f;
        dyv = 0.0f;
        dzf = 0.0f;
      }
      cD[q] = dl;
      cS[q] = sg;
      cU[q] = uu;
      cDy[q] = dyv;
      cDz[q] = dzf;
      sm.dw[g * KC + q][lane] = make_float2(dl, dl * uu);
      sm.dy[g * KC + q][lane] = dyv;
    }
  };
  // kStageOut: the next tile's inputs are read by channel runs (16 rows of
  // 32 bytes per instruction) and meet the lanes that own their channels in
  // LDS in the output phase
  const int64_t d_st = (int64_t)(k.gi % s.groups_per_batch) * kLanes + c_st;
  const int64_t row_st = (int64_t)k.b * s.dim + (d_st < s.dim ? d_st : s.dim - 1);
  auto load_r_staged = [&](int64_t tile_base) {
    const int64_t t = tile_base + 4 * q_st;
    const int64_t nv = s.L - t;
    const int64_t off = row_st * s.L + t;
    load_chunk<BF16, true, KC>(nu, u, off, nv);
    load_chunk<BF16, true, KC>(nd, delta, off, nv);
    if constexpr (HAS_Z) load_chunk<BF16, true, KC>(nz, z, off, nv);
    load_chunk<BF16, true, KC>(no, dout, off, nv);
  };
  auto load_r = [&](int64_t tile_base) {
    const int64_t tc = tile_base + g * KC;
    const int64_t nv = s.L - tc;
    const int64_t off = k.rowoff + tc * s.ts;
    load_chunk<BF16, VEC, KC>(nu, u, off, nv, s.ts);
    load_chunk<BF16, VEC, KC>(nd, delta, off, nv, s.ts);
    if constexpr (HAS_Z) load_chunk<BF16, VEC, KC>(nz, z, off, nv, s.ts);
    load_chunk<BF16, VEC, KC>(no, dout, off, nv, s.ts);
  };
  // state at the start of a tile: kept from zero, plus the decayed h_in
  // The checkpoint is loaded a tile ahead and combined where it is used: an
  // arithmetic use right after the load would wait for every load in flight.
  auto load_checkpoint = [&](int tile, float (&raw)[NPW + 1]) {
#pragma unroll
    for (int j = 0; j < NPW; ++j) raw[j] = ck[((int64_t)tile * N + n0 + j) * kLanes + lane];
    raw[NPW] = cd[(int64_t)tile * kLanes + lane];
  };
  auto finish_checkpoint = [&](const float (&raw)[NPW + 1], float (&hc)[NPW]) {
#pragma unroll
    for (int j = 0; j < NPW; ++j) hc[j] = fmaf(hw_exp2(A2[j] * raw[NPW]), hin[j], raw[j]);
  };

  const int last = k.tile_end - 1;
  load_r((int64_t)last * T);
  prep_r((int64_t)last * T);
  float hck[NPW];
  {
    float raw[NPW + 1];
    load_checkpoint(last, raw);
    finish_checkpoint(raw, hck);
  }
  __syncthreads();

  for (int ti = last; ti >= k.tile_begin; --ti) {
    const int64_t tb = (int64_t)ti * T;
    const bool more = ti > k.tile_begin;
    // prefetch the previous tile's inputs and checkpoint, warm its B/C lines
    float hraw[NPW + 1];
    if (more) {
      if constexpr (kStageOut)
        load_r_staged(tb - T);
      else
        load_r(tb - T);
      load_checkpoint(ti - 1, hraw);
    }
    const uint32_t touch = more ? warm_tile<WPS>(bcw, ti - 1) : 0u;

    // recompute e_t and h_t of the tile (and the partial readouts for dz)
    float e[T][NPW], H[T][NPW];
    {
      float hc[NPW];
#pragma unroll
      for (int j = 0; j < NPW; ++j) hc[j] = hck[j];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        const Batch bc = *reinterpret_cast<const Batch*>(bcw + (tb + kb * KB) * WPS);
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          const int t = kb * KB + i;
          const float2 dw = sm.dw[t][lane];
          float y = 0.0f;
#pragma unroll
          for (int j = 0; j < NPW; ++j) {
            e[t][j] = hw_exp2(dw.x * A2[j]);
            hc[j] = fmaf(e[t][j], hc[j], dw.y * bc_val<NPW, BF16>(bc.w, i, j));
            H[t][j] = hc[j];
            if constexpr (HAS_Z) y = fmaf(bc_val<NPW, BF16>(bc.w, i, NPW + j), hc[j], y);
          }
          if constexpr (HAS_Z) sm.y[g][t][lane] = y;
        }
      }
    }

    // reverse recurrence over the tile.  The channel sums of dB and dC of a
    // unit of RS steps are taken back while the next unit computes.
    int pend_t = -1;  // first step of the unit whose sums are in flight
    auto take_sums = [&]() {
      const float tot = red_take(sm.red[g], lane);
      if ((lane & 3) == 0) {
        const int kk = lane >> 2;
        const int j = kk % NPW;
        const int q = (kk / NPW) & 1;
        const int ii = kk / (2 * NPW);
        sm.dbc[pend_t + ii][q * N + n0 + j] = tot;
      }
    };
#pragma unroll
    for (int kb = NB - 1; kb >= 0; --kb) {
      const Batch bc = *reinterpret_cast<const Batch*>(bcw + (tb + kb * KB) * WPS);
#pragma unroll
      for (int ru = KB / RS - 1; ru >= 0; --ru) {
        float pv[kRedItems];
#pragma unroll
        for (int ii = RS - 1; ii >= 0; --ii) {
          const int i = ru * RS + ii;
          const int t = kb * KB + i;
          const float2 dw = sm.dw[t][lane];
          const float dyv = sm.dy[t][lane];
          float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
          for (int j = 0; j < NPW; ++j) {
            const float Bv = bc_val<NPW, BF16>(bc.w, i, j);
            const float Cv = bc_val<NPW, BF16>(bc.w, i, NPW + j);
            gr[j] = fmaf(dyv, Cv, gr[j]);
            pv[(ii * 2 + 0) * NPW + j] = gr[j] * dw.y;    // dB term
            pv[(ii * 2 + 1) * NPW + j] = dyv * H[t][j];   // dC term
            s1 = fmaf(gr[j], Bv, s1);
            const float gp = gr[j] * e[t][j];
            const float r = gp * (t > 0 ? H[t > 0 ? t - 1 : 0][j] : hck[j]);
            s2 = fmaf(Av[j], r, s2);
            dA[j] = fmaf(dw.x, r, dA[j]);
            gr[j] = gp;
          }
          sm.s[g][t][lane] = make_float2(s1, s2);
        }
        if (pend_t >= 0) take_sums();
        red_put(sm.red[g], pv, lane);
        pend_t = kb * KB + ru * RS;
      }
    }
    take_sums();
    __syncthreads();

    // the tile's dB, dC sums are one contiguous block of the workspace:
    // stored as 8-byte pieces from LDS (scattered 4-byte stores from the
    // reduction lanes kept the CU's store queue full)
    {
      float2* dst = reinterpret_cast<float2*>(ws_dbc + ((int64_t)k.gi * Lp + tb) * (2 * N));
      const float2* src = reinterpret_cast<const float2*>(&sm.dbc[0][0]);
      for (int idx = threadIdx.x; idx < T * N; idx += kLanes * NG) dst[idx] = src[idx];
    }

    // output phase: this wave's chunk of the tile
    {
      const int64_t tc = tb + g * KC;
      const int64_t nv = s.L - tc;
      float odu[KC], odd[KC], odz[KC];
#pragma unroll
      for (int q = 0; q < KC; ++q) {
        const int t = g * KC + q;
        float y = 0.0f, s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int w = 0; w < NG; ++w) {
          if constexpr (HAS_Z) y += sm.y[w][t][lane];
          const float2 sv = sm.s[w][t][lane];
          s1 += sv.x;
          s2 += sv.y;
        }
        odu[q] = fmaf(cD[q], s1, Dd * cDy[q]);
        const float ddl = fmaf(cU[q], s1, s2) * cS[q];
        odd[q] = ddl;
        if constexpr (HAS_Z) odz[q] = fmaf(Dd, cU[q], y) * cDz[q];
        dDacc = fmaf(cDy[q], cU[q], dDacc);
        dbacc += q < nv ? ddl : 0.0f;
      }
      if constexpr (kStageOut) {
        // The tile's du, ddelta, dz leave through LDS, and the next tile's
        // inputs arrive through it (the reduction blocks are free: the tile's
        // sums were taken before the barrier above).  Each wave stages its 4
        // steps of every channel; after a barrier wave g stores (and has
        // loaded) channels 16 g .. 16 g + 15 over the tile's 16 steps, so a
        // memory instruction moves 16 rows of 32 contiguous bytes rather than
        // 8 bytes of each of 64 rows.
        auto put = [&](int tt, const float (&o)[KC]) {
          *stg_at(tt, lane, g) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        };
        put(0, odu);
        put(1, odd);
        if constexpr (HAS_Z) put(2, odz);
        if (more) {
          *stg_at(3, c_st, q_st) = make_uint2(nu.w[0], nu.w[1]);
          *stg_at(4, c_st, q_st) = make_uint2(nd.w[0], nd.w[1]);
          if constexpr (HAS_Z) *stg_at(5, c_st, q_st) = make_uint2(nz.w[0], nz.w[1]);
          *stg_at(6, c_st, q_st) = make_uint2(no.w[0], no.w[1]);
        }
        __syncthreads();
        if (more) {
          uint2 v = *stg_at(3, lane, g);
          nu.w[0] = v.x; nu.w[1] = v.y;
          v = *stg_at(4, lane, g);
          nd.w[0] = v.x; nd.w[1] = v.y;
          if constexpr (HAS_Z) {
            v = *stg_at(5, lane, g);
            nz.w[0] = v.x; nz.w[1] = v.y;
          }
          v = *stg_at(6, lane, g);
          no.w[0] = v.x; no.w[1] = v.y;
          prep_r(tb - T);
          finish_checkpoint(hraw, hck);
        }
        const int64_t t_o = tb + 4 * q_st;
        if (d_st < s.dim && t_o < s.L) {
          const int64_t off = row_st * s.L + t_o;
          auto st = [&](void* base, int tt) {
            *reinterpret_cast<uint2*>(static_cast<char*>(base) + off * 2) = *stg_at(tt, c_st, q_st);
          };
          st(du, 0);
          st(ddelta, 1);
          if constexpr (HAS_Z) st(dz, 2);
        }
      } else {
        // the prefetched inputs and checkpoint are consumed before the
        // stores: the counter a load's wait reads also counts stores issued
        // after it
        if (more) {
          prep_r(tb - T);
          finish_checkpoint(hraw, hck);
        }
        if (k.valid) {
        const int64_t off = k.rowoff + tc * s.ts;
        store_chunk<BF16, VEC, KC>(du, off, odu, nv, s.ts);
        store_chunk<BF16, VEC, KC>(ddelta, off, odd, nv, s.ts);
        if constexpr (HAS_Z) store_chunk<BF16, VEC, KC>(dz, off, odz, nv, s.ts);
        }
      }
    }
    asm volatile("" ::"s"(touch));  // keeps the warming loads
    __syncthreads();
  }

  const int64_t part = (int64_t)k.seg * s.batch * s.dim + k.row;
  if (k.valid) {
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
      if (dh0 && k.seg == 0) dh0[k.row * N + n0 + j] = gr[j];
      ws_dA[part * N + n0 + j] = dA[j];
    }
  }
  // dD and dbias: sum the waves' chunks (the loop ended on a barrier)
  sm.y[g][0][lane] = dDacc;
  sm.y[g][1][lane] = dbacc;
  __syncthreads();
  if (g == 0 && k.valid) {
    float sD = 0.0f, sb = 0.0f;
#pragma unroll
    for (int w = 0; w < NG; ++w) {
      sD += sm.y[w][0][lane];
      sb += sm.y[w][1][lane];
    }
    ws_dDb[part * 2 + 0] = sD;
    ws_dDb[part * 2 + 1] = sb;
  }
}

// ---------------------------------------------------------------- reduce ---
// Sum of count values stride apart, added in index order; the loads of 8
// terms are issued before they are added, so a thread waits once per 8.
template <typename Idx>
__device__ __forceinline__ float strided_sum(const float* __restrict__ p, Idx stride,
                                             int count) {
  float acc = 0.0f;
  int k = 0;
  for (; k + 8 <= count; k += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = p[(Idx)(k + j) * stride];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += v[j];
  }
  for (; k < count; ++k) acc += p[(Idx)k * stride];
  return acc;
}

// dB, dC: sum of the channel groups' sums; dA, dD, dbias: sum over segments
// and the batch (partial k = segment * batch + b sits k * dim rows in).
// Every output element is one thread adding its terms in a fixed order.
template <int N, typename Idx>
__global__ void __launch_bounds__(256)
    bwd_reduce_kernel(const float* __restrict__ ws_dbc,
                      const float* __restrict__ ws_dA,
                      const float* __restrict__ ws_dDb, float* __restrict__ dB,
                      float* __restrict__ dC, float* __restrict__ dA,
                      float* __restrict__ dD, float* __restrict__ dbias,
                      Idx batch, Idx dim, Idx L, Idx Lp, int gpb, int segments,
                      int groups, int state_major) {
  Idx i = (Idx)blockIdx.x * blockDim.x + threadIdx.x;
  const Idx n_bc = batch * L * (Idx)groups * 2 * N;
  if (i < n_bc) {
    // i -> (b, t, group, q, n) with n fastest; the group's channel groups
    // are gpb / groups consecutive ones
    const Idx n = i % N;
    Idx r = i / N;
    const Idx q = r % 2;
    r /= 2;
    const Idx grp = r % (Idx)groups;
    r /= (Idx)groups;
    const Idx t = r % L;
    const Idx b = r / L;
    const int per = gpb / groups;
    const float* src =
        ws_dbc + ((b * (Idx)gpb + grp * (Idx)per) * Lp + t) * (2 * N) + q * N + n;
    const float acc = strided_sum<Idx>(src, Lp * 2 * N, per);
    (q ? dC : dB)[state_major ? ((b * (Idx)groups + grp) * N + n) * L + t
                              : ((b * L + t) * (Idx)groups + grp) * N + n] = acc;
    return;
  }
  i -= n_bc;
  const int parts = segments * (int)batch;
  if (i < dim * N) {
    dA[i] = strided_sum<Idx>(ws_dA + i, dim * N, parts);
    return;
  }
  i -= dim * N;
  if (i < dim) {
    const float aD = strided_sum<Idx>(ws_dDb + i * 2 + 0, dim * 2, parts);
    const float ab = strided_sum<Idx>(ws_dDb + i * 2 + 1, dim * 2, parts);
    if (dD) dD[i] = aD;
    if (dbias) dbias[i] = ab;
  }
}

template <int N, bool BF16, bool VEC, bool HAS_Z>
hipError_t launch_passes(const BwdParams& p, const BwdShape& s, hipStream_t st) {
  constexpr int NG = kBwdWaves<N>;
  const int64_t G = p.batch * p.groups_per_batch;
  const dim3 grid((unsigned)(G * p.segments)), block(kLanes * NG);
  const uint32_t* bcp = (const uint32_t*)p.ws_bc;
  hipError_t e;
  if (p.ev_start) {
    e = hipEventRecord((hipEvent_t)p.ev_start, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((bwd_pass_f_kernel<N, NG, BF16, VEC, HAS_Z>), grid, block, 0,
                     st, p.u, p.delta, p.z, p.dout, p.A, p.bias, p.ws_ck,
                     p.ws_cd, p.ws_S, p.ws_R, p.ws_sum, bcp, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = G * N * kLanes;
  hipLaunchKernelGGL(bwd_combine_kernel, dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, st, p.A, p.h0, p.dlast, p.ws_S, p.ws_R,
                     p.ws_sum, p.ws_hin, p.ws_gin, s, N, G);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_pass_r_kernel<N, NG, BF16, VEC, HAS_Z>), grid, block, 0,
                     st, p.u, p.delta, p.z, p.dout, p.A, p.D, p.bias, p.du,
                     p.ddelta, p.dz, p.dh0, p.ws_ck, p.ws_cd, p.ws_hin, p.ws_gin,
                     p.ws_dbc, p.ws_dA, p.ws_dDb, bcp, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.ev_stop) e = hipEventRecord((hipEvent_t)p.ev_stop, st);
  return e;
}

template <int N, bool BF16, bool VEC>
hipError_t launch_n(const BwdParams& p, hipStream_t st) {
  constexpr int NG = kBwdWaves<N>;
  constexpr int WPS = BCLayout<N / NG, BF16>::kWordsPerStep;
  const int64_t Lp = (int64_t)p.tiles * kT;
  BwdShape s;
  s.dim = p.dim;
  s.L = p.L;
  s.ts = p.layout_bld ? p.dim : 1;
  s.ngroups = p.ngroups > 1 ? p.ngroups : 1;
  s.reserved = 0;
  s.groups_per_batch = p.groups_per_batch;
  s.tiles = p.tiles;
  s.segments = p.segments;
  s.seg_tiles = p.seg_tiles;
  s.softplus = p.softplus;
  s.batch = (int32_t)p.batch;
  hipError_t e = launch_bc_pack(p.B, p.C, p.ws_bc, p.batch, s.ngroups, p.L, Lp, N,
                                NG, BF16, BF16, Lp * WPS, nullptr, 0,
                                p.bc_state_major != 0, st);
  if (e != hipSuccess) return e;
  e = p.z ? launch_passes<N, BF16, VEC, true>(p, s, st)
          : launch_passes<N, BF16, VEC, false>(p, s, st);
  if (e != hipSuccess) return e;
  const int64_t threads = p.batch * p.L * s.ngroups * 2 * N + p.dim * N + p.dim;
  const dim3 grid((unsigned)((threads + 255) / 256));
  // 32-bit indices when the largest workspace index and the thread count
  // stay below 2^31
  const int64_t G = p.batch * p.groups_per_batch;
  const int64_t top = std::max({G * Lp * 2 * N, (int64_t)p.segments * p.batch * p.dim * N,
                                (int64_t)p.segments * p.batch * p.dim * 2, threads + 256});
  if (top < (int64_t(1) << 31))
    hipLaunchKernelGGL((bwd_reduce_kernel<N, uint32_t>), grid, dim3(256), 0, st,
                       p.ws_dbc, p.ws_dA, p.ws_dDb, p.dB, p.dC, p.dA, p.dD, p.dbias,
                       (uint32_t)p.batch, (uint32_t)p.dim, (uint32_t)p.L, (uint32_t)Lp,
                       p.groups_per_batch, p.segments, s.ngroups, p.bc_state_major);
  else
    hipLaunchKernelGGL((bwd_reduce_kernel<N, int64_t>), grid, dim3(256), 0, st,
                       p.ws_dbc, p.ws_dA, p.ws_dDb, p.dB, p.dC, p.dA, p.dD, p.dbias,
                       p.batch, p.dim, p.L, Lp, p.groups_per_batch, p.segments,
                       s.ngroups, p.bc_state_major);
  return hipGetLastError();
}

template <int N>
hipError_t launch_dtype(const BwdParams& p, bool bf16, bool vec, hipStream_t st) {
  if (bf16) return vec ? launch_n<N, true, true>(p, st) : launch_n<N, true, false>(p, st);
  return vec ? launch_n<N, false, true>(p, st) : launch_n<N, false, false>(p, st);
}

int64_t up256(int64_t x) { return (x + 255) / 256 * 256; }

}  // namespace

int bwd_tile() { return kT; }

int bwd_waves_per_group(int N) { return N >= 4 ? N / 4 : 1; }

namespace {
template <int N>
hipError_t pass_r_occupancy(bool bf16, int* blocks) {
  constexpr int NG = kBwdWaves<N>;
  const void* f = bf16 ? reinterpret_cast<const void*>(
                             &bwd_pass_r_kernel<N, NG, true, true, true>)
                       : reinterpret_cast<const void*>(
                             &bwd_pass_r_kernel<N, NG, false, true, true>);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, f, kLanes * NG, 0);
}
}  // namespace

int bwd_wgs_per_cu(int N, bool bf16) {
  static std::atomic<int> cache[2][6];
  int idx = 0;
  while (idx < 5 && (1 << idx) < N) ++idx;
  std::atomic<int>& slot = cache[bf16 ? 1 : 0][idx];
  int v = slot.load(std::memory_order_relaxed);
  if (v > 0) return v;
  int blocks = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (N) {
    case 1: e = pass_r_occupancy<1>(bf16, &blocks); break;
    case 2: e = pass_r_occupancy<2>(bf16, &blocks); break;
    case 4: e = pass_r_occupancy<4>(bf16, &blocks); break;
    case 8: e = pass_r_occupancy<8>(bf16, &blocks); break;
    case 16: e = pass_r_occupancy<16>(bf16, &blocks); break;
    case 32: e = pass_r_occupancy<32>(bf16, &blocks); break;
    default: break;
  }
  v = (e == hipSuccess && blocks > 0) ? blocks : 2;
  slot.store(v, std::memory_order_relaxed);
  return v;
}

int bwd_segments(int64_t groups, int64_t tiles, int cus, int wgs_per_cu, int forced) {
  int64_t P = 1;
  if (forced > 0) {
    P = forced;
  } else {
    // Pass R holds wgs_per_cu workgroups per CU.  Take the fewest segments
    // that give at least two rounds of tasks, all of them full (a last round
    // short by even a tenth cost 6% at 320 groups x 2048 steps); else the
    // fullest last round.
    const int64_t slots = (int64_t)std::max(wgs_per_cu, 1) * std::max(cus, 1);
    const int64_t pmax = std::max<int64_t>(1, tiles / kMinSegTiles);
    double best = -1.0;
    for (int64_t q = 1; q <= pmax; ++q) {
      const int64_t seg_tiles = (tiles + q - 1) / q;
      const int64_t pq = (tiles + seg_tiles - 1) / seg_tiles;
      const int64_t tasks = groups * pq;
      const int64_t rounds = (tasks + slots - 1) / slots;
      const double fill = (double)tasks / (double)(rounds * slots);
      if (tasks >= 2 * slots && fill >= 0.99) {
        P = pq;
        break;
      }
      if (fill > best + 1e-9) {
        best = fill;
        P = pq;
      }
    }
  }
  P = std::max<int64_t>(1, std::min<int64_t>(P, tiles));
  // whole tiles per segment; the count follows from the segment length
  const int64_t seg_tiles = (tiles + P - 1) / P;
  return (int)((tiles + seg_tiles - 1) / seg_tiles);
}

int64_t bwd_workspace(int64_t batch, int64_t dim, int64_t L, int N, bool bf16,
                      int segments, int64_t groups, void* ws, BwdParams* p) {
  const int NG = bwd_waves_per_group(N);
  const int npw = N / NG;
  const int wps = bf16 ? npw : 2 * npw;
  const int64_t tiles = (L + kT - 1) / kT;
  const int64_t Lp = tiles * kT;
  const int64_t gpb = (dim + kLanes - 1) / kLanes;
  const int64_t G = batch * gpb;
  const int64_t tasks = G * segments;
  const int64_t sizes[12] = {
      batch * groups * NG * Lp * wps * 4,  // packed B/C runs
      G * tiles * N * kLanes * 4,       // tile checkpoints
      G * tiles * kLanes * 4,           // running sums of Delta at tiles
      tasks * N * kLanes * 4,           // segment end states
      tasks * N * kLanes * 4,           // segment reverse aggregates
      tasks * kLanes * 8,               // segment sums of Delta
      tasks * N * kLanes * 4,           // segment initial states
      tasks * N * kLanes * 4,           // segment incoming gradients
      G * Lp * 2 * N * 4,               // channel-group dB/dC sums
      segments * batch * dim * N * 4,   // partial dA
      segments * batch * dim * 2 * 4,   // partial dD, dbias
      0};
  int64_t off[12], total = 0;
  for (int i = 0; i < 12; ++i) {
    off[i] = total;
    total += up256(sizes[i]);
  }
  if (p && ws) {
    char* base = static_cast<char*>(ws);
    p->ws_bc = base + off[0];
    p->ws_ck = reinterpret_cast<float*>(base + off[1]);
    p->ws_cd = reinterpret_cast<float*>(base + off[2]);
    p->ws_S = reinterpret_cast<float*>(base + off[3]);
    p->ws_R = reinterpret_cast<float*>(base + off[4]);
    p->ws_sum = reinterpret_cast<double*>(base + off[5]);
    p->ws_hin = reinterpret_cast<float*>(base + off[6]);
    p->ws_gin = reinterpret_cast<float*>(base + off[7]);
    p->ws_dbc = reinterpret_cast<float*>(base + off[8]);
    p->ws_dA = reinterpret_cast<float*>(base + off[9]);
    p->ws_dDb = reinterpret_cast<float*>(base + off[10]);
  }
  return total;
}

hipError_t launch_scan_bwd(const BwdParams& p, int N, bool bf16, bool vec,
                           hipStream_t st) {
  switch (N) {
    case 1: return launch_dtype<1>(p, bf16, vec, st);
    case 2: return launch_dtype<2>(p, bf16, vec, st);
    case 4: return launch_dtype<4>(p, bf16, vec, st);
    case 8: return launch_dtype<8>(p, bf16, vec, st);
    case 16: return launch_dtype<16>(p, bf16, vec, st);
    case 32: return launch_dtype<32>(p, bf16, vec, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mssm
