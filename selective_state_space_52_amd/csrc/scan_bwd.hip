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
// Mapping (the forward kernel's, extended):
//   * one lane per channel, 64 channels of one batch entry per workgroup;
//     the N states of a channel are split over NG waves (4 states each);
//     B_t and C_t are wave-uniform and read with wide scalar loads from a
//     per-wave packed run (zero-padded to whole tiles);
//   * pass F scans the row forwards and stores the state at the start of
//     every 16-step tile (workspace, lane-contiguous);
//   * pass R walks the tiles backwards.  Per tile each wave recomputes its
//     states' e_t and h_t from the tile's checkpoint into registers, then runs
//     the reverse recurrence; sums over n of a channel (y, g.B, A g e h) go
//     through LDS to the wave that owns the timestep, as in the forward
//     output phase;
//   * dB and dC need sums over the 64 channels of a wave: 16 values per lane
//     are written to a per-wave LDS block and read back transposed, so each
//     lane adds 16 values and two DPP steps finish the sum; the per-group
//     sums go to workspace and a last kernel adds the groups (fixed order,
//     so the result is deterministic), together with the batch sums of dA,
//     dD and dbias.
#include "dev_math.h"
#include "mssm_internal.h"
#include "scan_common.h"

namespace mssm {
namespace {

constexpr int kT = 16;                 // timesteps per tile (and checkpoint)
constexpr int kRedItems = 16;          // values per lane per channel reduction
constexpr int kRedPitch = kLanes + 4;  // padded row: conflict-free b128 reads

// Waves per 64-channel workgroup: four states per wave.
template <int N>
constexpr int kBwdWaves = N >= 4 ? N / 4 : 1;

struct BwdShape {
  int64_t dim, L;
  int32_t groups_per_batch, tiles;
  int32_t softplus, reserved;
};

template <int NG>
struct alignas(16) BwdSmem {
  float2 dw[kT][kLanes];                // (Delta, Delta*u) of the tile
  float dy[kT][kLanes];                 // dout * silu(z)
  float y[NG][kT][kLanes];              // per-wave partial readouts
  float2 s[NG][kT][kLanes];             // per-wave (sum g B, sum A g e h_prev)
  float red[NG][kRedItems][kRedPitch];  // per-wave channel-sum transpose
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

// Sum of v[k] over the 64 lanes of the wave, for k < kRedItems; lanes
// 4k .. 4k+3 return the sum of item k.
__device__ __forceinline__ float wave_sum_items(float (&red)[kRedItems][kRedPitch],
                                                const float (&v)[kRedItems],
                                                int lane) {
#pragma unroll
  for (int k = 0; k < kRedItems; ++k) red[k][lane] = v[k];
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

template <int N, int NG, bool BF16, bool VEC, bool HAS_Z>
__global__ void __launch_bounds__(kLanes* NG)
    scan_bwd_kernel(const void* __restrict__ u, const void* __restrict__ delta,
                    const void* __restrict__ z, const void* __restrict__ dout,
                    const float* __restrict__ A, const float* __restrict__ Dv,
                    const float* __restrict__ bias, const float* __restrict__ h0,
                    const float* __restrict__ dlast, void* __restrict__ du,
                    void* __restrict__ ddelta, void* __restrict__ dz,
                    float* __restrict__ dh0, float* __restrict__ ws_ck,
                    float* __restrict__ ws_dbc, float* __restrict__ ws_dA,
                    float* __restrict__ ws_dDb, const uint32_t* __restrict__ bcp,
                    const BwdShape s) {
  constexpr int NPW = N / NG;
  constexpr int T = kT;
  constexpr int KC = T / NG;  // timesteps a wave prepares and emits per tile
  constexpr int WPS = BCLayout<NPW, BF16>::kWordsPerStep;
  constexpr int KB = BCLayout<NPW, BF16>::kSteps;  // timesteps per B/C batch
  constexpr int NB = T / KB;
  constexpr int RS = kRedItems / (2 * NPW);  // timesteps per channel reduction
  static_assert(T % KB == 0 && KB % RS == 0, "tile, batch and reduction nest");
  using Batch = BCBatch<NPW, BF16>;
  __shared__ BwdSmem<NG> sm;

  const int lane = threadIdx.x & (kLanes - 1);
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = g * NPW;
  const int gi = blockIdx.x;
  const int64_t b = gi / s.groups_per_batch;
  const int64_t d = (int64_t)(gi % s.groups_per_batch) * kLanes + lane;
  const bool valid = d < s.dim;
  const int64_t dc = valid ? d : s.dim - 1;
  const int64_t row = b * s.dim + dc;
  const int64_t rowoff = row * s.L;
  const int64_t Lp = (int64_t)s.tiles * T;
  const uint32_t* __restrict__ bcw = bcp + (b * NG + g) * Lp * WPS;
  float* __restrict__ ck = ws_ck + (int64_t)gi * s.tiles * N * kLanes;
  const bool sp = s.softplus != 0;

  float A2[NPW], Av[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    Av[j] = A[dc * N + n0 + j];
    A2[j] = Av[j] * kLog2e;
  }
  const float bv = bias ? bias[dc] : 0.0f;
  const float Dd = Dv ? Dv[dc] : 0.0f;

  // ---------------- pass F: the state at the start of every tile ----------
  {
    float h[NPW];
#pragma unroll
    for (int j = 0; j < NPW; ++j) h[j] = h0 ? h0[row * N + n0 + j] : 0.0f;
    Raw<BF16, KC> ru, rd;
    auto prep_f = [&](const Raw<BF16, KC>& pu, const Raw<BF16, KC>& pd,
                      int64_t nv) {
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const float x = raw_get(pd, k) + bv;
        float dl = sp ? softplus_f32(x) : x;
        dl = k < nv ? dl : 0.0f;
        sm.dw[g * KC + k][lane] = make_float2(dl, dl * raw_get(pu, k));
      }
    };
    {
      const int64_t tc = g * KC;
      load_chunk<BF16, VEC, KC>(ru, u, rowoff + tc, s.L - tc);
      load_chunk<BF16, VEC, KC>(rd, delta, rowoff + tc, s.L - tc);
      prep_f(ru, rd, s.L - tc);
    }
    __syncthreads();
    for (int ti = 0; ti < s.tiles; ++ti) {
      const int64_t tb = (int64_t)ti * T;
      const int64_t tcn = tb + T + g * KC;
      load_chunk<BF16, VEC, KC>(ru, u, rowoff + tcn, s.L - tcn);
      load_chunk<BF16, VEC, KC>(rd, delta, rowoff + tcn, s.L - tcn);
#pragma unroll
      for (int j = 0; j < NPW; ++j)
        ck[((int64_t)ti * N + n0 + j) * kLanes + lane] = h[j];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        const Batch bc = *reinterpret_cast<const Batch*>(bcw + (tb + kb * KB) * WPS);
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          const float2 dw = sm.dw[kb * KB + i][lane];
#pragma unroll
          for (int j = 0; j < NPW; ++j)
            h[j] = fmaf(hw_exp2(dw.x * A2[j]), h[j],
                        dw.y * bc_val<NPW, BF16>(bc.w, i, j));
        }
      }
      __syncthreads();
      prep_f(ru, rd, s.L - tcn);
      __syncthreads();
    }
  }

  // ---------------- pass R: tiles in reverse ------------------------------
  float gr[NPW], dA[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    gr[j] = (dlast && valid) ? dlast[row * N + n0 + j] : 0.0f;
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
    for (int k = 0; k < KC; ++k) {
      const bool ok = valid && k < nv;
      const float uu = raw_get(nu, k);
      const float x = raw_get(nd, k) + bv;
      float dl = x, sg = 1.0f;
      if (sp) {
        dl = softplus_f32(x);
        sg = hw_rcp(1.0f + hw_exp2(-x * kLog2e));
      }
      const float o = raw_get(no, k);
      float dyv = o, dzf = 0.0f;
      if constexpr (HAS_Z) {
        const float zz = raw_get(nz, k);
        const float sz = hw_rcp(1.0f + hw_exp2(-zz * kLog2e));
        dyv = o * (zz * sz);
        dzf = o * (sz * fmaf(zz, 1.0f - sz, 1.0f));
      }
      if (!ok) {
        dl = 0.0f;
        dyv = 0.0f;
        dzf = 0.0f;
      }
      cD[k] = dl;
      cS[k] = sg;
      cU[k] = uu;
      cDy[k] = dyv;
      cDz[k] = dzf;
      sm.dw[g * KC + k][lane] = make_float2(dl, dl * uu);
      sm.dy[g * KC + k][lane] = dyv;
    }
  };
  auto load_r = [&](int64_t tile_base) {
    const int64_t tc = tile_base + g * KC;
    const int64_t nv = s.L - tc;
    load_chunk<BF16, VEC, KC>(nu, u, rowoff + tc, nv);
    load_chunk<BF16, VEC, KC>(nd, delta, rowoff + tc, nv);
    if constexpr (HAS_Z) load_chunk<BF16, VEC, KC>(nz, z, rowoff + tc, nv);
    load_chunk<BF16, VEC, KC>(no, dout, rowoff + tc, nv);
  };

  const int last = s.tiles - 1;
  load_r((int64_t)last * T);
  prep_r((int64_t)last * T);
  float hck[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) hck[j] = ck[((int64_t)last * N + n0 + j) * kLanes + lane];
  __syncthreads();

  for (int ti = last; ti >= 0; --ti) {
    const int64_t tb = (int64_t)ti * T;
    // prefetch the previous tile's inputs and checkpoint
    float hnx[NPW];
    if (ti > 0) {
      load_r(tb - T);
#pragma unroll
      for (int j = 0; j < NPW; ++j)
        hnx[j] = ck[((int64_t)(ti - 1) * N + n0 + j) * kLanes + lane];
    } else {
#pragma unroll
      for (int j = 0; j < NPW; ++j) hnx[j] = 0.0f;
    }

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

    // reverse recurrence over the tile
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
        const float tot = wave_sum_items(sm.red[g], pv, lane);
        if ((lane & 3) == 0) {
          const int k = lane >> 2;
          const int j = k % NPW;
          const int q = (k / NPW) & 1;
          const int ii = k / (2 * NPW);
          const int64_t t_abs = tb + kb * KB + ru * RS + ii;
          ws_dbc[((int64_t)gi * Lp + t_abs) * (2 * N) + q * N + n0 + j] = tot;
        }
      }
    }
    __syncthreads();

    // output phase: this wave's chunk of the tile
    {
      const int64_t tc = tb + g * KC;
      const int64_t nv = s.L - tc;
      float odu[KC], odd[KC], odz[KC];
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const int t = g * KC + k;
        float y = 0.0f, s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int w = 0; w < NG; ++w) {
          if constexpr (HAS_Z) y += sm.y[w][t][lane];
          const float2 sv = sm.s[w][t][lane];
          s1 += sv.x;
          s2 += sv.y;
        }
        odu[k] = fmaf(cD[k], s1, Dd * cDy[k]);
        const float ddl = fmaf(cU[k], s1, s2) * cS[k];
        odd[k] = ddl;
        if constexpr (HAS_Z) odz[k] = fmaf(Dd, cU[k], y) * cDz[k];
        dDacc = fmaf(cDy[k], cU[k], dDacc);
        dbacc += k < nv ? ddl : 0.0f;
      }
      if (valid) {
        store_chunk<BF16, VEC, KC>(du, rowoff + tc, odu, nv);
        store_chunk<BF16, VEC, KC>(ddelta, rowoff + tc, odd, nv);
        if constexpr (HAS_Z) store_chunk<BF16, VEC, KC>(dz, rowoff + tc, odz, nv);
      }
    }
    if (ti > 0) prep_r(tb - T);
#pragma unroll
    for (int j = 0; j < NPW; ++j) hck[j] = hnx[j];
    __syncthreads();
  }

  if (valid) {
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
      if (dh0) dh0[row * N + n0 + j] = gr[j];
      ws_dA[row * N + n0 + j] = dA[j];
    }
  }
  // dD and dbias: sum the waves' chunks (the loop ended on a barrier)
  sm.y[g][0][lane] = dDacc;
  sm.y[g][1][lane] = dbacc;
  __syncthreads();
  if (g == 0 && valid) {
    float sD = 0.0f, sb = 0.0f;
#pragma unroll
    for (int w = 0; w < NG; ++w) {
      sD += sm.y[w][0][lane];
      sb += sm.y[w][1][lane];
    }
    ws_dDb[row * 2 + 0] = sD;
    ws_dDb[row * 2 + 1] = sb;
  }
}

// dB, dC: sum of the channel groups' sums; dA, dD, dbias: sum over the batch.
// Every output element is one thread adding its terms in a fixed order.
__global__ void __launch_bounds__(256)
    bwd_reduce_kernel(const float* __restrict__ ws_dbc,
                      const float* __restrict__ ws_dA,
                      const float* __restrict__ ws_dDb, float* __restrict__ dB,
                      float* __restrict__ dC, float* __restrict__ dA,
                      float* __restrict__ dD, float* __restrict__ dbias,
                      int64_t batch, int64_t dim, int64_t L, int64_t Lp, int N,
                      int gpb) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n_bc = batch * L * 2 * N;
  if (i < n_bc) {
    const int n = (int)(i % N);
    int64_t r = i / N;
    const int q = (int)(r % 2);
    r /= 2;
    const int64_t t = r % L;
    const int64_t b = r / L;
    const float* src = ws_dbc + ((b * gpb) * Lp + t) * (2 * N) + q * N + n;
    const int64_t stride = Lp * 2 * N;
    float acc = 0.0f;
    for (int k = 0; k < gpb; ++k) acc += src[k * stride];
    (q ? dC : dB)[(b * L + t) * N + n] = acc;
    return;
  }
  i -= n_bc;
  if (i < dim * N) {
    float acc = 0.0f;
    for (int64_t b = 0; b < batch; ++b) acc += ws_dA[b * dim * N + i];
    dA[i] = acc;
    return;
  }
  i -= dim * N;
  if (i < dim) {
    float aD = 0.0f, ab = 0.0f;
    for (int64_t b = 0; b < batch; ++b) {
      aD += ws_dDb[(b * dim + i) * 2 + 0];
      ab += ws_dDb[(b * dim + i) * 2 + 1];
    }
    if (dD) dD[i] = aD;
    if (dbias) dbias[i] = ab;
  }
}

template <int N, bool BF16, bool VEC, bool HAS_Z>
hipError_t launch_main(const BwdParams& p, const BwdShape& s, hipStream_t st) {
  constexpr int NG = kBwdWaves<N>;
  const dim3 grid((unsigned)(p.batch * p.groups_per_batch)), block(kLanes * NG);
  hipLaunchKernelGGL((scan_bwd_kernel<N, NG, BF16, VEC, HAS_Z>), grid, block, 0,
                     st, p.u, p.delta, p.z, p.dout, p.A, p.D, p.bias, p.h0,
                     p.dlast, p.du, p.ddelta, p.dz, p.dh0, p.ws_ck, p.ws_dbc,
                     p.ws_dA, p.ws_dDb, (const uint32_t*)p.ws_bc, s);
  return hipGetLastError();
}

template <int N, bool BF16, bool VEC>
hipError_t launch_n(const BwdParams& p, hipStream_t st) {
  constexpr int NG = kBwdWaves<N>;
  constexpr int WPS = BCLayout<N / NG, BF16>::kWordsPerStep;
  const int64_t Lp = (int64_t)p.tiles * kT;
  BwdShape s;
  s.dim = p.dim;
  s.L = p.L;
  s.groups_per_batch = p.groups_per_batch;
  s.tiles = p.tiles;
  s.softplus = p.softplus;
  s.reserved = 0;
  hipError_t e = launch_bc_pack(p.B, p.C, p.ws_bc, p.batch, p.L, Lp, N, NG,
                                BF16, Lp * WPS, st);
  if (e != hipSuccess) return e;
  if (p.ev_start) {
    e = hipEventRecord((hipEvent_t)p.ev_start, st);
    if (e != hipSuccess) return e;
  }
  e = p.z ? launch_main<N, BF16, VEC, true>(p, s, st)
          : launch_main<N, BF16, VEC, false>(p, s, st);
  if (e != hipSuccess) return e;
  if (p.ev_stop) {
    e = hipEventRecord((hipEvent_t)p.ev_stop, st);
    if (e != hipSuccess) return e;
  }
  const int64_t threads = p.batch * p.L * 2 * N + p.dim * N + p.dim;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, st, p.ws_dbc, p.ws_dA, p.ws_dDb, p.dB, p.dC,
                     p.dA, p.dD, p.dbias, p.batch, p.dim, p.L, Lp, N,
                     p.groups_per_batch);
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

int64_t bwd_workspace(int64_t batch, int64_t dim, int64_t L, int N, bool bf16,
                      void* ws, BwdParams* p) {
  const int NG = bwd_waves_per_group(N);
  const int npw = N / NG;
  const int wps = bf16 ? npw : 2 * npw;
  const int64_t tiles = (L + kT - 1) / kT;
  const int64_t Lp = tiles * kT;
  const int64_t gpb = (dim + kLanes - 1) / kLanes;
  const int64_t G = batch * gpb;
  const int64_t sizes[5] = {
      batch * NG * Lp * wps * 4,   // packed B/C runs
      G * tiles * N * kLanes * 4,  // tile checkpoints
      G * Lp * 2 * N * 4,          // channel-group dB/dC sums
      batch * dim * N * 4,         // per-batch dA
      batch * dim * 2 * 4};        // per-batch dD, dbias
  int64_t off[5], total = 0;
  for (int i = 0; i < 5; ++i) {
    off[i] = total;
    total += up256(sizes[i]);
  }
  if (p && ws) {
    char* base = static_cast<char*>(ws);
    p->ws_bc = base + off[0];
    p->ws_ck = reinterpret_cast<float*>(base + off[1]);
    p->ws_dbc = reinterpret_cast<float*>(base + off[2]);
    p->ws_dA = reinterpret_cast<float*>(base + off[3]);
    p->ws_dDb = reinterpret_cast<float*>(base + off[4]);
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
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mssm
