// mamba2.hip -- the Mamba-2 block's scan for gfx950, in the chunked matrix
// form on the matrix cores (MFMA).
//
// The recurrence is the selective scan's with one A, one step and one D per
// head of P channels, B and C shared by a group of heads (page "Mamba:
// Selective State Space Models", "Use the Mamba2 block", names the block and
// its state sizes of 64 or 128; the per-head structure is the Mamba-2
// architecture's).  For channel p of head h, group g(h), state n:
//   Delta_t = softplus(dt_t + bias_h),   a_t = Delta_t A_h
//   H_t[p,n] = exp(a_t) H_{t-1}[p,n] + Delta_t x_t[p] B_t[n]
//   y_t[p]   = sum_n C_t[n] H_t[p,n] + D_h x_t[p],   out = y silu(z)
// Because the decay exp(a_t) is one number per head and step, a chunk of Q
// steps starting from state H0 unrolls into dense products (cum_t the
// inclusive sum of a over the chunk):
//   Y      = diag(exp(cum)) C H0^T  +  (L o C B^T) X,
//            L[t,s] = exp(cum_t - cum_s) Delta_s for s <= t, else 0
//   H_end  = exp(cum_end) H0  +  (X o w)^T B,  w_s = Delta_s exp(cum_end - cum_s)
// One workgroup owns one (batch, head) and walks its chunks in order with
// H in registers, so no state goes to memory between chunks.  C B^T,
// (L o C B^T) X, C H0^T and (X o w)^T B are 32x32x16 bf16 MFMAs with fp32
// accumulation.  B, C and x are bf16 inputs and enter exactly; an fp32
// operand (L o C B^T, X o w, H0) enters as hi + lo bf16 halves (hi = RNE(v),
// lo = RNE(v - hi)), which keeps 16 mantissa bits, and costs a second MFMA.
// The cumulative sums are kept in fp64, so the decay between two steps
// carries the rounding of that difference only.
#include "dev_math.h"
#include "mssm_internal.h"

namespace mssm {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kQ = 64;         // timesteps per chunk
constexpr int kP = 64;         // channels per head
constexpr int kThreads = 256;  // 4 waves
constexpr int kQP = kQ + 8;    // row pitch (bf16) of [*][kQ] tiles: 16 bytes of
                               // padding keep 16-byte operand reads conflict-free

// 32x32x16 bf16 MFMA lane layout:
//   A operand (32 rows x 16 k): lane l holds A[l % 32][8 (l / 32) + j], j < 8
//   B operand (16 k x 32 cols): lane l holds B[8 (l / 32) + j][l % 32]
//   result register v of lane l: D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32]
__device__ __forceinline__ int acc_row(int v, int lane) {
  return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}
__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) {  // 16-byte aligned
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void split(float v, uint16_t& hi, uint16_t& lo) {
  hi = to_bf16(v);
  lo = to_bf16(v - bf16_bits(hi));
}

template <int N>
struct alignas(16) Smem {
  static constexpr int NP = N + 8;
  uint16_t B[kQ][NP];        // B_t[n] of the chunk, [t][n]
  uint16_t Bt[N][kQP];       // the same, [n][t]
  uint16_t C[kQ][NP];        // C_t[n], [t][n]
  uint16_t Xt[kP][kQP];      // x_t[p], [p][t]
  uint16_t Xw[2][kP][kQP];   // x_t[p] w_t, hi / lo, [p][t]
  uint16_t M[2][kQ][kQP];    // (L o C B^T)[t][s], hi / lo
  uint16_t H[2][kP][NP];     // state entering the chunk, hi / lo, [p][n]
  double cum[kQ];            // inclusive sum of a over the chunk
  float delta[kQ], ecum[kQ], w[kQ];
  float dec_end;             // exp(cum_end)
};

struct M2Shape {
  int64_t L;
  int32_t H, G;  // heads, B/C groups
  int32_t softplus, load_state;
};

// Grid: one workgroup per (batch entry, head), block = b * H + h.
template <int N, bool HAS_Z>
__global__ void __launch_bounds__(kThreads)
    mamba2_scan_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ dt,
                       const float* __restrict__ A, const uint16_t* __restrict__ Bm,
                       const uint16_t* __restrict__ Cm, const float* __restrict__ Dv,
                       const uint16_t* __restrict__ z, const float* __restrict__ bias,
                       uint16_t* __restrict__ out, float* __restrict__ state,
                       const M2Shape s) {
  constexpr int NT = N / 64;  // 32 x 32 state tiles per wave
  __shared__ Smem<N> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int col = lane & 31;
  const int kq = 8 * (lane >> 5);     // this lane's k offset in an operand
  const int tb = wv >> 1;             // row block of the C B^T and Y tiles (t)
  const int pb = wv & 1;              // p block of the Y and state tiles; s block of C B^T
  const int nbase = (wv >> 1) * (N / 2);
  const int64_t b = blockIdx.x / s.H;
  const int h = (int)(blockIdx.x - b * s.H);
  const int g = h / (s.H / s.G);
  const int64_t L = s.L;
  const float Ah = A[h];
  const float Dh = Dv ? Dv[h] : 0.0f;
  const float bh = bias ? bias[h] : 0.0f;
  const int64_t srow = ((int64_t)b * s.H + h) * kP;  // first state row of the head

  // state tiles: rows p = 32 pb + acc_row, cols n = nbase + 32 i + col
  f32x16 hacc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      hacc[i][v] = s.load_state
                       ? state[(srow + 32 * pb + acc_row(v, lane)) * N + nbase + 32 * i + col]
                       : 0.0f;
  auto state_to_lds = [&]() {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int p = 32 * pb + acc_row(v, lane), n = nbase + 32 * i + col;
        split(hacc[i][v], sm.H[0][p][n], sm.H[1][p][n]);
      }
  };
  state_to_lds();

  const int64_t chunks = (L + kQ - 1) / kQ;
  for (int64_t c = 0; c < chunks; ++c) {
    const int64_t t0 = c * kQ;
    // ---- phase 1: the chunk's inputs into LDS
    if (wv == 0) {
      const int64_t t = t0 + lane;
      float dl = 0.0f;
      if (t < L) {
        const float v = bf16_bits(dt[(b * L + t) * s.H + h]) + bh;
        dl = s.softplus ? softplus_f32(v) : v;
      }
      double cs = (double)(dl * Ah);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(cs, off);
        if (lane >= off) cs += o;
      }
      const double end = __shfl(cs, 63);
      sm.cum[lane] = cs;
      sm.delta[lane] = dl;
      sm.ecum[lane] = hw_exp2((float)cs * kLog2e);
      sm.w[lane] = dl * hw_exp2((float)(end - cs) * kLog2e);
      if (lane == 0) sm.dec_end = hw_exp2((float)end * kLog2e);
    }
    {
      constexpr int kPer = N / 8;  // 16-byte pieces per row
      for (int i = tid; i < kQ * kPer; i += kThreads) {
        const int t = i / kPer, n8 = (i % kPer) * 8;
        uint4 vb = make_uint4(0u, 0u, 0u, 0u), vc = vb;
        if (t0 + t < L) {
          const int64_t off = ((b * L + t0 + t) * s.G + g) * N + n8;
          vb = *reinterpret_cast<const uint4*>(Bm + off);
          vc = *reinterpret_cast<const uint4*>(Cm + off);
        }
        *reinterpret_cast<uint4*>(&sm.B[t][n8]) = vb;
        *reinterpret_cast<uint4*>(&sm.C[t][n8]) = vc;
        const uint32_t q[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sm.Bt[n8 + 2 * j][t] = (uint16_t)(q[j] & 0xffffu);
          sm.Bt[n8 + 2 * j + 1][t] = (uint16_t)(q[j] >> 16);
        }
      }
    }
    constexpr int kXPer = kQ * kP / 8 / kThreads;  // 16-byte pieces of x per thread
    uint4 xr[kXPer];
#pragma unroll
    for (int k = 0; k < kXPer; ++k) {
      const int i = tid + k * kThreads;
      const int t = i / (kP / 8), p8 = (i % (kP / 8)) * 8;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (t0 + t < L) v = *reinterpret_cast<const uint4*>(x + ((b * L + t0 + t) * s.H + h) * kP + p8);
      xr[k] = v;
      const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sm.Xt[p8 + 2 * j][t] = (uint16_t)(q[j] & 0xffffu);
        sm.Xt[p8 + 2 * j + 1][t] = (uint16_t)(q[j] >> 16);
      }
    }
    float zr[16];
    if constexpr (HAS_Z) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t t = t0 + 32 * tb + acc_row(v, lane);
        zr[v] = t < L ? bf16_bits(z[((b * L + t) * s.H + h) * kP + 32 * pb + col]) : 0.0f;
      }
    }
    __syncthreads();

    // ---- phase 2: x o w, L o C B^T, and the entering state's part of Y
#pragma unroll
    for (int k = 0; k < kXPer; ++k) {
      const int i = tid + k * kThreads;
      const int t = i / (kP / 8), p8 = (i % (kP / 8)) * 8;
      const float wt = sm.w[t];
      const uint32_t q[4] = {xr[k].x, xr[k].y, xr[k].z, xr[k].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        split(bf16_lo(q[j]) * wt, sm.Xw[0][p8 + 2 * j][t], sm.Xw[1][p8 + 2 * j][t]);
        split(bf16_hi(q[j]) * wt, sm.Xw[0][p8 + 2 * j + 1][t], sm.Xw[1][p8 + 2 * j + 1][t]);
      }
    }
    if (pb <= tb) {  // the block above the diagonal is all zero
      f32x16 gacc = {};
#pragma unroll
      for (int k0 = 0; k0 < N; k0 += 16)
        gacc = mfma(lds8(&sm.C[32 * tb + col][k0 + kq]), lds8(&sm.B[32 * pb + col][k0 + kq]),
                    gacc);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = 32 * tb + acc_row(v, lane), sc = 32 * pb + col;
        float m = 0.0f;
        if (sc <= t)
          m = gacc[v] * hw_exp2((float)(sm.cum[t] - sm.cum[sc]) * kLog2e) * sm.delta[sc];
        split(m, sm.M[0][t][sc], sm.M[1][t][sc]);
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = 32 * tb + acc_row(v, lane), sc = 32 * pb + col;
        sm.M[0][t][sc] = sm.M[1][t][sc] = 0;
      }
    }
    f32x16 yacc = {};
#pragma unroll
    for (int k0 = 0; k0 < N; k0 += 16) {
      const bf16x8 a = lds8(&sm.C[32 * tb + col][k0 + kq]);
      yacc = mfma(a, lds8(&sm.H[0][32 * pb + col][k0 + kq]), yacc);
      yacc = mfma(a, lds8(&sm.H[1][32 * pb + col][k0 + kq]), yacc);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) yacc[v] *= sm.ecum[32 * tb + acc_row(v, lane)];
    __syncthreads();

    // ---- phase 3: (L o C B^T) X, the output, and the state at the chunk end
#pragma unroll
    for (int k0 = 0; k0 < kQ; k0 += 16) {
      const bf16x8 bx = lds8(&sm.Xt[32 * pb + col][k0 + kq]);
      yacc = mfma(lds8(&sm.M[0][32 * tb + col][k0 + kq]), bx, yacc);
      yacc = mfma(lds8(&sm.M[1][32 * tb + col][k0 + kq]), bx, yacc);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int t = 32 * tb + acc_row(v, lane), p = 32 * pb + col;
      if (t0 + t < L) {
        float y = fmaf(Dh, bf16_bits(sm.Xt[p][t]), yacc[v]);
        if constexpr (HAS_Z) y *= silu_f32(zr[v]);
        out[((b * L + t0 + t) * s.H + h) * kP + p] = to_bf16(y);
      }
    }
    const float dec = sm.dec_end;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) hacc[i][v] *= dec;
#pragma unroll
      for (int k0 = 0; k0 < kQ; k0 += 16) {
        const bf16x8 bb = lds8(&sm.Bt[nbase + 32 * i + col][k0 + kq]);
        hacc[i] = mfma(lds8(&sm.Xw[0][32 * pb + col][k0 + kq]), bb, hacc[i]);
        hacc[i] = mfma(lds8(&sm.Xw[1][32 * pb + col][k0 + kq]), bb, hacc[i]);
      }
    }
    __syncthreads();
    state_to_lds();  // read by the next chunk after its first barrier
  }

  if (state) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        state[(srow + 32 * pb + acc_row(v, lane)) * N + nbase + 32 * i + col] = hacc[i][v];
  }
}

template <int N>
hipError_t launch_n(const Mamba2Params& p, hipStream_t st) {
  const M2Shape s{p.L, (int32_t)p.nheads, (int32_t)p.ngroups, p.softplus, p.load_state};
  const dim3 grid((unsigned)(p.batch * p.nheads)), block(kThreads);
  const auto* x = static_cast<const uint16_t*>(p.x);
  const auto* dt = static_cast<const uint16_t*>(p.dt);
  const auto* B = static_cast<const uint16_t*>(p.B);
  const auto* C = static_cast<const uint16_t*>(p.C);
  const auto* z = static_cast<const uint16_t*>(p.z);
  auto* out = static_cast<uint16_t*>(p.out);
  if (p.z)
    hipLaunchKernelGGL((mamba2_scan_kernel<N, true>), grid, block, 0, st, x, dt, p.A, B, C,
                       p.D, z, p.bias, out, p.state, s);
  else
    hipLaunchKernelGGL((mamba2_scan_kernel<N, false>), grid, block, 0, st, x, dt, p.A, B,
                       C, p.D, z, p.bias, out, p.state, s);
  return hipGetLastError();
}

}  // namespace

int mamba2_headdim() { return kP; }

hipError_t launch_mamba2_scan(const Mamba2Params& p, hipStream_t st) {
  switch (p.N) {
    case 64: return launch_n<64>(p, st);
    case 128: return launch_n<128>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mssm
