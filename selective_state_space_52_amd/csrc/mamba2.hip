// mamba2.hip -- the Mamba-2 block's scan for gfx950, in the chunked matrix
// form on the matrix cores (MFMA).
//
// The recurrence is the selective scan's with one A, one step and one D per
// head of P channels, B and C shared by a group of heads (page "Mamba State
// Space Model", "Use the Mamba2 block", names the block and its state sizes
// of 64 or 128; the per-head structure is the Mamba-2 architecture's).  For channel p of head h, group g(h), state n:
//   Delta_t = softplus(dt_t + bias_h),   a_t = Delta_t A_h
//   H_t[p,n] = exp(a_t) H_{t-1}[p,n] + Delta_t x_t[p] B_t[n]
//   y_t[p]   = sum_n C_t[n] H_t[p,n] + D_h x_t[p],   out = y silu(z)
// Because the decay exp(a_t) is one number per head and step, a chunk of Q
// steps starting from state H0 unrolls into dense products (cum_t the
// inclusive sum of a over the chunk):
//   Y      = diag(exp(cum)) C H0^T  +  (L o C B^T) X,
//            L[t,s] = exp(cum_t - cum_s) Delta_s for s <= t, else 0
//   H_end  = exp(cum_end) H0  +  (X o w)^T B,  w_s = Delta_s exp(cum_end - cum_s)
// One workgroup (8 waves) owns one (batch, head) and walks its chunks in order with
// H in registers (as H^T), so no state goes to memory between chunks.  C B^T,
// (L o C B^T) X, C H0^T and B^T (X o w) are 32x32x16 bf16 MFMAs with fp32
// accumulation.  B, C and x are bf16 inputs and enter exactly; an fp32
// operand (L o C B^T, X o w, H0) enters as hi + lo bf16 halves (hi = RNE(v),
// lo = RNE(v - hi)), which keeps 16 mantissa bits, and costs a second MFMA.
// The cumulative sums are kept in fp64, so the decay between two steps
// carries the rounding of that difference only.
#include <algorithm>

#include "dev_math.h"
#include "mssm_internal.h"

namespace mssm {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kQ = 64;         // timesteps per chunk
constexpr int kP = 64;         // channels per head
constexpr int kThreads = 512;  // 8 waves: 4 for the output, 4 for the state
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
__device__ __forceinline__ void split_hl(float v, uint16_t& hi, uint16_t& lo) {
  hi = to_bf16(v);
  lo = to_bf16(v - bf16_bits(hi));
}

// A double moved across lanes by DPP: lanes the pattern gives no source (or
// rows outside row_mask) read 0.  The chunk's inclusive sum over its 64 steps
// (one per lane) is then four row_shr steps within each row of 16 lanes and
// two row broadcasts across rows, with no trip through LDS.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROWS, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROWS, 0xf, false);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ double lane_f64(double v, int l) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

template <int N>
struct alignas(16) Smem {
  static constexpr int NP = N + 8;
  uint16_t B[kQ][NP];        // B_t[n] of the chunk, [t][n]
  uint16_t Bt[N][kQP];       // the same, [n][t]
  uint16_t C[kQ][NP];        // C_t[n], [t][n]
  uint16_t Xt[kP][kQP];      // x_t[p], [p][t]
  uint16_t Zt[kP][kQP];      // z_t[p], [p][t]
  uint16_t Yo[kQ][kP + 8];   // the chunk's outputs, [t][p], staged for 16-byte stores
  uint16_t Xw[2][kP][kQP];   // x_t[p] w_t, hi / lo, [p][t]
  uint16_t M[2][kQ][kQP];    // (L o C B^T)[t][s], hi / lo
  // the entering state's part of Y, C H^T, one partial per n half of the
  // state, in the MFMA result layout: [n half][t block][p block][v / 4][lane]
  float4 Yp[2][2][2][4][64];
  double cum[kQ];            // inclusive sum of a over the chunk
  float delta[kQ], ecum[kQ], w[kQ];
  float dec_end;             // exp(cum_end)
};

struct M2Shape {
  int64_t L;
  int32_t H, G;  // heads, B/C groups
  int32_t softplus, load_state;
  // Time split: (batch, head) pairs [0, whole) are scanned whole; the others
  // are cut into P segments of seg_chunks chunks.  Pass 0 runs n_agg
  // aggregate tasks (segments 0 .. P-2 of the split pairs, from a zero state,
  // state only) ahead of the whole pairs; pass 1 runs every segment of the
  // split pairs from its entering state.
  int32_t whole, P, seg_chunks, n_agg, pass;
};

struct M2Work {
  float* S;         // aggregate tasks' end states, (split, P - 1, 64, N)
  double* sum;      // aggregate tasks' sums of Delta A, (split, P - 1)
  const float* hin; // segments' entering states, (split, P, 64, N)
};

// Grid: one workgroup per (batch entry, head), block = b * H + h.  Waves
// 0-3 own the output: each a 32 x 32 tile (t block, p block) of Y and the
// matching tile of C B^T.  Waves 4-7 own the state: each the 32 x (N / 2)
// block (p block, n half) of H.  Every wave loads part of each chunk.
template <int N, bool HAS_Z>
__global__ void __launch_bounds__(kThreads)
    mamba2_scan_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ dt,
                       const float* __restrict__ A, const uint16_t* __restrict__ Bm,
                       const uint16_t* __restrict__ Cm, const float* __restrict__ Dv,
                       const uint16_t* __restrict__ z, const float* __restrict__ bias,
                       uint16_t* __restrict__ out, float* __restrict__ state,
                       const M2Shape s, const M2Work ws) {
  constexpr int NT = N / 64;  // 32 x 32 state tiles per state wave
  __shared__ Smem<N> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const bool ywave = wv < 4;          // output wave (else state wave)
  const int col = lane & 31;
  const int kq = 8 * (lane >> 5);     // this lane's k offset in an operand
  const int r4 = wv & 3;
  const int tb = r4 >> 1;             // output waves: t block of Y and C B^T
  const int pb = r4 & 1;              // p block (Y, H); s block of C B^T
  const int nbase = (r4 >> 1) * (N / 2);  // state waves: n half
  // task -> (pair, segment, kind)
  int pair, seg = 0;
  bool agg = false, split = false;
  if (s.pass == 0) {
    if ((int)blockIdx.x < s.n_agg) {
      agg = true;
      pair = s.whole + (int)blockIdx.x / (s.P - 1);
      seg = (int)blockIdx.x % (s.P - 1);
    } else {
      pair = (int)blockIdx.x - s.n_agg;
    }
  } else {
    split = true;
    pair = s.whole + (int)blockIdx.x / s.P;
    seg = (int)blockIdx.x % s.P;
  }
  const int sp = pair - s.whole;  // index among the split pairs
  const int64_t b = pair / s.H;
  const int h = pair - (int)b * s.H;
  const int g = h / (s.H / s.G);
  const int L = (int)s.L;
  const int t_begin = (agg || split) ? seg * s.seg_chunks * kQ : 0;
  const int t_end = (agg || split) ? min(L, t_begin + s.seg_chunks * kQ) : L;
  const bool emit = !agg;  // outputs are written (not by aggregate tasks)
  const int64_t seg_elems = (int64_t)kP * N;
  // this (batch, head)'s rows: step t of x, z, out at t * HP (+ channel), of
  // B, C at t * GN (+ state), of dt at t * H; the host keeps every such
  // offset below 2^31
  const int HP = s.H * kP, GN = s.G * N;
  const uint16_t* __restrict__ xb = x + ((int64_t)b * L * s.H + h) * kP;
  const uint16_t* __restrict__ zb = HAS_Z ? z + ((int64_t)b * L * s.H + h) * kP : nullptr;
  uint16_t* __restrict__ ob = out + ((int64_t)b * L * s.H + h) * kP;
  const uint16_t* __restrict__ Bb = Bm + ((int64_t)b * L * s.G + g) * N;
  const uint16_t* __restrict__ Cb = Cm + ((int64_t)b * L * s.G + g) * N;
  const uint16_t* __restrict__ db = dt + (int64_t)b * L * s.H + h;
  const float Ah = A[h];
  const float Dh = Dv ? Dv[h] : 0.0f;
  const float bh = bias ? bias[h] : 0.0f;
  const int64_t srow = ((int64_t)b * s.H + h) * kP;  // first state row of the head

  // state waves: the state is held transposed, tiles of rows n = nbase +
  // 32 i + acc_row and cols p = 32 pb + col.  The entering state is the
  // caller's (whole pairs), zero (aggregate tasks) or the segment's entering
  // state (split pairs).
  const float* h_in = split ? ws.hin + ((int64_t)sp * s.P + seg) * seg_elems
                            : (s.load_state && !agg ? state + srow * N : nullptr);
  f32x16 hacc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      hacc[i][v] = (!ywave && h_in)
                       ? h_in[(32 * pb + col) * N + nbase + 32 * i + acc_row(v, lane)]
                       : 0.0f;
  // The block of M above the diagonal (t block 0, s block 1) is zero in every
  // chunk, and no other step writes it: it is cleared once here.
  if (ywave && pb > tb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int t = 32 * tb + acc_row(v, lane), sc = 32 * pb + col;
      sm.M[0][t][sc] = sm.M[1][t][sc] = 0;
    }
  }

  // Inputs of a chunk, loaded into registers one chunk ahead.  Lane = step t
  // of the chunk (consecutive lanes write consecutive LDS addresses of the
  // transposed tiles).  The output waves load x and z (16-byte pieces 2 wv
  // and 2 wv + 1 of a row, and dt in wave 0) at the start of phase 2; the
  // state waves load B and C (pieces r, r + 4, ... for state wave r), which
  // every head of a batch shares and mostly finds in L2, at the end of
  // phase 3.  Issued all at one point, the CU's loads queued behind each
  // other for thousands of cycles.
  constexpr int kBPer = N / 8 / 4;   // pieces of a B (or C) row per state wave
  uint4 rb[kBPer], rc[kBPer], rx[2], rz[2];
  uint16_t rdt = 0;
  // steps past the task's end load its last step (clamped address) and are
  // zeroed when written to LDS
  auto load_xz = [&](int t0) {
    const int t = min(t0 + lane, t_end - 1);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      rx[k] = *reinterpret_cast<const uint4*>(xb + t * HP + (2 * wv + k) * 8);
      if constexpr (HAS_Z) rz[k] = *reinterpret_cast<const uint4*>(zb + t * HP + (2 * wv + k) * 8);
    }
    if (wv == 0) rdt = db[t * s.H];
  };
  auto load_bc = [&](int t0) {
    const int t = min(t0 + lane, t_end - 1);
#pragma unroll
    for (int k = 0; k < kBPer; ++k) {
      const int off = t * GN + (r4 + 4 * k) * 8;
      rb[k] = *reinterpret_cast<const uint4*>(Bb + off);
      rc[k] = *reinterpret_cast<const uint4*>(Cb + off);
    }
  };
  auto put_t = [](uint16_t (*dst)[kQP], int r0, int t, uint4 v) {  // dst[r0 + j][t]
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dst[r0 + 2 * j][t] = (uint16_t)(q[j] & 0xffffu);
      dst[r0 + 2 * j + 1][t] = (uint16_t)(q[j] >> 16);
    }
  };

  const int chunks = (t_end - t_begin + kQ - 1) / kQ;
  double seg_sum = 0.0;  // aggregate tasks: sum of Delta A over the segment
  if (ywave)
    load_xz(t_begin);
  else
    load_bc(t_begin);
  for (int c = 0; c < chunks; ++c) {
    const int t0 = t_begin + c * kQ;
    // ---- phase 1: the chunk's inputs into LDS
    if (wv == 0) {
      float dl = 0.0f;
      if (t0 + lane < t_end) {
        const float v = bf16_bits(rdt) + bh;
        dl = s.softplus ? softplus_f32(v) : v;
      }
      double cs = (double)(dl * Ah);
      cs += dpp_f64<0x111, 0xf>(cs);  // row_shr:1
      cs += dpp_f64<0x112, 0xf>(cs);  // row_shr:2
      cs += dpp_f64<0x114, 0xf>(cs);  // row_shr:4
      cs += dpp_f64<0x118, 0xf>(cs);  // row_shr:8
      cs += dpp_f64<0x142, 0xa>(cs);  // row_bcast:15 into rows 1 and 3
      cs += dpp_f64<0x143, 0xc>(cs);  // row_bcast:31 into rows 2 and 3
      const double end = lane_f64(cs, 63);
      sm.cum[lane] = cs;
      sm.delta[lane] = dl;
      sm.ecum[lane] = hw_exp2((float)cs * kLog2e);
      sm.w[lane] = dl * hw_exp2((float)(end - cs) * kLog2e);
      if (lane == 0) sm.dec_end = hw_exp2((float)end * kLog2e);
      seg_sum += end;
    }
    const bool live = t0 + lane < t_end;
    const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
    if (ywave) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        put_t(sm.Xt, (2 * wv + k) * 8, lane, live ? rx[k] : zero4);
        if constexpr (HAS_Z) put_t(sm.Zt, (2 * wv + k) * 8, lane, live ? rz[k] : zero4);
      }
    } else {
#pragma unroll
      for (int k = 0; k < kBPer; ++k) {
        const int n8 = (r4 + 4 * k) * 8;
        const uint4 vb = live ? rb[k] : zero4, vc = live ? rc[k] : zero4;
        *reinterpret_cast<uint4*>(&sm.B[lane][n8]) = vb;
        *reinterpret_cast<uint4*>(&sm.C[lane][n8]) = vc;
        put_t(sm.Bt, n8, lane, vb);
      }
    }
    __syncthreads();
    if (ywave && c + 1 < chunks) load_xz(t0 + kQ);  // lands during phases 2 and 3

    f32x16 ya = {}, yb = {};  // output waves: Y, as hi and lo partial sums
    if (ywave && emit) {
      // ---- phase 2 (output): L o C B^T
      if (pb <= tb) {  // the block above the diagonal is all zero
        f32x16 g0 = {}, g1 = {};
#pragma unroll
        for (int k0 = 0; k0 < N; k0 += 32) {
          g0 = mfma(lds8(&sm.C[32 * tb + col][k0 + kq]), lds8(&sm.B[32 * pb + col][k0 + kq]),
                    g0);
          g1 = mfma(lds8(&sm.C[32 * tb + col][k0 + 16 + kq]),
                    lds8(&sm.B[32 * pb + col][k0 + 16 + kq]), g1);
        }
        const int sc = 32 * pb + col;
        const double cs = sm.cum[sc];
        const float ds = sm.delta[sc];
        double ct[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) ct[v] = sm.cum[32 * tb + acc_row(v, lane)];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int t = 32 * tb + acc_row(v, lane);
          const float m =
              sc <= t ? (g0[v] + g1[v]) * hw_exp2((float)(ct[v] - cs) * kLog2e) * ds : 0.0f;
          split_hl(m, sm.M[0][t][sc], sm.M[1][t][sc]);
        }
      }
    } else if (!ywave) {
      // ---- phase 2 (state): x o w.  A lane takes 16 consecutive steps of
      // one channel, so its reads and writes are 16-byte pieces (10 LDS
      // operations instead of 48 single values).
      const int L = (wv - 4) * 64 + lane;  // 0 .. 255
      const int p = L >> 2, tq = (L & 3) * 16;
      const uint4 xq[2] = {*reinterpret_cast<const uint4*>(&sm.Xt[p][tq]),
                           *reinterpret_cast<const uint4*>(&sm.Xt[p][tq + 8])};
      float wts[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = *reinterpret_cast<const float4*>(&sm.w[tq + 4 * q]);
        wts[4 * q] = f.x; wts[4 * q + 1] = f.y; wts[4 * q + 2] = f.z; wts[4 * q + 3] = f.w;
      }
      uint32_t hw[8], lw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 v4 = xq[i >> 2];
        const uint32_t word = (i & 3) == 0 ? v4.x : (i & 3) == 1 ? v4.y : (i & 3) == 2 ? v4.z : v4.w;
        const float a = bf16_lo(word) * wts[2 * i], c = bf16_hi(word) * wts[2 * i + 1];
        hw[i] = pack_bf16x2(a, c);
        lw[i] = pack_bf16x2(a - bf16_lo(hw[i]), c - bf16_hi(hw[i]));
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t* src = h ? lw : hw;
        *reinterpret_cast<uint4*>(&sm.Xw[h][p][tq]) = make_uint4(src[0], src[1], src[2], src[3]);
        *reinterpret_cast<uint4*>(&sm.Xw[h][p][tq + 8]) = make_uint4(src[4], src[5], src[6], src[7]);
      }
      if (emit) {
        // the entering state's part of Y over this wave's n half,
        // C[t][n] H[p][n] summed over n, taken straight from the state
        // registers.  Registers 8 q .. 8 q + 7 of tile i hold, in lane half
        // hl, the states n = 32 i + 16 q + 4 hl + (0..3) and the same + 8:
        // those are the lane's 8 k values of a 16-deep product, so the C
        // operand is read in that order (two 8-byte pieces) and the state
        // enters as hi + lo bf16 halves without a trip through LDS.
        const int hl4 = 4 * (lane >> 5);
        bf16x8 bh[NT][2], bl[NT][2];
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            uint32_t hw4[4], lw4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float v0 = hacc[i][8 * q + 2 * j], v1 = hacc[i][8 * q + 2 * j + 1];
              hw4[j] = pack_bf16x2(v0, v1);
              lw4[j] = pack_bf16x2(v0 - bf16_lo(hw4[j]), v1 - bf16_hi(hw4[j]));
            }
            bh[i][q] = __builtin_bit_cast(bf16x8, make_uint4(hw4[0], hw4[1], hw4[2], hw4[3]));
            bl[i][q] = __builtin_bit_cast(bf16x8, make_uint4(lw4[0], lw4[1], lw4[2], lw4[3]));
          }
        const int nh = wv >= 6 ? 1 : 0;  // this wave's n half
        // both t blocks at once: two independent accumulator chains
        f32x16 acc[2] = {};
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            bf16x8 a[2];
#pragma unroll
            for (int tbk = 0; tbk < 2; ++tbk) {
              const uint16_t* cp = &sm.C[32 * tbk + col][nbase + 32 * i + 16 * q + hl4];
              const uint2 c0 = *reinterpret_cast<const uint2*>(cp);
              const uint2 c1 = *reinterpret_cast<const uint2*>(cp + 8);
              a[tbk] = __builtin_bit_cast(bf16x8, make_uint4(c0.x, c0.y, c1.x, c1.y));
            }
            acc[0] = mfma(a[0], bh[i][q], acc[0]);
            acc[1] = mfma(a[1], bh[i][q], acc[1]);
            acc[0] = mfma(a[0], bl[i][q], acc[0]);
            acc[1] = mfma(a[1], bl[i][q], acc[1]);
          }
#pragma unroll
        for (int tbk = 0; tbk < 2; ++tbk)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            sm.Yp[nh][tbk][pb][q4][lane] = make_float4(acc[tbk][4 * q4], acc[tbk][4 * q4 + 1],
                                                       acc[tbk][4 * q4 + 2], acc[tbk][4 * q4 + 3]);
      }
    }
    __syncthreads();

    if (ywave && emit) {
      // ---- phase 3 (output): the entering state's part (the state waves'
      // two partials, decayed to each step), (L o C B^T) X, the skip, the
      // gate, the store
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 p0 = sm.Yp[0][tb][pb][q4][lane], p1 = sm.Yp[1][tb][pb][q4][lane];
        const float4 e4 = *reinterpret_cast<const float4*>(&sm.ecum[32 * tb + acc_row(4 * q4, lane)]);
        ya[4 * q4] = (p0.x + p1.x) * e4.x;
        ya[4 * q4 + 1] = (p0.y + p1.y) * e4.y;
        ya[4 * q4 + 2] = (p0.z + p1.z) * e4.z;
        ya[4 * q4 + 3] = (p0.w + p1.w) * e4.w;
      }
#pragma unroll
      for (int k0 = 0; k0 < kQ; k0 += 16) {
        const bf16x8 bx = lds8(&sm.Xt[32 * pb + col][k0 + kq]);
        ya = mfma(lds8(&sm.M[0][32 * tb + col][k0 + kq]), bx, ya);
        yb = mfma(lds8(&sm.M[1][32 * tb + col][k0 + kq]), bx, yb);
      }
      // x for the D skip and z for the gate: each group of 4 result
      // registers is 4 consecutive steps of this lane's channel, one 8-byte
      // read each
      uint16_t xs[16], zs[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t4 = 32 * tb + acc_row(4 * q, lane);
        const uint2 x4 = *reinterpret_cast<const uint2*>(&sm.Xt[32 * pb + col][t4]);
        xs[4 * q] = (uint16_t)(x4.x & 0xffffu);
        xs[4 * q + 1] = (uint16_t)(x4.x >> 16);
        xs[4 * q + 2] = (uint16_t)(x4.y & 0xffffu);
        xs[4 * q + 3] = (uint16_t)(x4.y >> 16);
        if constexpr (HAS_Z) {
          const uint2 z4 = *reinterpret_cast<const uint2*>(&sm.Zt[32 * pb + col][t4]);
          zs[4 * q] = (uint16_t)(z4.x & 0xffffu);
          zs[4 * q + 1] = (uint16_t)(z4.x >> 16);
          zs[4 * q + 2] = (uint16_t)(z4.y & 0xffffu);
          zs[4 * q + 3] = (uint16_t)(z4.y >> 16);
        }
      }
      // the wave's 32 x 32 tile of outputs goes through LDS so that it
      // leaves as 16-byte pieces (8 channels of one step) rather than 2-byte
      // stores; only this wave touches its tile of Yo
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float y = fmaf(Dh, bf16_bits(xs[v]), ya[v] + yb[v]);
        if constexpr (HAS_Z) y *= silu_f32(bf16_bits(zs[v]));
        sm.Yo[32 * tb + acc_row(v, lane)][32 * pb + col] = to_bf16(y);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int piece = lane + 64 * k;          // 128 pieces: 32 steps x 4
        const int t = 32 * tb + (piece >> 2), p = 32 * pb + 8 * (piece & 3);
        const uint4 v = *reinterpret_cast<const uint4*>(&sm.Yo[t][p]);
        if (t0 + t < t_end) *reinterpret_cast<uint4*>(ob + (t0 + t) * HP + p) = v;
      }
    } else if (!ywave) {
      // ---- phase 3 (state): H^T = exp(cum_end) H^T + B^T (X o w)
      const float dec = sm.dec_end;
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        f32x16 lo = {};
#pragma unroll
        for (int v = 0; v < 16; ++v) hacc[i][v] *= dec;
#pragma unroll
        for (int k0 = 0; k0 < kQ; k0 += 16) {
          const bf16x8 bb = lds8(&sm.Bt[nbase + 32 * i + col][k0 + kq]);
          hacc[i] = mfma(bb, lds8(&sm.Xw[0][32 * pb + col][k0 + kq]), hacc[i]);
          lo = mfma(bb, lds8(&sm.Xw[1][32 * pb + col][k0 + kq]), lo);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) hacc[i][v] += lo[v];
      }
    }
    if (!ywave && c + 1 < chunks) load_bc(t0 + kQ);  // lands during the barrier wait
    __syncthreads();
  }

  // the end state: the caller's (whole pairs, a split pair's last segment)
  // or the aggregate task's
  float* h_out = agg ? ws.S + ((int64_t)sp * (s.P - 1) + seg) * seg_elems
                     : ((!split || seg == s.P - 1) && state ? state + srow * N : nullptr);
  if (!ywave && h_out) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        h_out[(32 * pb + col) * N + nbase + 32 * i + acc_row(v, lane)] = hacc[i][v];
  }
  if (agg && tid == 0) ws.sum[(int64_t)sp * (s.P - 1) + seg] = seg_sum;
}

// Entering state of every segment of the split pairs, per (split pair, state
// element): h_in[0] = the caller's initial state (or 0), h_in[k + 1] =
// exp(sum_k) h_in[k] + S_k, in fp64.
__global__ void __launch_bounds__(256)
    mamba2_combine_kernel(const float* __restrict__ state, const float* __restrict__ S,
                          const double* __restrict__ sum, float* __restrict__ hin,
                          int whole, int split, int P, int64_t seg_elems, int load_state) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)split * seg_elems) return;
  const int sp = (int)(i / seg_elems);
  const int64_t e = i - (int64_t)sp * seg_elems;
  double h = load_state ? (double)state[(int64_t)(whole + sp) * seg_elems + e] : 0.0;
  for (int k = 0; k < P; ++k) {
    hin[((int64_t)sp * P + k) * seg_elems + e] = (float)h;
    if (k + 1 < P)
      h = exp(sum[(int64_t)sp * (P - 1) + k]) * h +
          (double)S[((int64_t)sp * (P - 1) + k) * seg_elems + e];
  }
}

template <int N, bool HAS_Z>
hipError_t launch_pass(const Mamba2Params& p, const M2Shape& s, const M2Work& ws,
                       int grid, hipStream_t st) {
  hipLaunchKernelGGL((mamba2_scan_kernel<N, HAS_Z>), dim3((unsigned)grid), dim3(kThreads), 0,
                     st, static_cast<const uint16_t*>(p.x), static_cast<const uint16_t*>(p.dt),
                     p.A, static_cast<const uint16_t*>(p.B), static_cast<const uint16_t*>(p.C),
                     p.D, static_cast<const uint16_t*>(p.z), p.bias,
                     static_cast<uint16_t*>(p.out), p.state, s, ws);
  return hipGetLastError();
}

template <int N>
hipError_t launch_n(const Mamba2Params& p, hipStream_t st) {
  M2Shape s{p.L, (int32_t)p.nheads, (int32_t)p.ngroups, p.softplus, p.load_state,
            (int32_t)p.whole, p.segments, p.seg_chunks, 0, 0};
  const int split = (int)(p.batch * p.nheads - p.whole);
  const M2Work ws{p.ws_S, p.ws_sum, p.ws_hin};
  s.n_agg = split > 0 ? split * (p.segments - 1) : 0;
  auto pass = [&](int grid) {
    return p.z ? launch_pass<N, true>(p, s, ws, grid, st)
               : launch_pass<N, false>(p, s, ws, grid, st);
  };
  hipError_t e = hipSuccess;
  if (s.n_agg + s.whole > 0) {
    s.pass = 0;
    e = pass(s.n_agg + s.whole);
  }
  if (e == hipSuccess && split > 0) {
    const int64_t seg_elems = (int64_t)kP * N;
    const int64_t threads = split * seg_elems;
    hipLaunchKernelGGL(mamba2_combine_kernel, dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, st, p.state, p.ws_S, p.ws_sum, p.ws_hin, (int)p.whole,
                       split, p.segments, seg_elems, p.load_state);
    e = hipGetLastError();
    if (e == hipSuccess) {
      s.pass = 1;
      e = pass(split * p.segments);
    }
  }
  return e;
}

}  // namespace

int mamba2_headdim() { return kP; }

// The time split (pure arithmetic).  A workgroup scans its rows in a fixed
// time per chunk whatever the load, so pairs beyond whole rounds of CUs (or
// all pairs, when there are fewer than CUs) are cut into segments that fill
// the CUs, at the cost of a state-only pass over all but their last segment.
void mamba2_plan(int64_t pairs, int64_t L, int cus, int forced, Mamba2Params* p) {
  const int64_t chunks = (L + kQ - 1) / kQ;
  int64_t whole = pairs, P = 1;
  if (forced > 0) {
    P = forced;
    if (P > 1) whole = 0;
  } else if (pairs >= cus) {
    const int64_t rest = pairs % cus;
    if (rest > 0) {
      P = cus / rest;
      if (P > 1) whole = pairs - rest;
    }
  } else {
    P = cus / pairs;
    if (P > 1) whole = 0;
  }
  P = std::min<int64_t>(P, chunks);
  int64_t seg_chunks = chunks;
  if (P > 1) {
    seg_chunks = (chunks + P - 1) / P;
    P = (chunks + seg_chunks - 1) / seg_chunks;  // whole chunks per segment
  }
  if (P < 2) {
    whole = pairs;
    P = 1;
    seg_chunks = chunks;
  }
  p->whole = whole;
  p->segments = (int32_t)P;
  p->seg_chunks = (int32_t)seg_chunks;
}

int64_t mamba2_workspace(const Mamba2Params& p, void* ws, Mamba2Params* q) {
  const int64_t split = p.batch * p.nheads - p.whole;
  if (split <= 0) return 0;
  const int64_t seg = (int64_t)kP * p.N;
  const int64_t bS = split * (p.segments - 1) * seg * 4;
  const int64_t bsum = split * (p.segments - 1) * 8;
  const int64_t bhin = split * p.segments * seg * 4;
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  if (ws && q) {
    char* base = static_cast<char*>(ws);
    q->ws_S = reinterpret_cast<float*>(base);
    q->ws_sum = reinterpret_cast<double*>(base + up(bS));
    q->ws_hin = reinterpret_cast<float*>(base + up(bS) + up(bsum));
  }
  return up(bS) + up(bsum) + up(bhin);
}

hipError_t launch_mamba2_scan(const Mamba2Params& p, hipStream_t st) {
  switch (p.N) {
    case 64: return launch_n<64>(p, st);
    case 128: return launch_n<128>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mssm
