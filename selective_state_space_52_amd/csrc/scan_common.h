// scan_common.h -- device helpers shared by the forward and backward scan
// kernels: per-lane loads and stores of a row's timesteps, and the packed
// per-wave B/C runs read with wide scalar loads.
#pragma once

#include "dev_math.h"

namespace mssm {

constexpr int kLanes = 64;

// KC consecutive io values of one row, as loaded (bf16 pairs or fp32 words).
template <bool BF16, int KC>
struct Raw {
  static constexpr int W = BF16 ? KC / 2 : KC;
  uint32_t w[W];
};

template <bool BF16, int KC>
__device__ __forceinline__ float raw_get(const Raw<BF16, KC>& r, int k) {
  if constexpr (BF16)
    return (k & 1) ? bf16_hi(r.w[k >> 1]) : bf16_lo(r.w[k >> 1]);
  else
    return __uint_as_float(r.w[k]);
}

template <bool BF16, int KC>
__device__ __forceinline__ void raw_zero(Raw<BF16, KC>& r) {
#pragma unroll
  for (int i = 0; i < Raw<BF16, KC>::W; ++i) r.w[i] = 0u;
}

// Values [t, t + KC) of a row starting at element offset `off`; `nvalid` of
// them exist (the rest read as 0).  VEC: the row and every 16-byte piece
// (the whole chunk when it is 8 or 4 bytes) are aligned, and a piece is
// either whole or absent.  Without VEC, consecutive timesteps sit `ts`
// elements apart (1 for rows stored time-fastest, the channel count for the
// (batch, length, channel) layout).
template <bool BF16, bool VEC, int KC>
__device__ __forceinline__ void load_chunk(Raw<BF16, KC>& r, const void* base,
                                           int64_t off, int64_t nvalid,
                                           int64_t ts = 1) {
  constexpr int W = Raw<BF16, KC>::W;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(
      static_cast<const char*>(base) + off * (BF16 ? 2 : 4));
  if constexpr (VEC) {
    constexpr int PV = BF16 ? 2 : 1;  // values per 32-bit word
    if constexpr (W >= 4) {
#pragma unroll
      for (int q = 0; q < W / 4; ++q) {
        if (4 * q * PV < nvalid) {
          const uint4 v = reinterpret_cast<const uint4*>(src)[q];
          r.w[4 * q] = v.x; r.w[4 * q + 1] = v.y; r.w[4 * q + 2] = v.z; r.w[4 * q + 3] = v.w;
        } else {
          r.w[4 * q] = r.w[4 * q + 1] = r.w[4 * q + 2] = r.w[4 * q + 3] = 0u;
        }
      }
    } else if constexpr (W == 2) {
      if (nvalid > 0) {
        const uint2 v = *reinterpret_cast<const uint2*>(src);
        r.w[0] = v.x; r.w[1] = v.y;
      } else {
        r.w[0] = r.w[1] = 0u;
      }
    } else {
      static_assert(W == 1, "chunk of 1 word");
      r.w[0] = nvalid > 0 ? src[0] : 0u;
    }
  } else {
    if constexpr (BF16) {
      const uint16_t* s = static_cast<const uint16_t*>(base) + off;
#pragma unroll
      for (int i = 0; i < W; ++i) {
        const uint32_t lo = (2 * i < nvalid) ? s[2 * i * ts] : 0u;
        const uint32_t hi = (2 * i + 1 < nvalid) ? s[(2 * i + 1) * ts] : 0u;
        r.w[i] = lo | (hi << 16);
      }
    } else {
      const uint32_t* s = static_cast<const uint32_t*>(base) + off;
#pragma unroll
      for (int i = 0; i < W; ++i) r.w[i] = (i < nvalid) ? s[i * ts] : 0u;
    }
  }
}

template <bool BF16, bool VEC, int KC>
__device__ __forceinline__ void store_chunk(void* base, int64_t off,
                                            const float (&o)[KC],
                                            int64_t nvalid, int64_t ts = 1) {
  if (VEC && nvalid >= KC) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<char*>(base) +
                                                off * (BF16 ? 2 : 4));
    constexpr int W = BF16 ? KC / 2 : KC;
    uint32_t w[W];
#pragma unroll
    for (int i = 0; i < W; ++i)
      w[i] = BF16 ? pack_bf16x2(o[2 * i], o[2 * i + 1]) : __float_as_uint(o[i]);
    if constexpr (W >= 4) {
#pragma unroll
      for (int q = 0; q < W / 4; ++q)
        reinterpret_cast<uint4*>(dst)[q] =
            make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
    } else if constexpr (W == 2) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    } else {
      dst[0] = w[0];
    }
  } else if constexpr (BF16) {
    uint16_t* dst = static_cast<uint16_t*>(base) + off;
#pragma unroll
    for (int k = 0; k < KC; ++k)
      if (k < nvalid) dst[k * ts] = to_bf16(o[k]);
  } else {
    float* dst = static_cast<float*>(base) + off;
#pragma unroll
    for (int k = 0; k < KC; ++k)
      if (k < nvalid) dst[k * ts] = o[k];
  }
}

// Vector-path loads and stores from a lane's own row pointer `row` (bytes):
// values [t, t + KC) of the row, t uniform across the wave.  The caller keeps
// [t, t + KC) inside the row and 16-byte aligned pieces (8-byte for a 4-value
// bf16 chunk), so the only per-tile vector work is one 64-bit address add.
template <bool BF16, int KC>
__device__ __forceinline__ void load_chunk_row(Raw<BF16, KC>& r, const char* row, int t) {
  constexpr int W = Raw<BF16, KC>::W;
  const uint32_t* src =
      reinterpret_cast<const uint32_t*>(row + (int64_t)t * (BF16 ? 2 : 4));
  if constexpr (W >= 4) {
#pragma unroll
    for (int q = 0; q < W / 4; ++q) {
      const uint4 v = reinterpret_cast<const uint4*>(src)[q];
      r.w[4 * q] = v.x; r.w[4 * q + 1] = v.y; r.w[4 * q + 2] = v.z; r.w[4 * q + 3] = v.w;
    }
  } else if constexpr (W == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(src);
    r.w[0] = v.x; r.w[1] = v.y;
  } else {
    r.w[0] = src[0];
  }
}

// Stores the whole chunk [t, t + KC) when `nvalid` > 0: on the vector path a
// row's length and its time segments are multiples of the chunk, so a chunk
// is either whole or past the end.
template <bool BF16, int KC>
__device__ __forceinline__ void store_chunk_row(char* row, int t, const float (&o)[KC],
                                                int nvalid) {
  if (nvalid <= 0) return;
  uint32_t* dst = reinterpret_cast<uint32_t*>(row + (int64_t)t * (BF16 ? 2 : 4));
  constexpr int W = BF16 ? KC / 2 : KC;
  uint32_t w[W];
#pragma unroll
  for (int i = 0; i < W; ++i)
    w[i] = BF16 ? pack_bf16x2(o[2 * i], o[2 * i + 1]) : __float_as_uint(o[i]);
  if constexpr (W >= 4) {
#pragma unroll
    for (int q = 0; q < W / 4; ++q)
      reinterpret_cast<uint4*>(dst)[q] =
          make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
  } else if constexpr (W == 2) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  } else {
    dst[0] = w[0];
  }
}

// B_t and C_t packed for the scan, in the io dtype, laid out
// [b][wave g][t][B_t[n0..n0+NPW), C_t[n0..n0+NPW)] so that one wave's values
// for a batch of consecutive tokens are one contiguous 64-byte run read by a
// single wide scalar load (the address is the same for every lane).  bf16
// stays packed two to a word and is widened where it is used, which keeps the
// scalar-cache footprint of the runs small.
template <int NPW, bool BF16>
struct BCLayout {
  static constexpr int kWordsPerStep = BF16 ? NPW : 2 * NPW;  // 32-bit words
  // tokens per batch: a 64-byte batch, or one token when a token is larger
  static constexpr int kSteps = kWordsPerStep >= 16 ? 1 : 16 / kWordsPerStep;
  static constexpr int kWordsPerBatch = kSteps * kWordsPerStep;
};

// words of one wave's run, padded to whole 64-byte batches
__host__ __device__ inline int64_t bc_run_words(int64_t L, int words_per_step) {
  return (L * words_per_step + 15) / 16 * 16;
}

template <int NPW, bool BF16>
struct alignas(16) BCBatch {
  uint32_t w[BCLayout<NPW, BF16>::kWordsPerBatch];
};

// value j (B for j < NPW, C after) of token i of a batch (or a raw run)
template <int NPW, bool BF16>
__device__ __forceinline__ float bc_val(const uint32_t* w, int i, int j) {
  constexpr int WPS = BCLayout<NPW, BF16>::kWordsPerStep;
  if constexpr (BF16) {
    const uint32_t x = w[i * WPS + (j >> 1)];
    return (j & 1) ? bf16_hi(x) : bf16_lo(x);
  } else {
    return __uint_as_float(w[i * WPS + j]);
  }
}

}  // namespace mssm
