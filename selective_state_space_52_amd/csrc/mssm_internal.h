// mssm_internal.h -- launch parameters shared by the host API and the kernels.
// Not part of the public ABI (include/mssm.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mssm.h"

namespace mssm {

// One forward-scan call, as the kernels see it.
//
// Work is cut into 64-channel groups: group gi covers channels
// [64*(gi % groups_per_batch), +64) of batch gi / groups_per_batch, one lane
// per channel.  Groups [0, whole_groups) are scanned in one piece; the other
// groups are cut into `segments` time segments of `seg_len` steps.  For those,
// aggregate tasks summarise every segment but the last (its end state and its
// sum of Delta; segment 0 from the initial state, the others from zero), and
// each segment's main task folds the summaries of the segments before it into
// its initial state.  Aggregate and main tasks run in one launch; an
// aggregate task publishes its summary through a flag that the main tasks
// after it wait for.
struct ScanParams {
  const void* u;
  const void* delta;
  const void* z;          // may be null
  const float* A;
  const void* B;
  const void* C;
  const float* D;         // may be null
  const float* bias;      // may be null
  void* out;
  float* last_state;      // may be null; read first when load_state
  int64_t batch, dim, L;
  int32_t softplus;
  int32_t load_state;
  int32_t groups_per_batch;
  int32_t whole_groups;
  int32_t split_groups;
  int32_t segments;
  int64_t seg_len;
  // workspace of the split groups, indexed by split row sr = 64*sj + lane
  float* ws_S;            // [sr][segments-1][N] segment end states
  double* ws_sum;         // [sr][segments-1] segment sums of Delta
  float* ws_h0;           // [sr][N] initial state (with load_state)
  uint32_t* ws_flags;     // [segment][split group] summary published; zeroed
                          // by the B/C pack ahead of every scan launch
  void* ws_bc;            // B, C packed per wave run, io dtype
                          // [b][wave][t][B, C of the wave's N / waves states]
  void* ev_start;         // optional hipEvent_t recorded around the scan
  void* ev_stop;          // kernel (timing hook), or null
  // causal conv feeding the scan (conv_w null: `u` is the scan input itself;
  // otherwise `u` holds the conv input x)
  const float* conv_w;    // (dim, 4) fp32
  const float* conv_b;    // (dim) fp32 or null
  const void* conv_init;  // (batch, dim, 3) io dtype or null
  void* u_out;            // (batch, dim, L) io dtype: conv output, or null
  int32_t layout_bld;     // u, delta, z, out, u_out are (batch, L, dim)
  int32_t ngroups;        // B/C groups (B, C are (batch, L, ngroups, N))
  int32_t bc_state_major; // B, C are (batch, ngroups, N, L)
  int32_t cus;            // compute units of the device (work plan)
};

// Standalone causal depthwise conv: out = act(bias + sum_k w[k] x[t-K+1+k]).
struct ConvParams {
  const void* x;
  const float* w;         // (dim, width) fp32
  const float* bias;      // (dim) fp32 or null
  const void* init;       // (batch, dim, width-1) io dtype or null
  void* out;
  int64_t batch, dim, L;
  int32_t width;          // 2, 3 or 4
  int32_t silu;
  int32_t layout_bld;     // x, out are (batch, L, dim)
};

// Gradients of the causal conv: x, dout, dx (batch, dim, L) io dtype; w
// (dim, width) fp32; dw (dim, width) and dbias (dim) fp32 (dbias may be
// null); init, dinit (batch, dim, width-1) io dtype (both may be null).
struct ConvBwdParams {
  const void* x;
  const float* w;
  const float* bias;
  const void* init;
  const void* dout;
  void* dx;
  float* dw;
  float* dbias;
  void* dinit;
  int64_t batch, dim, L;
  int32_t width;          // 2, 3 or 4
  int32_t silu;
};

struct UpdateParams {
  float* state;
  const void* x;
  const void* dt;
  const void* z;          // may be null
  const float* A;
  const void* B;
  const void* C;
  const float* D;         // may be null
  const float* bias;      // may be null
  void* out;
  int64_t batch, dim;
  int32_t softplus;
  int32_t ngroups;        // B, C are (batch, ngroups, N)
  int32_t stream_state;   // the state with non-temporal loads and stores
};

// One backward-scan call.  Gradients of sum(dout * out) + sum(dlast *
// last_state) with respect to every input of the forward scan.
//
// Rows are cut into `segments` time segments of `seg_tiles` tiles; a task is
// one (64-channel group, segment).  Pass F scans every segment from a zero
// state (all tasks in parallel), keeping the state and the running sum of
// Delta at every tile start, the segment's end state and sum of Delta, and
// its reverse aggregate (the gradient the segment sends to its start for a
// zero incoming gradient).  A combine pass turns these into each segment's
// true initial state and incoming gradient; pass R then walks each segment's
// tiles backwards (all tasks in parallel).
struct BwdParams {
  const void* u;
  const void* delta;
  const void* z;          // may be null (then dz is null)
  const void* dout;
  const float* A;
  const void* B;
  const void* C;
  const float* D;         // may be null
  const float* bias;      // may be null
  const float* h0;        // may be null (zero initial state)
  const float* dlast;     // may be null (zero)
  void* du;
  void* ddelta;
  void* dz;               // may be null
  float* dA;
  float* dB;
  float* dC;
  float* dD;              // may be null
  float* dbias;           // may be null
  float* dh0;             // may be null
  int64_t batch, dim, L;
  int32_t softplus;
  int32_t groups_per_batch;
  int32_t tiles;          // ceil(L / tile); runs and partials hold tiles*tile steps
  int32_t segments;       // time segments per row
  int32_t seg_tiles;      // tiles per segment (the last may have fewer)
  int32_t layout_bld;     // the per-element arrays are (batch, L, dim)
  int32_t ngroups;        // B/C groups (B, C, dB, dC are (batch, L, ngroups, N))
  int32_t bc_state_major; // B, C, dB, dC are (batch, ngroups, N, L)
  // workspace (task = group * segments + segment; lane-contiguous rows)
  void* ws_bc;            // B, C packed per wave run, zero-padded to whole tiles
  float* ws_ck;           // [group][tile][n][lane] state at tile start, from a
                          // zero state at the segment start
  float* ws_cd;           // [group][tile][lane] sum of Delta from the segment
                          // start to the tile start
  float* ws_S;            // [task][n][lane] segment end state from zero
  float* ws_R;            // [task][n][lane] segment reverse aggregate
  double* ws_sum;         // [task][lane] segment sum of Delta
  float* ws_hin;          // [task][n][lane] segment initial state
  float* ws_gin;          // [task][n][lane] gradient entering the segment end
  float* ws_dbc;          // [b][group in batch][t][B, C][n] channel-group sums
  float* ws_dA;           // [segment][b][d][n] partial dA
  float* ws_dDb;          // [segment][b][d][dD, dbias] partial sums
  void* ev_start;         // optional timing events around pass F, the
  void* ev_stop;          // combine and pass R
};

// Where a forward call's workspace comes from: allocated stream-ordered for
// the call (kAllocate), supplied by the caller (kCaller), or the library's
// fixed scratch array of the current device (kScratch: ws_bytes is its size).
enum class WsMode { kAllocate, kCaller, kScratch };

// Device address of the current device's allocation-free scratch array
// (noalloc.hip), looked up on the first call per device; nullptr and *err set
// if the lookup fails.
void* noalloc_scratch(hipError_t* err);

// The forward scan entry shared by the C ABI's forward calls (mssm_api.cpp);
// returns an MSSM_* status.  conv_w non-null: `u` is the conv input x.
int scan_fwd_entry(const void* u, const void* delta, const float* A,
                   const void* B, const void* C, const float* D, const void* z,
                   const float* delta_bias, int softplus, void* out,
                   float* last_state, const float* conv_w, const float* conv_b,
                   const void* conv_init, void* u_out, void* ws, int64_t ws_bytes,
                   WsMode mode, const ::mssm_dims* dims, void* stream);

// Waves per 64-channel workgroup: each wave owns dstate / waves states.
int scan_waves_per_group(int N);
// Repack B and C, (batch, L, groups, N), into per-wave runs, one per
// (batch entry, group, wave) for `waves` waves per channel group: `steps`
// (>= L) timesteps per run, zeros from L on, `run_words` 32-bit words per
// run; the runs hold bf16 pairs (dst_bf16) or fp32 values.  With
// state_major, B and C are (batch, groups, N, L) instead.  The same launch
// zeroes `nflags` words at `flags` (may be 0 / null).
// ALU issue-rate probe (kind 0: fma, 1: exp, 2: the state-element mix),
// `blocks` workgroups of 256 threads, one float per thread into sink.
hipError_t launch_valu_probe(int kind, int blocks, int iters, float* sink,
                             hipStream_t stream);
hipError_t launch_bc_pack(const void* B, const void* C, void* packed,
                          int64_t batch, int64_t groups, int64_t L, int64_t steps,
                          int N, int waves, bool src_bf16, bool dst_bf16,
                          int64_t run_words, uint32_t* flags, int64_t nflags,
                          bool state_major, hipStream_t stream);
// Bytes of the packed B/C runs of one forward call.
int64_t scan_bc_workspace_bytes(int64_t batch, int64_t L, int N, bool bf16);

hipError_t launch_scan(const ScanParams& p, int N, bool bf16, bool vec,
                       hipStream_t stream);
// the forward scan per state size (one translation unit per group of sizes)
hipError_t launch_scan_n1(const ScanParams&, bool, bool, hipStream_t);
hipError_t launch_scan_n2(const ScanParams&, bool, bool, hipStream_t);
hipError_t launch_scan_n4(const ScanParams&, bool, bool, hipStream_t);
hipError_t launch_scan_n8(const ScanParams&, bool, bool, hipStream_t);
hipError_t launch_scan_n16(const ScanParams&, bool, bool, hipStream_t);
hipError_t launch_scan_n32(const ScanParams&, bool, bool, hipStream_t);
hipError_t launch_scan_n64(const ScanParams&, bool, bool, hipStream_t);
hipError_t launch_scan_n128(const ScanParams&, bool, bool, hipStream_t);
// Backward: timesteps per tile, waves per group, segments, workspace, launch.
int bwd_tile();
int bwd_waves_per_group(int N);
// Pass R workgroups resident per CU (runtime occupancy query, cached).
int bwd_wgs_per_cu(int N, bool bf16);
// Time segments per row: `forced` (> 0) if given, else enough tasks to fill
// the CUs' workgroup slots in whole rounds, with segments of at least 4 tiles.
int bwd_segments(int64_t groups, int64_t tiles, int cus, int wgs_per_cu, int forced);
// Workspace bytes of one backward call; with ws and p non-null also points
// p's workspace fields into ws.
int64_t bwd_workspace(int64_t batch, int64_t dim, int64_t L, int N, bool bf16,
                      int segments, int64_t groups, void* ws, BwdParams* p);
hipError_t launch_scan_bwd(const BwdParams& p, int N, bool bf16, bool vec,
                           hipStream_t stream);
hipError_t launch_state_update(const UpdateParams& p, int N, bool bf16,
                               hipStream_t stream);
hipError_t launch_causal_conv1d_bwd(const ConvBwdParams& p, bool bf16, bool vec,
                                    hipStream_t stream);
hipError_t launch_causal_conv1d(const ConvParams& p, bool bf16, bool vec,
                                hipStream_t stream);

// The Mamba-2 block's scan: x, z, out (batch, L, nheads, headdim) bf16; dt
// (batch, L, nheads) bf16; A, D, bias (nheads) fp32; B, C (batch, L, ngroups,
// N) bf16; state (batch, nheads * headdim, N) fp32, read first when
// load_state.
struct Mamba2Params {
  const void* x;
  const void* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* D;     // may be null
  const void* z;      // may be null
  const float* bias;  // may be null
  void* out;
  float* state;       // may be null unless load_state
  int64_t batch, L, nheads, ngroups, N;
  int32_t softplus, load_state;
  // time split (mamba2_plan) and its workspace (mamba2_workspace)
  int64_t whole;
  int32_t segments, seg_chunks;
  float* ws_S;
  double* ws_sum;
  float* ws_hin;
};
int mamba2_headdim();
// Pairs scanned whole, segments and chunks per segment of the rest; forced
// > 0 asks for that many segments of every pair.
void mamba2_plan(int64_t pairs, int64_t L, int cus, int forced, Mamba2Params* p);
// Workspace bytes of the split; with ws and q non-null also points q's
// workspace fields into ws.
int64_t mamba2_workspace(const Mamba2Params& p, void* ws, Mamba2Params* q);
hipError_t launch_mamba2_scan(const Mamba2Params& p, hipStream_t stream);

}  // namespace mssm
