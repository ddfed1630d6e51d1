// mssm_api.cpp -- the C ABI of libmssm (declared in include/mssm.h):
// argument validation (always before the first HIP call), the work plan of
// the forward scan, and kernel dispatch on the caller's stream.
#include "mssm.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "mssm_internal.h"

namespace {

thread_local char g_last_error[512] = "";
thread_local void* g_ev_start = nullptr;  // timing hook events of this thread
thread_local void* g_ev_stop = nullptr;

void set_hip_error(const char* what, hipError_t e) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", what,
                hipGetErrorString(e), (int)e);
}

constexpr int64_t kLanes = 64;
constexpr int64_t kMinSegment = 512;  // shortest time segment worth a summary
constexpr int kDefaultCUs = 256;      // MI355X compute units

int g_cu_count = 0;  // cached compute-unit count of the current device

// Caches the current device's compute-unit count (first HIP call of a call
// that launches work; validation has finished by then).
void refresh_cu_count() {
  if (g_cu_count > 0) return;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      cus > 0)
    g_cu_count = cus;
}

bool valid_dstate(int64_t n) {
  return n == 1 || n == 2 || n == 4 || n == 8 || n == 16 || n == 32 || n == 64 ||
         n == 128;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
  if (!p || bytes <= 0) return Range{0, 0};
  return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes};
}

bool overlap(Range a, Range b) {
  return a.lo != a.hi && b.lo != b.hi && a.lo < b.hi && b.lo < a.hi;
}

// Overflow-safe a * b * c <= limit for positive values.
bool product_ok(int64_t a, int64_t b, int64_t c, int64_t limit) {
  if (a <= 0 || b <= 0 || c <= 0) return false;
  if (a > limit / b) return false;
  const int64_t ab = a * b;
  return ab <= limit / c;
}

int check_common_dims(const mssm_dims* dims) {
  if (!dims) return MSSM_ERR_NULL;
  if (dims->io_dtype != MSSM_F32 && dims->io_dtype != MSSM_BF16)
    return MSSM_ERR_UNSUPPORTED;
  if (dims->ngroups < 0) return MSSM_ERR_DIMS;
  if (dims->batch <= 0 || dims->dim <= 0 || dims->dstate <= 0 ||
      dims->seqlen <= 0)
    return MSSM_ERR_DIMS;
  if (!valid_dstate(dims->dstate)) return MSSM_ERR_UNSUPPORTED;
  return MSSM_OK;
}

// A caller-supplied workspace: present, 256-byte aligned and large enough
// when the call needs one (need > 0).
int check_workspace(const void* ws, int64_t ws_bytes, int64_t need) {
  if (need <= 0) return MSSM_OK;
  if (!ws || ws_bytes < need || !aligned(ws, 256)) {
    std::snprintf(g_last_error, sizeof(g_last_error),
                  "workspace %p of %lld bytes; the call needs %lld bytes, 256-byte aligned",
                  ws, (long long)ws_bytes, (long long)need);
    return MSSM_ERR_WORKSPACE;
  }
  return MSSM_OK;
}

// B/C groups of a call (0 means 1).
int64_t groups_of(const mssm_dims* dims) { return dims->ngroups > 1 ? dims->ngroups : 1; }

// The scans read one group per 64-channel workgroup.
int check_scan_groups(const mssm_dims* dims) {
  const int64_t G = groups_of(dims);
  if (G > 1 && dims->dim % (kLanes * G) != 0) return MSSM_ERR_UNSUPPORTED;
  return MSSM_OK;
}

// Layout of the forward's workspace: the packed B/C runs, then for the split
// groups' rows the segment end states, the segment sums of Delta, the kept
// initial states and one flag per aggregate.  Sets *bytes, and with p
// non-null points p's workspace fields into ws.
void fwd_workspace(int64_t bc_batches, int64_t L, int N, bool bf16, int64_t split,
                   int64_t segments, void* ws, int64_t* bytes, mssm::ScanParams* p) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  int64_t off = up(mssm::scan_bc_workspace_bytes(bc_batches, L, N, bf16));
  char* base = static_cast<char*>(ws);
  if (p) p->ws_bc = ws;
  if (split > 0) {
    const int64_t rows = split * kLanes;
    if (p) p->ws_S = reinterpret_cast<float*>(base + off);
    off += up(rows * (segments - 1) * N * 4);
    if (p) p->ws_sum = reinterpret_cast<double*>(base + off);
    off += up(rows * (segments - 1) * 8);
    if (p) p->ws_h0 = reinterpret_cast<float*>(base + off);
    off += up(rows * N * 4);
    if (p) p->ws_flags = reinterpret_cast<uint32_t*>(base + off);
    off += up(split * (segments - 1) * 4);
  }
  *bytes = off;
}

// The work plan of the forward scan (pure arithmetic, no HIP call).
//
// A 64-channel group scanned in one piece is one workgroup.  When the groups
// do not fill the CUs evenly, some are cut into time segments joined by a
// carried state: the remainder beyond a whole number of CU rounds is spread
// over the CUs, and when there are few groups and long rows (long sequences)
// every group is cut.  Cutting costs an extra summary pass over all but the
// last segment, so it is only used where idle CUs would cost more.
int make_plan(const mssm_dims* dims, int cus, mssm_plan* plan) {
  const int64_t L = dims->seqlen;
  const int64_t N = dims->dstate;
  const int waves = mssm::scan_waves_per_group((int)N);
  const int64_t tile = 32;  // timesteps per kernel tile
  const int64_t gpb = (dims->dim + kLanes - 1) / kLanes;
  if (gpb > INT32_MAX / dims->batch) return MSSM_ERR_DIMS;
  const int64_t G = gpb * dims->batch;

  int64_t whole = G, segments = 1;
  if (dims->time_segments > 0) {
    segments = dims->time_segments;
    if (segments > 1) whole = 0;
  } else if (L >= 2 * kMinSegment) {
    if (G >= cus) {
      const int64_t rest = G % cus;
      if (rest > 0) {
        whole = G - rest;
        segments = std::min<int64_t>(L / kMinSegment,
                                     std::max<int64_t>(2, (cus + rest - 1) / rest));
      }
    } else if (2 * G <= cus) {
      whole = 0;
      segments = std::min<int64_t>(L / kMinSegment, (4 * cus + G - 1) / G);
    }
  }
  int64_t seg_len = L;
  if (segments > 1) {
    seg_len = (L + segments - 1) / segments;
    seg_len = (seg_len + tile - 1) / tile * tile;  // whole tiles per segment
    segments = (L + seg_len - 1) / seg_len;
  }
  if (segments <= 1) {
    segments = 1;
    whole = G;
    seg_len = L;
  }
  const int64_t split = G - whole;
  if (whole + split * segments > INT32_MAX) return MSSM_ERR_DIMS;

  int64_t ws = 0;
  fwd_workspace(dims->batch * groups_of(dims), L, (int)N, dims->io_dtype == MSSM_BF16,
                split, segments, nullptr, &ws, nullptr);
  std::memset(plan, 0, sizeof(*plan));
  plan->groups = (int32_t)G;
  plan->whole_groups = (int32_t)whole;
  plan->split_groups = (int32_t)split;
  plan->segments = (int32_t)segments;
  plan->segment_len = seg_len;
  plan->waves_per_group = waves;
  plan->kernels = 2;
  plan->workspace_bytes = ws;
  const int64_t io = dims->io_dtype == MSSM_BF16 ? 2 : 4;
  // (batch, dim, L): 8- or 16-byte pieces of a row; (batch, L, dim): 4
  // adjacent channels of one step per lane
  if (dims->flags & MSSM_FLAG_LAYOUT_BLD)
    plan->vector_path = (dims->dim % 4 == 0 && dims->dim * io <= INT32_MAX) ? 1 : 0;
  else
    plan->vector_path = ((L * io) % 16 == 0 && (L % 8) == 0) ? 1 : 0;
  return MSSM_OK;
}

}  // namespace

extern "C" {

int mssm_abi_version(void) { return MSSM_ABI_VERSION; }

int mssm_set_scan_timing_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr)) return MSSM_ERR_NULL;
  g_ev_start = start;
  g_ev_stop = stop;
  return MSSM_OK;
}

int mssm_valu_probe(int kind, int blocks, int iters, float* sink, void* stream) {
  if (sink == nullptr) return MSSM_ERR_NULL;
  if (blocks <= 0 || iters <= 0 || kind < 0 || kind > 4) return MSSM_ERR_DIMS;
  const hipError_t e =
      mssm::launch_valu_probe(kind, blocks, iters, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_hip_error("probe launch", e);
    return MSSM_ERR_HIP;
  }
  return MSSM_OK;
}

const char* mssm_last_error(void) { return g_last_error; }

const char* mssm_status_string(int status) {
  switch (status) {
    case MSSM_OK: return "ok";
    case MSSM_ERR_NULL: return "a required pointer is NULL";
    case MSSM_ERR_DIMS: return "invalid sizes (non-positive, decode seqlen != 1, or too large)";
    case MSSM_ERR_UNSUPPORTED: return "unsupported dstate, dtype, flag or group split";
    case MSSM_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case MSSM_ERR_ALIAS: return "an output overlaps another argument";
    case MSSM_ERR_HIP: return "a HIP runtime call failed (see mssm_last_error)";
    case MSSM_ERR_WORKSPACE:
      return "workspace missing, too small or not 256-byte aligned (see mssm_last_error)";
    default: return "unknown status";
  }
}

int mssm_selective_scan_fwd_plan(const mssm_dims* dims, mssm_plan* plan) {
  if (!plan) return MSSM_ERR_NULL;
  int rc = check_common_dims(dims);
  if (rc != MSSM_OK) return rc;
  if (dims->flags & ~(MSSM_FLAG_LOAD_STATE | MSSM_FLAG_LAYOUT_BLD | MSSM_FLAG_BC_STATE_MAJOR))
    return MSSM_ERR_UNSUPPORTED;
  rc = check_scan_groups(dims);
  if (rc != MSSM_OK) return rc;
  if (dims->time_segments < 0) return MSSM_ERR_DIMS;
  return make_plan(dims, g_cu_count > 0 ? g_cu_count : kDefaultCUs, plan);
}

}  // extern "C"

namespace mssm {

// The forward scan, optionally fed by the causal conv (conv_w non-null: `u`
// is the conv input x).  Workspace: `ws` (ws_bytes long) from the caller, or
// with ws == nullptr and WsMode::kAllocate taken stream-ordered from HIP's
// pool for this call, or (WsMode::kScratch) the library's fixed scratch array
// of ws_bytes.
int scan_fwd_entry(const void* u, const void* delta, const float* A,
                   const void* B, const void* C, const float* D, const void* z,
                   const float* delta_bias, int softplus, void* out,
                   float* last_state, const float* conv_w, const float* conv_b,
                   const void* conv_init, void* u_out, void* ws_in, int64_t ws_bytes,
                   WsMode mode, const mssm_dims* dims, void* stream) {
  int rc = check_common_dims(dims);
  if (rc != MSSM_OK) return rc;
  if (dims->flags & ~(MSSM_FLAG_LOAD_STATE | MSSM_FLAG_LAYOUT_BLD | MSSM_FLAG_BC_STATE_MAJOR))
    return MSSM_ERR_UNSUPPORTED;
  const bool bld = (dims->flags & MSSM_FLAG_LAYOUT_BLD) != 0;
  rc = check_scan_groups(dims);
  if (rc != MSSM_OK) return rc;
  const int64_t G = groups_of(dims);
  if (dims->time_segments < 0) return MSSM_ERR_DIMS;
  const bool load_state = (dims->flags & MSSM_FLAG_LOAD_STATE) != 0;
  if (!u || !delta || !A || !B || !C || !out) return MSSM_ERR_NULL;
  if (load_state && !last_state) return MSSM_ERR_NULL;

  const int64_t batch = dims->batch, dim = dims->dim, N = dims->dstate,
                L = dims->seqlen;
  const size_t io = dims->io_dtype == MSSM_BF16 ? 2 : 4;
  const int64_t lim = INT64_MAX / 16;
  if (L > INT32_MAX - 64 || !product_ok(batch, dim, L, lim) ||
      !product_ok(batch, L, N, lim) || !product_ok(batch, dim, N, lim))
    return MSSM_ERR_DIMS;

  const void* ios[] = {u, delta, B, C, out, z, conv_init, u_out};
  for (const void* p : ios)
    if (p && !aligned(p, io)) return MSSM_ERR_ALIGN;
  const void* f32s[] = {A, D, delta_bias, last_state, conv_w, conv_b};
  for (const void* p : f32s)
    if (p && !aligned(p, 4)) return MSSM_ERR_ALIGN;

  const int64_t ebytes = batch * dim * L * (int64_t)io;
  const int64_t bcbytes = batch * L * G * N * (int64_t)io;
  const Range r_out = range_of(out, ebytes);
  const Range r_state = range_of(last_state, batch * dim * N * 4);
  const Range r_uout = range_of(u_out, ebytes);
  const Range ins[] = {range_of(u, ebytes),      range_of(delta, ebytes),
                       range_of(z, ebytes),      range_of(B, bcbytes),
                       range_of(C, bcbytes),     range_of(A, dim * N * 4),
                       range_of(D, dim * 4),     range_of(delta_bias, dim * 4),
                       range_of(conv_w, dim * 16), range_of(conv_b, dim * 4),
                       range_of(conv_init, batch * dim * 3 * (int64_t)io)};
  for (const Range& r : ins)
    if (overlap(r_out, r) || overlap(r_state, r) || overlap(r_uout, r))
      return MSSM_ERR_ALIAS;
  if (overlap(r_out, r_state) || overlap(r_out, r_uout) || overlap(r_state, r_uout))
    return MSSM_ERR_ALIAS;

  // --- validation done; HIP calls from here on ---
  refresh_cu_count();
  mssm_plan plan;
  rc = make_plan(dims, g_cu_count > 0 ? g_cu_count : kDefaultCUs, &plan);
  if (rc != MSSM_OK) return rc;

  // the (batch, L, dim) vector path reads 4 channels at once and has no conv
  const size_t qa = 4 * io;
  const bool vec =
      bld ? plan.vector_path && !conv_w && aligned(u, qa) && aligned(delta, qa) &&
                aligned(out, qa) && (!z || aligned(z, qa))
          : plan.vector_path && aligned(u, 16) && aligned(delta, 16) && aligned(out, 16) &&
                aligned(B, 16) && aligned(C, 16) && (!z || aligned(z, 16)) &&
                (!u_out || aligned(u_out, 16));

  mssm::ScanParams p;
  std::memset(&p, 0, sizeof(p));
  p.u = u; p.delta = delta; p.z = z; p.A = A; p.B = B; p.C = C; p.D = D;
  p.bias = delta_bias; p.out = out; p.last_state = last_state;
  p.batch = batch; p.dim = dim; p.L = L;
  p.softplus = softplus ? 1 : 0;
  p.load_state = load_state ? 1 : 0;
  p.groups_per_batch = (int32_t)((dim + kLanes - 1) / kLanes);
  p.ngroups = (int32_t)G;
  p.whole_groups = plan.whole_groups;
  p.split_groups = plan.split_groups;
  p.segments = plan.segments;
  p.seg_len = plan.segment_len;
  p.ev_start = g_ev_start;
  p.ev_stop = g_ev_stop;
  p.conv_w = conv_w;
  p.conv_b = conv_b;
  p.conv_init = conv_init;
  p.u_out = u_out;
  p.layout_bld = bld ? 1 : 0;
  p.bc_state_major = (dims->flags & MSSM_FLAG_BC_STATE_MAJOR) ? 1 : 0;
  p.cus = g_cu_count > 0 ? g_cu_count : kDefaultCUs;

  if (mode == WsMode::kCaller) {
    rc = check_workspace(ws_in, ws_bytes, plan.workspace_bytes);
    if (rc != MSSM_OK) return rc;
  } else if (mode == WsMode::kScratch) {
    if (plan.workspace_bytes > ws_bytes) {
      std::snprintf(g_last_error, sizeof(g_last_error),
                    "the call needs %lld bytes of workspace; the allocation-free entry "
                    "point's scratch holds %lld",
                    (long long)plan.workspace_bytes, (long long)ws_bytes);
      return MSSM_ERR_WORKSPACE;
    }
    if (plan.workspace_bytes > 0) {
      hipError_t e = hipSuccess;
      ws_in = mssm::noalloc_scratch(&e);
      if (!ws_in) {
        set_hip_error("hipGetSymbolAddress(scratch)", e);
        return MSSM_ERR_HIP;
      }
    }
  }
  hipStream_t st = (hipStream_t)stream;
  void* ws = ws_in;
  if (mode == WsMode::kAllocate) {
    hipError_t e = hipMallocAsync(&ws, (size_t)plan.workspace_bytes, st);
    if (e != hipSuccess) {
      set_hip_error("hipMallocAsync(workspace)", e);
      return MSSM_ERR_HIP;
    }
  }
  {
    int64_t nb = 0;
    fwd_workspace(batch * G, L, (int)N, io == 2, plan.split_groups, plan.segments, ws, &nb,
                  &p);
  }
  hipError_t e = mssm::launch_scan(p, (int)N, io == 2, vec, st);
  if (e != hipSuccess) set_hip_error("scan launch", e);
  if (mode == WsMode::kAllocate && ws) {
    hipError_t f = hipFreeAsync(ws, st);
    if (e == hipSuccess && f != hipSuccess) {
      set_hip_error("hipFreeAsync(workspace)", f);
      e = f;
    }
  }
  return e == hipSuccess ? MSSM_OK : MSSM_ERR_HIP;
}

}  // namespace mssm

using mssm::WsMode;
using mssm::scan_fwd_entry;

extern "C" {

int mssm_selective_scan_fwd(const void* u, const void* delta, const float* A,
                            const void* B, const void* C, const float* D,
                            const void* z, const float* delta_bias,
                            int softplus, void* out, float* last_state,
                            const mssm_dims* dims, void* stream) {
  return scan_fwd_entry(u, delta, A, B, C, D, z, delta_bias, softplus, out,
                        last_state, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                        WsMode::kAllocate, dims, stream);
}

int mssm_selective_scan_fwd_ws(const void* u, const void* delta, const float* A,
                               const void* B, const void* C, const float* D,
                               const void* z, const float* delta_bias, int softplus,
                               void* out, float* last_state, void* workspace,
                               int64_t workspace_bytes, const mssm_dims* dims,
                               void* stream) {
  return scan_fwd_entry(u, delta, A, B, C, D, z, delta_bias, softplus, out,
                        last_state, nullptr, nullptr, nullptr, nullptr, workspace,
                        workspace_bytes, WsMode::kCaller, dims, stream);
}

int mssm_selective_scan_fwd_conv(const void* x, const float* conv_weight,
                                 const float* conv_bias, const void* conv_init,
                                 const void* delta, const float* A,
                                 const void* B, const void* C, const float* D,
                                 const void* z, const float* delta_bias,
                                 int softplus, void* out, float* last_state,
                                 void* u_out, const mssm_dims* dims,
                                 void* stream) {
  if (!conv_weight) return MSSM_ERR_NULL;
  return scan_fwd_entry(x, delta, A, B, C, D, z, delta_bias, softplus, out,
                        last_state, conv_weight, conv_bias, conv_init, u_out, nullptr, 0,
                        WsMode::kAllocate, dims, stream);
}

int mssm_selective_scan_fwd_conv_ws(const void* x, const float* conv_weight,
                                    const float* conv_bias, const void* conv_init,
                                    const void* delta, const float* A, const void* B,
                                    const void* C, const float* D, const void* z,
                                    const float* delta_bias, int softplus, void* out,
                                    float* last_state, void* u_out, void* workspace,
                                    int64_t workspace_bytes, const mssm_dims* dims,
                                    void* stream) {
  if (!conv_weight) return MSSM_ERR_NULL;
  return scan_fwd_entry(x, delta, A, B, C, D, z, delta_bias, softplus, out,
                        last_state, conv_weight, conv_bias, conv_init, u_out, workspace,
                        workspace_bytes, WsMode::kCaller, dims, stream);
}

int mssm_causal_conv1d_fwd(const void* x, const float* weight,
                           const float* bias, const void* init, int width,
                           int silu, void* out, const mssm_dims* dims,
                           void* stream) {
  if (!dims) return MSSM_ERR_NULL;
  if (dims->io_dtype != MSSM_F32 && dims->io_dtype != MSSM_BF16)
    return MSSM_ERR_UNSUPPORTED;
  if ((dims->flags & ~MSSM_FLAG_LAYOUT_BLD) != 0 || dims->ngroups > 1)
    return MSSM_ERR_UNSUPPORTED;
  if (dims->time_segments != 0) return MSSM_ERR_DIMS;
  if (dims->batch <= 0 || dims->dim <= 0 || dims->seqlen <= 0) return MSSM_ERR_DIMS;
  if (width < 2 || width > 4) return MSSM_ERR_UNSUPPORTED;
  if (!x || !weight || !out) return MSSM_ERR_NULL;
  const int64_t batch = dims->batch, dim = dims->dim, L = dims->seqlen;
  const size_t io = dims->io_dtype == MSSM_BF16 ? 2 : 4;
  if (!product_ok(batch, dim, L, INT64_MAX / 16)) return MSSM_ERR_DIMS;
  const void* ios[] = {x, init, out};
  for (const void* p : ios)
    if (p && !aligned(p, io)) return MSSM_ERR_ALIGN;
  const void* f32s[] = {weight, bias};
  for (const void* p : f32s)
    if (p && !aligned(p, 4)) return MSSM_ERR_ALIGN;
  const int64_t ebytes = batch * dim * L * (int64_t)io;
  const Range r_out = range_of(out, ebytes);
  const Range ins[] = {range_of(x, ebytes), range_of(weight, dim * width * 4),
                       range_of(bias, dim * 4),
                       range_of(init, batch * dim * (width - 1) * (int64_t)io)};
  for (const Range& r : ins)
    if (overlap(r_out, r)) return MSSM_ERR_ALIAS;

  mssm::ConvParams p;
  p.x = x; p.w = weight; p.bias = bias; p.init = init; p.out = out;
  p.batch = batch; p.dim = dim; p.L = L;
  p.width = width;
  p.silu = silu ? 1 : 0;
  p.layout_bld = (dims->flags & MSSM_FLAG_LAYOUT_BLD) ? 1 : 0;
  const bool vec = (L % 8) == 0 && ((L * (int64_t)io) % 16) == 0 &&
                   aligned(x, 16) && aligned(out, 16);
  hipError_t e = mssm::launch_causal_conv1d(p, io == 2, vec, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_hip_error("causal_conv1d launch", e);
    return MSSM_ERR_HIP;
  }
  return MSSM_OK;
}

int mssm_causal_conv1d_bwd(const void* x, const float* weight, const float* bias,
                           const void* init, int width, int silu, const void* dout,
                           void* dx, float* dweight, float* dbias, void* dinit,
                           const mssm_dims* dims, void* stream) {
  if (!dims) return MSSM_ERR_NULL;
  if (dims->io_dtype != MSSM_F32 && dims->io_dtype != MSSM_BF16)
    return MSSM_ERR_UNSUPPORTED;
  if (dims->flags != 0 || dims->ngroups > 1) return MSSM_ERR_UNSUPPORTED;
  if (dims->time_segments != 0) return MSSM_ERR_DIMS;
  if (dims->batch <= 0 || dims->dim <= 0 || dims->seqlen <= 0) return MSSM_ERR_DIMS;
  if (width < 2 || width > 4) return MSSM_ERR_UNSUPPORTED;
  if (!x || !weight || !dout || !dx || !dweight) return MSSM_ERR_NULL;
  const int64_t batch = dims->batch, dim = dims->dim, L = dims->seqlen;
  const size_t io = dims->io_dtype == MSSM_BF16 ? 2 : 4;
  if (!product_ok(batch, dim, L, INT64_MAX / 16) || dim > INT32_MAX) return MSSM_ERR_DIMS;
  const void* ios[] = {x, init, dout, dx, dinit};
  for (const void* p : ios)
    if (p && !aligned(p, io)) return MSSM_ERR_ALIGN;
  const void* f32s[] = {weight, bias, dweight, dbias};
  for (const void* p : f32s)
    if (p && !aligned(p, 4)) return MSSM_ERR_ALIGN;
  const int64_t ebytes = batch * dim * L * (int64_t)io;
  const int64_t ibytes = batch * dim * (width - 1) * (int64_t)io;
  const Range outs[] = {range_of(dx, ebytes), range_of(dweight, dim * width * 4),
                        range_of(dbias, dim * 4), range_of(dinit, ibytes)};
  const Range ins[] = {range_of(x, ebytes), range_of(weight, dim * width * 4),
                       range_of(bias, dim * 4), range_of(init, ibytes),
                       range_of(dout, ebytes)};
  for (int i = 0; i < 4; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return MSSM_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return MSSM_ERR_ALIAS;
  }

  mssm::ConvBwdParams p;
  p.x = x; p.w = weight; p.bias = bias; p.init = init; p.dout = dout;
  p.dx = dx; p.dw = dweight; p.dbias = dbias; p.dinit = dinit;
  p.batch = batch; p.dim = dim; p.L = L;
  p.width = width;
  p.silu = silu ? 1 : 0;
  const bool vec = (L % 8) == 0 && ((L * (int64_t)io) % 16) == 0 && aligned(x, 16) &&
                   aligned(dout, 16) && aligned(dx, 16);
  hipError_t e = mssm::launch_causal_conv1d_bwd(p, io == 2, vec, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_hip_error("causal_conv1d_bwd launch", e);
    return MSSM_ERR_HIP;
  }
  return MSSM_OK;
}

}  // extern "C"

namespace {

// Backward work split and workspace size for dims (HIP calls: the CU count
// and pass R's occupancy); returns MSSM_OK or MSSM_ERR_DIMS.
int bwd_layout(const mssm_dims* dims, int* segments, int64_t* ws_bytes) {
  const int64_t batch = dims->batch, dim = dims->dim, N = dims->dstate, L = dims->seqlen;
  const int64_t gpb = (dim + kLanes - 1) / kLanes;
  const bool bf16 = dims->io_dtype == MSSM_BF16;
  const int tile = mssm::bwd_tile();
  refresh_cu_count();
  const int64_t tiles = (L + tile - 1) / tile;
  const int seg = mssm::bwd_segments(batch * gpb, tiles, g_cu_count > 0 ? g_cu_count : kDefaultCUs,
                                     mssm::bwd_wgs_per_cu((int)N, bf16), dims->time_segments);
  if (batch * gpb * seg > INT32_MAX) return MSSM_ERR_DIMS;
  *segments = seg;
  *ws_bytes = mssm::bwd_workspace(batch, dim, L, (int)N, bf16, seg, groups_of(dims), nullptr,
                                  nullptr);
  return MSSM_OK;
}

int scan_bwd_entry(const void* u, const void* delta, const float* A,
                   const void* B, const void* C, const float* D,
                   const void* z, const float* delta_bias,
                   int softplus, const float* h0, const void* dout,
                   const float* dlast, void* du, void* ddelta,
                   float* dA, float* dB, float* dC, float* dD,
                   void* dz, float* ddelta_bias, float* dh0, void* ws_in,
                   int64_t ws_in_bytes, bool allocate, const mssm_dims* dims,
                   void* stream) {
  int rc = check_common_dims(dims);
  if (rc != MSSM_OK) return rc;
  if (dims->dstate > 32) return MSSM_ERR_UNSUPPORTED;
  if (dims->flags & ~(MSSM_FLAG_LAYOUT_BLD | MSSM_FLAG_BC_STATE_MAJOR))
    return MSSM_ERR_UNSUPPORTED;
  const bool bld = (dims->flags & MSSM_FLAG_LAYOUT_BLD) != 0;
  rc = check_scan_groups(dims);
  if (rc != MSSM_OK) return rc;
  const int64_t G = groups_of(dims);
  if (dims->time_segments < 0) return MSSM_ERR_DIMS;
  if (!u || !delta || !A || !B || !C || !dout || !du || !ddelta || !dA ||
      !dB || !dC)
    return MSSM_ERR_NULL;
  if ((z == nullptr) != (dz == nullptr)) return MSSM_ERR_NULL;

  const int64_t batch = dims->batch, dim = dims->dim, N = dims->dstate,
                L = dims->seqlen;
  const size_t io = dims->io_dtype == MSSM_BF16 ? 2 : 4;
  const int64_t lim = INT64_MAX / 64;
  const int64_t gpb = (dim + kLanes - 1) / kLanes;
  if (L > INT32_MAX - 64 || !product_ok(batch, dim, L, lim) ||
      !product_ok(batch, L, N, lim) || !product_ok(batch, dim, N, lim) ||
      !product_ok(batch * gpb, L + 64, 2 * N * kLanes, lim) ||
      batch * gpb > INT32_MAX)
    return MSSM_ERR_DIMS;

  const void* ios[] = {u, delta, z, dout, B, C, du, ddelta, dz};
  for (const void* p : ios)
    if (p && !aligned(p, io)) return MSSM_ERR_ALIGN;
  const void* f32s[] = {A, D, delta_bias, h0, dlast, dA, dB, dC, dD,
                        ddelta_bias, dh0};
  for (const void* p : f32s)
    if (p && !aligned(p, 4)) return MSSM_ERR_ALIGN;

  const int64_t ebytes = batch * dim * L * (int64_t)io;
  const int64_t bcbytes = batch * L * G * N * (int64_t)io;
  const int64_t sbytes = batch * dim * N * 4;
  const Range outs[] = {range_of(du, ebytes),          range_of(ddelta, ebytes),
                        range_of(dz, ebytes),          range_of(dA, dim * N * 4),
                        range_of(dB, batch * L * G * N * 4),
                        range_of(dC, batch * L * G * N * 4), range_of(dD, dim * 4),
                        range_of(ddelta_bias, dim * 4), range_of(dh0, sbytes)};
  const Range ins[] = {range_of(u, ebytes),      range_of(delta, ebytes),
                       range_of(z, ebytes),      range_of(dout, ebytes),
                       range_of(B, bcbytes),     range_of(C, bcbytes),
                       range_of(A, dim * N * 4), range_of(D, dim * 4),
                       range_of(delta_bias, dim * 4), range_of(h0, sbytes),
                       range_of(dlast, sbytes)};
  const int n_outs = (int)(sizeof(outs) / sizeof(outs[0]));
  for (int i = 0; i < n_outs; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return MSSM_ERR_ALIAS;
    for (int j = i + 1; j < n_outs; ++j)
      if (overlap(outs[i], outs[j])) return MSSM_ERR_ALIAS;
  }

  // --- validation done; HIP calls from here on ---
  const bool vec = !bld && (L % 8) == 0 && ((L * (int64_t)io) % 16) == 0 &&
                   aligned(u, 16) && aligned(delta, 16) && aligned(dout, 16) &&
                   aligned(du, 16) && aligned(ddelta, 16) &&
                   (!z || aligned(z, 16)) && (!dz || aligned(dz, 16));
  const int tile = mssm::bwd_tile();
  const int64_t tiles = (L + tile - 1) / tile;
  int segments = 1;
  int64_t ws_bytes = 0;
  rc = bwd_layout(dims, &segments, &ws_bytes);
  if (rc != MSSM_OK) return rc;
  if (!allocate) {
    rc = check_workspace(ws_in, ws_in_bytes, ws_bytes);
    if (rc != MSSM_OK) return rc;
  }
  mssm::BwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.u = u; p.delta = delta; p.z = z; p.dout = dout; p.A = A; p.B = B; p.C = C;
  p.D = D; p.bias = delta_bias; p.h0 = h0; p.dlast = dlast;
  p.du = du; p.ddelta = ddelta; p.dz = dz; p.dA = dA; p.dB = dB; p.dC = dC;
  p.dD = dD; p.dbias = ddelta_bias; p.dh0 = dh0;
  p.batch = batch; p.dim = dim; p.L = L;
  p.softplus = softplus ? 1 : 0;
  p.groups_per_batch = (int32_t)gpb;
  p.ngroups = (int32_t)G;
  p.tiles = (int32_t)tiles;
  p.segments = segments;
  p.seg_tiles = (int32_t)((tiles + segments - 1) / segments);
  p.layout_bld = bld ? 1 : 0;
  p.bc_state_major = (dims->flags & MSSM_FLAG_BC_STATE_MAJOR) ? 1 : 0;
  p.ev_start = g_ev_start;
  p.ev_stop = g_ev_stop;

  hipStream_t st = (hipStream_t)stream;
  void* ws = ws_in;
  if (allocate) {
    hipError_t e = hipMallocAsync(&ws, (size_t)ws_bytes, st);
    if (e != hipSuccess) {
      set_hip_error("hipMallocAsync(workspace)", e);
      return MSSM_ERR_HIP;
    }
  }
  mssm::bwd_workspace(batch, dim, L, (int)N, io == 2, segments, G, ws, &p);
  hipError_t e = mssm::launch_scan_bwd(p, (int)N, io == 2, vec, st);
  if (e != hipSuccess) set_hip_error("backward scan launch", e);
  if (allocate) {
    hipError_t f = hipFreeAsync(ws, st);
    if (e == hipSuccess && f != hipSuccess) {
      set_hip_error("hipFreeAsync(workspace)", f);
      e = f;
    }
  }
  return e == hipSuccess ? MSSM_OK : MSSM_ERR_HIP;
}

}  // namespace

extern "C" {

int mssm_selective_scan_bwd(const void* u, const void* delta, const float* A,
                            const void* B, const void* C, const float* D,
                            const void* z, const float* delta_bias,
                            int softplus, const float* h0, const void* dout,
                            const float* dlast, void* du, void* ddelta,
                            float* dA, float* dB, float* dC, float* dD,
                            void* dz, float* ddelta_bias, float* dh0,
                            const mssm_dims* dims, void* stream) {
  return scan_bwd_entry(u, delta, A, B, C, D, z, delta_bias, softplus, h0, dout, dlast,
                        du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, nullptr, 0,
                        true, dims, stream);
}

int mssm_selective_scan_bwd_ws(const void* u, const void* delta, const float* A,
                               const void* B, const void* C, const float* D,
                               const void* z, const float* delta_bias,
                               int softplus, const float* h0, const void* dout,
                               const float* dlast, void* du, void* ddelta,
                               float* dA, float* dB, float* dC, float* dD,
                               void* dz, float* ddelta_bias, float* dh0,
                               void* workspace, int64_t workspace_bytes,
                               const mssm_dims* dims, void* stream) {
  return scan_bwd_entry(u, delta, A, B, C, D, z, delta_bias, softplus, h0, dout, dlast,
                        du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, workspace,
                        workspace_bytes, false, dims, stream);
}

int mssm_selective_state_update(float* state, const void* x, const void* dt,
                                const float* A, const void* B, const void* C,
                                const float* D, const void* z,
                                const float* dt_bias, int softplus, void* out,
                                const mssm_dims* dims, void* stream) {
  int rc = check_common_dims(dims);
  if (rc != MSSM_OK) return rc;
  if (dims->flags & ~MSSM_FLAG_STATE_STREAM) return MSSM_ERR_UNSUPPORTED;
  if (dims->seqlen != 1 || dims->time_segments != 0) return MSSM_ERR_DIMS;
  if (!state || !x || !dt || !A || !B || !C || !out) return MSSM_ERR_NULL;
  const int64_t batch = dims->batch, dim = dims->dim, N = dims->dstate;
  const size_t io = dims->io_dtype == MSSM_BF16 ? 2 : 4;
  if (!product_ok(batch, dim, N, INT64_MAX / 16)) return MSSM_ERR_DIMS;
  const int64_t G = groups_of(dims);
  if (dim % G != 0) return MSSM_ERR_DIMS;

  const void* ios[] = {x, dt, B, C, out, z};
  for (const void* p : ios)
    if (p && !aligned(p, io)) return MSSM_ERR_ALIGN;
  const void* f32s[] = {state, A, D, dt_bias};
  for (const void* p : f32s)
    if (p && !aligned(p, 4)) return MSSM_ERR_ALIGN;

  const int64_t rb = batch * dim * (int64_t)io;
  const Range r_out = range_of(out, rb);
  const Range r_state = range_of(state, batch * dim * N * 4);
  const Range ins[] = {range_of(x, rb), range_of(dt, rb), range_of(z, rb),
                       range_of(B, batch * G * N * (int64_t)io),
                       range_of(C, batch * G * N * (int64_t)io),
                       range_of(A, dim * N * 4), range_of(D, dim * 4),
                       range_of(dt_bias, dim * 4)};
  for (const Range& r : ins)
    if (overlap(r_out, r) || overlap(r_state, r)) return MSSM_ERR_ALIAS;
  if (overlap(r_out, r_state)) return MSSM_ERR_ALIAS;

  mssm::UpdateParams p;
  p.state = state; p.x = x; p.dt = dt; p.z = z; p.A = A; p.B = B; p.C = C;
  p.D = D; p.bias = dt_bias; p.out = out;
  p.batch = batch; p.dim = dim; p.softplus = softplus ? 1 : 0;
  p.ngroups = (int32_t)G;
  p.stream_state = (dims->flags & MSSM_FLAG_STATE_STREAM) ? 1 : 0;
  hipError_t e = mssm::launch_state_update(p, (int)N, io == 2,
                                           (hipStream_t)stream);
  if (e != hipSuccess) {
    set_hip_error("state_update launch", e);
    return MSSM_ERR_HIP;
  }
  return MSSM_OK;
}

}  // extern "C"

namespace {

int mamba2_entry(const void* x, const void* dt, const float* A, const void* B,
                 const void* C, const float* D, const void* z,
                 const float* dt_bias, int softplus, int64_t headdim, void* out,
                 float* last_state, void* ws_in, int64_t ws_in_bytes, bool allocate,
                 const mssm_dims* dims, void* stream) {
  if (!dims) return MSSM_ERR_NULL;
  if (dims->io_dtype != MSSM_BF16) return MSSM_ERR_UNSUPPORTED;
  if (dims->flags & ~MSSM_FLAG_LOAD_STATE) return MSSM_ERR_UNSUPPORTED;
  if (dims->batch <= 0 || dims->dim <= 0 || dims->seqlen <= 0 || dims->dstate <= 0 ||
      dims->ngroups < 0 || dims->time_segments < 0 || headdim <= 0)
    return MSSM_ERR_DIMS;
  if (dims->dstate != 64 && dims->dstate != 128) return MSSM_ERR_UNSUPPORTED;
  if (headdim != mssm::mamba2_headdim()) return MSSM_ERR_UNSUPPORTED;
  if (dims->dim % headdim != 0) return MSSM_ERR_DIMS;
  const int64_t batch = dims->batch, dim = dims->dim, N = dims->dstate,
                L = dims->seqlen;
  const int64_t H = dim / headdim;
  const int64_t G = groups_of(dims);
  if (H % G != 0) return MSSM_ERR_UNSUPPORTED;
  const bool load_state = (dims->flags & MSSM_FLAG_LOAD_STATE) != 0;
  if (!x || !dt || !A || !B || !C || !out) return MSSM_ERR_NULL;
  if (load_state && !last_state) return MSSM_ERR_NULL;
  const int64_t lim = INT64_MAX / 16;
  if (batch * H > INT32_MAX || !product_ok(batch, dim, L, lim) ||
      !product_ok(batch, L, G * N, lim) || !product_ok(batch, dim, N, lim))
    return MSSM_ERR_DIMS;
  // the kernel indexes one (batch, head)'s rows with 32-bit offsets
  if (L * dim >= (int64_t(1) << 31) || L * G * N >= (int64_t(1) << 31)) return MSSM_ERR_DIMS;

  // x, z, out and B, C rows are read and written in 16-byte pieces
  const void* vecs[] = {x, B, C, out, z};
  for (const void* p : vecs)
    if (p && !aligned(p, 16)) return MSSM_ERR_ALIGN;
  if (!aligned(dt, 2)) return MSSM_ERR_ALIGN;
  const void* f32s[] = {A, D, dt_bias, last_state};
  for (const void* p : f32s)
    if (p && !aligned(p, 4)) return MSSM_ERR_ALIGN;

  const int64_t ebytes = batch * L * dim * 2;
  const Range r_out = range_of(out, ebytes);
  const Range r_state = range_of(last_state, batch * dim * N * 4);
  const Range ins[] = {range_of(x, ebytes),         range_of(z, ebytes),
                       range_of(dt, batch * L * H * 2),
                       range_of(B, batch * L * G * N * 2),
                       range_of(C, batch * L * G * N * 2),
                       range_of(A, H * 4),          range_of(D, H * 4),
                       range_of(dt_bias, H * 4)};
  for (const Range& r : ins)
    if (overlap(r_out, r) || overlap(r_state, r)) return MSSM_ERR_ALIAS;
  if (overlap(r_out, r_state)) return MSSM_ERR_ALIAS;

  // --- validation done; HIP calls from here on ---
  refresh_cu_count();
  mssm::Mamba2Params p;
  std::memset(&p, 0, sizeof(p));
  p.x = x; p.dt = dt; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z; p.bias = dt_bias;
  p.out = out; p.state = last_state;
  p.batch = batch; p.L = L; p.nheads = H; p.ngroups = G; p.N = N;
  p.softplus = softplus ? 1 : 0;
  p.load_state = load_state ? 1 : 0;
  mssm::mamba2_plan(batch * H, L, g_cu_count > 0 ? g_cu_count : kDefaultCUs,
                    dims->time_segments, &p);
  hipStream_t st = (hipStream_t)stream;
  const int64_t ws_bytes = mssm::mamba2_workspace(p, nullptr, nullptr);
  if (!allocate) {
    const int rc = check_workspace(ws_in, ws_in_bytes, ws_bytes);
    if (rc != MSSM_OK) return rc;
  }
  void* ws = nullptr;
  hipError_t e = hipSuccess;
  if (ws_bytes > 0) {
    if (allocate) {
      e = hipMallocAsync(&ws, (size_t)ws_bytes, st);
      if (e != hipSuccess) {
        set_hip_error("hipMallocAsync(workspace)", e);
        return MSSM_ERR_HIP;
      }
    } else {
      ws = ws_in;
    }
    mssm::mamba2_workspace(p, ws, &p);
  }
  if (g_ev_start) e = hipEventRecord((hipEvent_t)g_ev_start, st);
  if (e == hipSuccess) e = mssm::launch_mamba2_scan(p, st);
  if (e == hipSuccess && g_ev_stop) e = hipEventRecord((hipEvent_t)g_ev_stop, st);
  if (e != hipSuccess) set_hip_error("mamba2 scan launch", e);
  if (allocate && ws) {
    const hipError_t f = hipFreeAsync(ws, st);
    if (e == hipSuccess && f != hipSuccess) {
      set_hip_error("hipFreeAsync(workspace)", f);
      e = f;
    }
  }
  return e == hipSuccess ? MSSM_OK : MSSM_ERR_HIP;
}

// The Mamba-2 scan's time split and workspace for dims (HIP call: the CU count).
int64_t mamba2_ws_bytes(const mssm_dims* dims, int64_t headdim) {
  refresh_cu_count();
  mssm::Mamba2Params p;
  std::memset(&p, 0, sizeof(p));
  p.batch = dims->batch;
  p.L = dims->seqlen;
  p.nheads = dims->dim / headdim;
  p.N = dims->dstate;
  mssm::mamba2_plan(p.batch * p.nheads, p.L, g_cu_count > 0 ? g_cu_count : kDefaultCUs,
                    dims->time_segments, &p);
  return mssm::mamba2_workspace(p, nullptr, nullptr);
}

}  // namespace

extern "C" {

int mssm_mamba2_scan_fwd(const void* x, const void* dt, const float* A, const void* B,
                         const void* C, const float* D, const void* z,
                         const float* dt_bias, int softplus, int64_t headdim, void* out,
                         float* last_state, const mssm_dims* dims, void* stream) {
  return mamba2_entry(x, dt, A, B, C, D, z, dt_bias, softplus, headdim, out, last_state,
                      nullptr, 0, true, dims, stream);
}

int mssm_mamba2_scan_fwd_ws(const void* x, const void* dt, const float* A, const void* B,
                            const void* C, const float* D, const void* z,
                            const float* dt_bias, int softplus, int64_t headdim, void* out,
                            float* last_state, void* workspace, int64_t workspace_bytes,
                            const mssm_dims* dims, void* stream) {
  return mamba2_entry(x, dt, A, B, C, D, z, dt_bias, softplus, headdim, out, last_state,
                      workspace, workspace_bytes, false, dims, stream);
}

int mssm_workspace_size(int op, const mssm_dims* dims, int64_t headdim, int64_t* bytes) {
  if (!bytes) return MSSM_ERR_NULL;
  *bytes = 0;
  int rc = MSSM_OK;
  switch (op) {
    case MSSM_OP_SCAN_FWD:
    case MSSM_OP_SCAN_FWD_CONV: {
      mssm_plan plan;
      refresh_cu_count();
      rc = mssm_selective_scan_fwd_plan(dims, &plan);
      if (rc == MSSM_OK) *bytes = plan.workspace_bytes;
      return rc;
    }
    case MSSM_OP_SCAN_BWD: {
      rc = check_common_dims(dims);
      if (rc != MSSM_OK) return rc;
      if (dims->dstate > 32 || (dims->flags & ~(MSSM_FLAG_LAYOUT_BLD | MSSM_FLAG_BC_STATE_MAJOR)))
        return MSSM_ERR_UNSUPPORTED;
      rc = check_scan_groups(dims);
      if (rc != MSSM_OK) return rc;
      if (dims->time_segments < 0) return MSSM_ERR_DIMS;
      int seg = 1;
      int64_t ws = 0;
      rc = bwd_layout(dims, &seg, &ws);
      if (rc == MSSM_OK) *bytes = ws;
      return rc;
    }
    case MSSM_OP_MAMBA2_FWD: {
      if (!dims) return MSSM_ERR_NULL;
      if (dims->batch <= 0 || dims->dim <= 0 || dims->seqlen <= 0 || dims->time_segments < 0 ||
          headdim <= 0 || dims->dim % headdim != 0)
        return MSSM_ERR_DIMS;
      if (dims->dstate != 64 && dims->dstate != 128) return MSSM_ERR_UNSUPPORTED;
      *bytes = mamba2_ws_bytes(dims, headdim);
      return MSSM_OK;
    }
    default:
      return MSSM_ERR_UNSUPPORTED;
  }
}

}  // extern "C"
