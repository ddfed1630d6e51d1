/*
 * mssm.h -- C ABI of libmssm, the gfx950 (MI355X) selective scan library.
 *
 * The library computes the selective state space recurrence of Mamba:
 *   - continuous model h'(t) = A h(t) + B x(t), y(t) = C h(t) + D x(t)
 *     (page "Mamba: Selective State Space Models", section "Mathematical
 *     Foundation / State Space Model");
 *   - B, C and the step Delta taken per token, Delta = tau_Delta(parameter +
 *     projection) with tau_Delta = softplus and the parameter a per-channel
 *     bias (same page, "Mathematical Foundation / Selective Mechanism");
 *   - Delta as the discretisation step (same page, "Architecture"), read as
 *     zero-order hold on A and an Euler step on B:
 *         h_t[n] = exp(Delta_t A[d,n]) h_{t-1}[n] + Delta_t B_t[n] u_t
 *         y_t    = sum_n C_t[n] h_t[n] + D[d] u_t
 *         out_t  = y_t * silu(z_t)          (the gated block, same page,
 *                                           "Features")
 *   - the forward scan over a whole sequence, and the single-token step that
 *     inference repeats with a fixed-size state (same page, "Mathematical
 *     Foundation / Efficient Scan"; the exported low-level scan op of page
 *     "Mamba State Space Model", "Use selective scan operations").
 *
 * Every (batch, channel) row is an independent recurrence.  A, D and the
 * delta bias are fp32, and so is the recurrent state.  The activations use
 * the io dtype (fp32 or bf16), which keeps parameters in fp32 as page "Mamba
 * State Space Model", "Troubleshoot model instability with precision
 * settings", recommends.
 *
 * Memory and ownership.  Every array pointer is a DEVICE pointer owned by the
 * caller.  All arrays are contiguous, row-major, last index fastest:
 *   u, delta, z, out   (batch, dim, seqlen)      io dtype
 *   B, C               (batch, seqlen, dstate)   io dtype, one N-vector/token
 *                      (batch, seqlen, g, dstate) with mssm_dims.ngroups = g
 *                      (batch, [g,] dstate, seqlen) with MSSM_FLAG_BC_STATE_MAJOR
 *   A                  (dim, dstate)             fp32 (real; negative for a
 *                                                 decaying state)
 *   D, delta_bias      (dim)                     fp32
 *   last_state         (batch, dim, dstate)      fp32
 * Each pointer must be aligned to its element size; 16-byte alignment of every
 * io pointer together with seqlen * sizeof(io) % 16 == 0 selects the
 * vector-load path, anything else the element-load path (same results).
 * The calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 * stream).  They never synchronise the host.
 *
 * Workspace.  The forward scans, the backward and the Mamba-2 scan need
 * device scratch memory (B and C repacked per wave, and the summaries of rows
 * split in time).  Each comes in two forms:
 *   - the *_ws call takes it from the caller (`workspace`, at least
 *     mssm_workspace_size() bytes, 256-byte aligned, owned by the caller and
 *     not touched by any other work until the call's kernels have finished on
 *     `stream`); these calls allocate, free and synchronise nothing;
 *   - the plain call takes it stream-ordered from HIP's default memory pool
 *     (hipMallocAsync / hipFreeAsync on `stream`) for the duration of the
 *     call.
 * Every launch of a call is on `stream`; the library creates no stream and
 * records no event of its own.
 *
 * Errors.  Every argument is validated before the first HIP call; a call that
 * fails validation returns a negative code and writes nothing.  A failing HIP
 * call returns MSSM_ERR_HIP; its message is kept per thread and returned by
 * mssm_last_error().  Non-finite inputs are not detected; they propagate
 * through the arithmetic.
 */
#ifndef MSSM_H
#define MSSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSSM_ABI_VERSION 2

typedef enum { MSSM_F32 = 0, MSSM_BF16 = 1 } mssm_dtype;

enum {
  MSSM_OK = 0,
  MSSM_ERR_NULL = -1,        /* a required pointer (or dims) is NULL        */
  MSSM_ERR_DIMS = -2,        /* a size <= 0, decode seqlen != 1, overflow   */
  MSSM_ERR_UNSUPPORTED = -3, /* dstate not in {1,2,4,...,128} (backward: up  */
                             /* to 32), unknown dtype, unknown flag          */
  MSSM_ERR_ALIGN = -4,       /* pointer not aligned to its element size     */
  MSSM_ERR_ALIAS = -5,       /* an output overlaps another argument         */
  MSSM_ERR_HIP = -6,         /* a HIP runtime call or launch failed         */
  MSSM_ERR_WORKSPACE = -7    /* workspace missing, too small or misaligned  */
                             /* (or, for the allocation-free call, larger    */
                             /* than the library's fixed scratch)            */
};

/* fwd: last_state holds the initial state h0 on entry (in/out). */
#define MSSM_FLAG_LOAD_STATE 1u
/* The per-element arrays (u/x, delta, z, out, u_out; dout, du, ddelta, dz)
 * are (batch, seqlen, dim) -- the block layout (batch, length, dim) of page
 * "Mamba: Selective State Space Models", "Quick Start" -- instead of
 * (batch, dim, seqlen).  B and C keep (batch, seqlen, dstate).  Accepted by
 * the forward scans, the backward and the causal conv. */
#define MSSM_FLAG_LAYOUT_BLD 2u
/* B and C are (batch, dstate, seqlen), (batch, g, dstate, seqlen) with
 * ngroups = g -- each state's values over time contiguous, the layout of the
 * exported low-level scan op (page "Mamba State Space Model", "Use selective
 * scan operations") -- instead of (batch, seqlen, dstate).  The backward
 * writes dB and dC in the same layout.  Accepted by the forward scans and the
 * backward; the results do not depend on the layout. */
#define MSSM_FLAG_BC_STATE_MAJOR 4u
/* Decode step only: the state is read and written with non-temporal
 * (streaming) hints.  For callers whose states do not stay in the GPU's
 * caches from one step to the next -- many layers, or more sequences than
 * the caches hold -- this keeps the state traffic from evicting other data
 * and streams it at a higher rate.  A state that is reused from the cache
 * (one layer's state, resident in the 256 MB Infinity Cache) is faster
 * without it.  The results do not depend on it. */
#define MSSM_FLAG_STATE_STREAM 8u

typedef struct {
  int64_t batch;       /* >= 1                                              */
  int64_t dim;         /* channels (D_inner), >= 1                          */
  int64_t dstate;      /* N, a power of two from 1 to 128 (backward: <= 32) */
  int64_t seqlen;      /* L >= 1 for the scan (at most 2^31 - 65); must be */
                       /* 1 for state_update                               */
  int32_t io_dtype;    /* mssm_dtype of u/delta/z/B/C/out (x/dt/z/B/C/out) */
  uint32_t flags;      /* MSSM_FLAG_*                                       */
  int32_t time_segments; /* scan only: 0 = the library picks; k >= 1 splits */
                         /* every row into k time segments (a carried state */
                         /* joins them; results agree up to rounding)       */
  int32_t ngroups;       /* B/C groups: 0 or 1 = one N-vector per token,     */
                         /* shared by all channels; g > 1: B, C hold g      */
                         /* vectors per token, (batch, seqlen, g, dstate)   */
                         /* ((batch, g, dstate) for state_update), and      */
                         /* channel d reads group d / (dim / g).  The scans */
                         /* need dim % (64 g) == 0 (a 64-channel workgroup  */
                         /* reads one group), state_update dim % g == 0.    */
} mssm_dims;

/*
 * Forward selective scan (the recurrence above over t = 0..seqlen-1).
 *   u, delta    : inputs; delta is the raw step before bias and softplus
 *   A           : (dim, dstate) fp32
 *   B, C        : (batch, seqlen, dstate) io dtype
 *   D           : (dim) fp32 skip weight, or NULL for no skip term
 *   z           : (batch, dim, seqlen) gate input, or NULL for no gate
 *   delta_bias  : (dim) fp32, added to delta BEFORE the softplus; NULL = 0
 *   softplus    : nonzero applies softplus to delta + bias
 *   out         : (batch, dim, seqlen) io dtype, must not overlap any input
 *   last_state  : (batch, dim, dstate) fp32 final state h_{L-1}, or NULL.
 *                 With MSSM_FLAG_LOAD_STATE it is read first as h0 (required).
 *                 Chaining calls with LOAD_STATE over consecutive pieces of a
 *                 sequence reproduces one call over the whole sequence.
 * Returns MSSM_OK or a negative MSSM_ERR_* code.
 */
int mssm_selective_scan_fwd(const void* u, const void* delta, const float* A,
                            const void* B, const void* C, const float* D,
                            const void* z, const float* delta_bias,
                            int softplus, void* out, float* last_state,
                            const mssm_dims* dims, void* stream);

/*
 * Causal depthwise convolution over time, the Mamba block's local
 * convolution that feeds the scan (width d_conv = 4 on page "Mamba State
 * Space Model", model construction; page "Mamba: Selective State Space
 * Models", "Quick Start"; provided by the causal-conv1d package the pages
 * name).  Per (batch, channel) row:
 *     v_t   = bias[d] + sum_{k=0}^{width-1} weight[d,k] * x_{t-(width-1)+k}
 *     out_t = silu(v_t) if silu, else v_t
 * so weight[d, width-1] multiplies the current step; x at t < 0 comes from
 * `init` or is 0.
 *   x, out  : (batch, dim, seqlen) io dtype; out must not overlap an input
 *   weight  : (dim, width) fp32;  bias : (dim) fp32 or NULL
 *   init    : (batch, dim, width-1) io dtype, x at t = -(width-1) .. -1
 *             (the last inputs of the previous piece of the sequence), or NULL
 *   width   : 2, 3 or 4
 * dims->dstate is ignored; flags may hold MSSM_FLAG_LAYOUT_BLD (x and out
 * then are (batch, seqlen, dim)); time_segments must be 0.
 */
int mssm_causal_conv1d_fwd(const void* x, const float* weight,
                           const float* bias, const void* init, int width,
                           int silu, void* out, const mssm_dims* dims,
                           void* stream);

/*
 * Gradients of mssm_causal_conv1d_fwd for an incoming dout = dLoss/dout:
 * with the scan's backward, whose du is the gradient of the convolution's
 * output, this completes the training step of the conv-fed block (the
 * pages' selective scan trained through its parallel scan, page "Mamba:
 * Selective State Space Models", "Efficient Scan").  Chain rule of the
 * forward definition, with g_t = dout_t * silu'(v_t) (or dout_t), silu'(v)
 * = s (1 + v (1 - s)), s = sigmoid(v):
 *     dx_s       = sum_k weight[d,k] * g_{s+(width-1)-k}  (steps inside the row)
 *     dinit_j    = sum_{k<=j} weight[d,k] * g_{j-k}       (x at t = j-(width-1))
 *     dweight[d,k] = sum over batch and time of g_t * x_{t-(width-1)+k}
 *     dbias[d]   = sum over batch and time of g_t
 *   x, dout, dx : (batch, dim, seqlen) io dtype
 *   weight      : (dim, width) fp32;  bias : (dim) fp32 or NULL
 *   init        : (batch, dim, width-1) io dtype or NULL (zeros), as in the
 *                 forward call
 *   dweight     : (dim, width) fp32, written
 *   dbias       : (dim) fp32, written, or NULL (not computed)
 *   dinit       : (batch, dim, width-1) io dtype, written, or NULL (not
 *                 computed); the gradient of the values before t = 0 (of the
 *                 zeros when init is NULL)
 *   width       : 2, 3 or 4
 * The outputs overwrite (no accumulation), must not overlap an input or each
 * other, and the channel sums are added in a fixed order, so repeated calls
 * give identical bits.  dims->dstate is ignored; flags must be 0 (the
 * (batch, dim, seqlen) layout); time_segments must be 0.  Errors as for the
 * forward call.  Allocates nothing; one launch on `stream`.
 */
int mssm_causal_conv1d_bwd(const void* x, const float* weight, const float* bias,
                           const void* init, int width, int silu, const void* dout,
                           void* dx, float* dweight, float* dbias, void* dinit,
                           const mssm_dims* dims, void* stream);

/*
 * The forward scan fed by the width-4 causal convolution: the scan input is
 * u = silu(conv(x)) as mssm_causal_conv1d_fwd(width = 4, silu = 1) computes
 * it, formed while the scan loads its input (u never goes to memory unless
 * u_out is given).  Arguments as in mssm_selective_scan_fwd, with
 *   x           : (batch, dim, seqlen) io dtype, the convolution input
 *   conv_weight : (dim, 4) fp32 (required);  conv_bias : (dim) fp32 or NULL
 *   conv_init   : (batch, dim, 3) io dtype x before t = 0, or NULL (zeros)
 *   u_out       : (batch, dim, seqlen) io dtype receiving u, or NULL
 */
int mssm_selective_scan_fwd_conv(const void* x, const float* conv_weight,
                                 const float* conv_bias, const void* conv_init,
                                 const void* delta, const float* A,
                                 const void* B, const void* C, const float* D,
                                 const void* z, const float* delta_bias,
                                 int softplus, void* out, float* last_state,
                                 void* u_out, const mssm_dims* dims,
                                 void* stream);

/*
 * Backward of the forward scan: the gradients of
 *     loss = sum(dout * out) + sum(dlast * h_{L-1})
 * with respect to every input, for training through the scan (page "Mamba:
 * Selective State Space Models", "Mathematical Foundation / Efficient Scan",
 * which trains with the parallel scan; and "Comparison with Transformers":
 * training memory linear in the sequence length).  The states h_t are not
 * stored by the forward call: this call rescans the rows, keeps the state at
 * every 16th step in workspace, and recomputes each 16-step tile from it.
 *   u, delta, A, B, C, D, z, delta_bias, softplus : as in the forward call
 *   h0          : (batch, dim, dstate) fp32 initial state, or NULL (zero)
 *   dout        : (batch, dim, seqlen) io dtype, gradient of out (required)
 *   dlast       : (batch, dim, dstate) fp32 gradient of the final state, or
 *                 NULL (zero)
 * Outputs (device memory owned by the caller, fully overwritten):
 *   du, ddelta  : (batch, dim, seqlen) io dtype (ddelta is the gradient of
 *                 the raw delta, through bias and softplus)
 *   dz          : (batch, dim, seqlen) io dtype; required iff z != NULL
 *   dA          : (dim, dstate) fp32, summed over the batch
 *   dB, dC      : (batch, seqlen, dstate) fp32, summed over channels
 *   dD, ddelta_bias : (dim) fp32 or NULL (not written), summed over batch
 *                 and time; written even when D / delta_bias are NULL (the
 *                 gradient at zero)
 *   dh0         : (batch, dim, dstate) fp32 gradient of h0, or NULL
 * dstate is at most 32 here.  No output may overlap an input or another
 * output.  flags may hold MSSM_FLAG_LAYOUT_BLD.
 * time_segments: 0 lets the library cut rows into time segments that run in
 * parallel (joined by a carried state and a carried gradient); k >= 1 asks
 * for about k segments (whole 16-step tiles each).  Results agree up to
 * rounding.  The sums over channels and the batch are taken
 * in a fixed order, so repeated calls give identical bits.  Stream-ordered
 * workspace: about 4 * dstate bytes per element of u plus 8 * dstate bytes
 * per token for each 64-channel group, returned on the same stream.
 */
int mssm_selective_scan_bwd(const void* u, const void* delta, const float* A,
                            const void* B, const void* C, const float* D,
                            const void* z, const float* delta_bias,
                            int softplus, const float* h0, const void* dout,
                            const float* dlast, void* du, void* ddelta,
                            float* dA, float* dB, float* dC, float* dD,
                            void* dz, float* ddelta_bias, float* dh0,
                            const mssm_dims* dims, void* stream);

/*
 * The Mamba-2 block's scan (page "Mamba State Space Model", "Use the Mamba2
 * block": the Mamba-2 architecture, state sizes of typically 64 or 128).  The pages give the block's API, not its scan; this is the
 * Mamba-2 architecture's: the selective recurrence with one A, one step and
 * one D per head of `headdim` channels, and B, C shared by a group of heads.
 * For channel p of head h (channel index d = h * headdim + p), head group
 * g = h / (nheads / ngroups), state n:
 *     Delta_t = softplus(dt_t[h] + dt_bias[h])   (or without softplus)
 *     h_t[d,n] = exp(Delta_t A[h]) h_{t-1}[d,n] + Delta_t x_t[d] B_t[g,n]
 *     out_t[d] = (sum_n C_t[g,n] h_t[d,n] + D[h] x_t[d]) * silu(z_t[d])
 * with nheads = dims->dim / headdim.  Layouts (last index fastest):
 *   x, z, out : (batch, seqlen, nheads, headdim) bf16; z may be NULL (no gate)
 *   dt        : (batch, seqlen, nheads) bf16
 *   A, D, dt_bias : (nheads) fp32; D and dt_bias may be NULL (zero)
 *   B, C      : (batch, seqlen, ngroups, dstate) bf16 (ngroups 0 means 1)
 *   last_state: (batch, nheads * headdim, dstate) fp32: the final state, or
 *               NULL; with MSSM_FLAG_LOAD_STATE it holds the initial state
 *               on entry (required then)
 * dims: io_dtype must be MSSM_BF16, dstate 64 or 128, headdim 64, nheads a
 * multiple of ngroups, and seqlen * dim and seqlen * ngroups * dstate below
 * 2^31; flags may hold only MSSM_FLAG_LOAD_STATE.  x, z, out, B and C must
 * be 16-byte aligned.  out and last_state must not overlap an input or each
 * other.  The call runs the chunked matrix form of the recurrence on the
 * matrix cores, one workgroup per (batch entry, head) and time segment;
 * results agree with the sequential recurrence up to rounding.
 * time_segments: 0 lets the library cut the rows of the (batch, head) pairs
 * beyond whole rounds of compute units (all pairs, when there are fewer
 * than compute units) into time segments joined by a carried state; k >= 1
 * cuts every pair into about k segments of whole 64-step chunks (1: none).
 * Segments take a stream-ordered workspace of about 8 * 64 * dstate bytes
 * per segment, returned on the same stream; unsplit calls allocate nothing.
 */
int mssm_mamba2_scan_fwd(const void* x, const void* dt, const float* A, const void* B,
                         const void* C, const float* D, const void* z,
                         const float* dt_bias, int softplus, int64_t headdim, void* out,
                         float* last_state, const mssm_dims* dims, void* stream);

/*
 * Single-token decode step: the scan with seqlen = 1 starting from `state`,
 * which is updated in place.
 *   state       : (batch, dim, dstate) fp32, in/out
 *   x, dt, z    : (batch, dim) io dtype; dt is the raw step; z may be NULL
 *   B, C        : (batch, dstate) io dtype
 *   A           : (dim, dstate) fp32;  D, dt_bias : (dim) fp32 or NULL
 *   out         : (batch, dim) io dtype, must not overlap any input or state
 * dims->seqlen must be 1 and time_segments 0; flags is 0 or
 * MSSM_FLAG_STATE_STREAM.
 */
int mssm_selective_state_update(float* state, const void* x, const void* dt,
                                const float* A, const void* B, const void* C,
                                const float* D, const void* z,
                                const float* dt_bias, int softplus, void* out,
                                const mssm_dims* dims, void* stream);

/* Same as mssm_selective_scan_fwd, with the caller's workspace (see
 * "Workspace" above; workspace_bytes >= mssm_workspace_size(MSSM_OP_SCAN_FWD)).
 * A call that needs no workspace accepts NULL. */
int mssm_selective_scan_fwd_ws(const void* u, const void* delta, const float* A,
                               const void* B, const void* C, const float* D,
                               const void* z, const float* delta_bias, int softplus,
                               void* out, float* last_state, void* workspace,
                               int64_t workspace_bytes, const mssm_dims* dims,
                               void* stream);

/* Same as mssm_selective_scan_fwd_conv, with the caller's workspace
 * (mssm_workspace_size(MSSM_OP_SCAN_FWD_CONV)). */
int mssm_selective_scan_fwd_conv_ws(const void* x, const float* conv_weight,
                                    const float* conv_bias, const void* conv_init,
                                    const void* delta, const float* A, const void* B,
                                    const void* C, const float* D, const void* z,
                                    const float* delta_bias, int softplus, void* out,
                                    float* last_state, void* u_out, void* workspace,
                                    int64_t workspace_bytes, const mssm_dims* dims,
                                    void* stream);

/* Same as mssm_selective_scan_bwd, with the caller's workspace
 * (mssm_workspace_size(MSSM_OP_SCAN_BWD)). */
int mssm_selective_scan_bwd_ws(const void* u, const void* delta, const float* A,
                               const void* B, const void* C, const float* D,
                               const void* z, const float* delta_bias,
                               int softplus, const float* h0, const void* dout,
                               const float* dlast, void* du, void* ddelta,
                               float* dA, float* dB, float* dC, float* dD,
                               void* dz, float* ddelta_bias, float* dh0,
                               void* workspace, int64_t workspace_bytes,
                               const mssm_dims* dims, void* stream);

/* Same as mssm_mamba2_scan_fwd, with the caller's workspace
 * (mssm_workspace_size(MSSM_OP_MAMBA2_FWD, headdim)); NULL when the call
 * needs none. */
int mssm_mamba2_scan_fwd_ws(const void* x, const void* dt, const float* A,
                            const void* B, const void* C, const float* D,
                            const void* z, const float* dt_bias, int softplus,
                            int64_t headdim, void* out, float* last_state,
                            void* workspace, int64_t workspace_bytes,
                            const mssm_dims* dims, void* stream);

/* Operations for mssm_workspace_size. */
enum {
  MSSM_OP_SCAN_FWD = 0,
  MSSM_OP_SCAN_FWD_CONV = 1,
  MSSM_OP_SCAN_BWD = 2,
  MSSM_OP_MAMBA2_FWD = 3
};

/* Workspace bytes (*bytes; 0 when none is needed) of one call of `op` with
 * these dims (and headdim, for MSSM_OP_MAMBA2_FWD; ignored otherwise).  The
 * split of rows in time depends on the current device's compute-unit count
 * (and, for the backward, on its occupancy), so the size is for calls on the
 * device that is current here.  Validates dims like the call itself. */
int mssm_workspace_size(int op, const mssm_dims* dims, int64_t headdim, int64_t* bytes);

/*
 * Allocation-free forward scan, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Arguments, results and errors as in
 * mssm_selective_scan_fwd.  Its workspace is a fixed scratch array of
 * MSSM_NOALLOC_SCRATCH_BYTES per device, built into the library (each device
 * holds its copy until the process ends); a call whose workspace
 * (mssm_workspace_size(MSSM_OP_SCAN_FWD)) is larger returns
 * MSSM_ERR_WORKSPACE and launches nothing.  The call allocates, frees and
 * synchronises nothing.  The first call
 * on a device looks up that device's scratch address (a HIP symbol query);
 * later calls make no such query.  Every call on a device shares that
 * device's scratch: calls that overlap in time on one device (on different
 * streams, or from several threads) race and give wrong results; order them.
 */
#define MSSM_NOALLOC_SCRATCH_BYTES (32ll << 20)
int mssm_selective_scan_fwd_noalloc(const void* u, const void* delta, const float* A,
                                    const void* B, const void* C, const float* D,
                                    const void* z, const float* delta_bias,
                                    int softplus, void* out, float* last_state,
                                    const mssm_dims* dims, void* stream);

/* How the forward scan would run for these dims (no HIP call, no launch). */
typedef struct {
  int32_t groups;           /* 64-channel groups (batch * ceil(dim / 64))     */
  int32_t whole_groups;     /* groups scanned in one piece                   */
  int32_t split_groups;     /* groups split in time                          */
  int32_t segments;         /* time segments of each split group             */
  int64_t segment_len;      /* timesteps per segment (last may be shorter)   */
  int32_t waves_per_group;  /* waves per workgroup (each owns dstate/waves   */
                            /* of the state)                                 */
  int32_t kernels;          /* launches per call: the B/C pack and the scan  */
  int64_t workspace_bytes;  /* workspace a call needs (mssm_workspace_size)  */
  int32_t vector_path;      /* 1 when a vector-load path applies: rows of   */
                            /* (batch, dim, L) with L % 8 == 0 read in       */
                            /* 16-byte pieces (pointers 16-byte aligned), or */
                            /* (batch, L, dim) with dim % 4 == 0 read as 4   */
                            /* channels of a step (pointers aligned to 4     */
                            /* values; not for the conv-fed forward)         */
  int32_t reserved;
} mssm_plan;

int mssm_selective_scan_fwd_plan(const mssm_dims* dims, mssm_plan* plan);

/*
 * Timing hook for benchmarks.  With both handles non-NULL (hipEvent_t, owned
 * by the caller), every later forward scan issued from this thread records
 * `start` on its stream right before its scan kernel (the one launch after
 * the B/C pack) and `stop` right after it, so hipEventElapsedTime(start,
 * stop) is that kernel's duration.  The Mamba-2 scan records them around its
 * launches.
 * The backward call records them around its three main kernels (pass F,
 * the segment combine and pass R).
 * Both NULL turns the hook off; one NULL is MSSM_ERR_NULL.  Per thread.
 */
int mssm_set_scan_timing_events(void* start, void* stop);

/*
 * Issue-rate probe of the vector ALU, for the roofline of the scan, which is
 * bound by its exponentials and fp32 multiply-adds rather than by HBM
 * (page "What are State Space Models (SSMs)?", Key Features: the selective
 * scan's hardware-aware algorithm).  Launches `blocks` workgroups of 256
 * threads on `stream`; each thread runs `iters` iterations of
 *   kind 0: 8 independent fp32 fma (v_fma_f32),
 *   kind 1: 8 independent exponentials (v_exp_f32),
 *   kind 2: 4 state elements of the scan's inner step, each a multiply, an
 *           exponential, a multiply, an fma and a readout fma (the first a
 *           multiply), plus 1 multiply per iteration (21 instructions when
 *           iters is a multiple of 4),
 *   kind 3: the same 4 state elements per iteration computed as an inclusive
 *           associative scan of (exp(Delta A), Delta u B) pairs across the
 *           wave's 64 lanes (one timestep per lane: six DPP levels), then the
 *           chunk's entering state and the readout,
 *   kind 4: 8 independent fp32 fma and 2 independent exponentials (no value
 *           passes between the two kinds), to see whether the exponentials
 *           overlap the fma work,
 * and writes one float per thread to `sink` (device, blocks * 256 floats,
 * caller-owned; the values carry no meaning).  The caller times the launch
 * (for instance with events on `stream`).  Errors: MSSM_ERR_NULL (sink),
 * MSSM_ERR_DIMS (kind outside 0..4, blocks or iters <= 0), MSSM_ERR_HIP.
 */
int mssm_valu_probe(int kind, int blocks, int iters, float* sink, void* stream);

/* Static text for a status code. */
const char* mssm_status_string(int status);

/* Message of the last MSSM_ERR_HIP on this thread ("" if none). */
const char* mssm_last_error(void);

/* MSSM_ABI_VERSION of the loaded library. */
int mssm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSSM_H */
