"""MI355X (gfx950) selective scan: a thin torch binding over libmssm.so.

Every step of the computation runs in the HIP kernels behind the C ABI in
``include/mssm.h``; this module only checks tensors and passes their device
pointers and the current HIP stream.  torch supplies device memory and streams.
There is no CPU fallback: if the library is missing, or a tensor is not on a
GPU, the call raises.

The operation (page "Mamba: Selective State Space Models", "Mathematical
Foundation"; discretisation by the step Delta, "Architecture"):
    Delta_t = softplus(delta_t + delta_bias)
    h_t     = exp(Delta_t A) * h_{t-1} + Delta_t B_t u_t
    out_t   = (C_t . h_t + D u_t) * silu(z_t)
"""
from __future__ import annotations

import torch

import ctypes

from ._lib import (MSSM_BF16, MSSM_F32, MSSM_FLAG_BC_STATE_MAJOR, MSSM_FLAG_LAYOUT_BLD,
                   MSSM_FLAG_LOAD_STATE, MSSM_FLAG_STATE_STREAM,
                   MSSM_OP_MAMBA2_FWD, MSSM_OP_SCAN_BWD, MSSM_OP_SCAN_FWD,
                   MSSM_OP_SCAN_FWD_CONV, Dims, MssmError, Plan, check, lib)

__all__ = ["selective_scan_fwd", "selective_scan_bwd", "selective_scan_fwd_conv",
           "causal_conv1d_fwd", "selective_state_update", "mamba2_scan_fwd", "scan_plan",
           "workspace_size", "set_scan_timing_events", "MssmError", "abi_version"]

_IO = {torch.float32: MSSM_F32, torch.bfloat16: MSSM_BF16}


def abi_version() -> int:
    return lib().mssm_abi_version()


def set_scan_timing_events(start=None, stop=None) -> None:
    """Record two hipEvent_t handles (ints) around the main scan kernel of the
    following forward calls from this thread (None, None turns it off)."""
    check(lib().mssm_set_scan_timing_events(start, stop))


def valu_probe(kind: int, blocks: int, iters: int, sink) -> None:
    """Launch the library's ALU issue-rate probe on the current stream: kind
    0 = fp32 fma, 1 = exp, 2 = the scan's state-element mix, 3 = the same
    recurrence as an in-wave associative scan, 4 = 8 fma and 2 exp on
    independent chains (their overlap); `sink` is a
    float32 device tensor of at least blocks * 256 values."""
    _need(sink, "sink", torch.float32)
    if sink.numel() < blocks * 256:
        raise ValueError("sink holds fewer than blocks * 256 values")
    check(lib().mssm_valu_probe(int(kind), int(blocks), int(iters), _ptr(sink),
                                _stream(sink.device)))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtype=None, shape=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


_LAYOUTS = ("bdl", "bld")


def _layout(layout):
    if layout not in _LAYOUTS:
        raise ValueError("layout must be 'bdl' (batch, dim, L) or 'bld' (batch, L, dim)")
    return MSSM_FLAG_LAYOUT_BLD if layout == "bld" else 0


def _dims_of(t, layout):
    """(batch, dim, L) of a per-element tensor in the given layout."""
    if layout == "bld":
        batch, L, dim = t.shape
    else:
        batch, dim, L = t.shape
    return batch, dim, L


def _eshape(batch, dim, L, layout):
    return (batch, L, dim) if layout == "bld" else (batch, dim, L)


_BC_LAYOUTS = ("token", "state")


def _bc_flag(bc_layout):
    if bc_layout not in _BC_LAYOUTS:
        raise ValueError("bc_layout must be 'token' (batch, L, [G,] N) or "
                         "'state' (batch, [G,] N, L)")
    return MSSM_FLAG_BC_STATE_MAJOR if bc_layout == "state" else 0


def _groups(B, batch, L, N, token_dim=True, bc_layout="token"):
    """B/C group count from B's shape: (batch, L, N) or (batch, L, G, N) for
    the scans (token_dim; (batch, N, L) or (batch, G, N, L) with bc_layout
    'state'), (batch, N) or (batch, G, N) for the decode step."""
    if token_dim:
        if B.dim() != 4:
            return 1
        return B.shape[1] if bc_layout == "state" else B.shape[2]
    return B.shape[1] if B.dim() == 3 else 1


def _bc_shape(batch, L, G, N, grouped, bc_layout="token"):
    if bc_layout == "state":
        return (batch, G, N, L) if grouped else (batch, N, L)
    return (batch, L, G, N) if grouped else (batch, L, N)


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def workspace_size(op, dims, headdim=0) -> int:
    """Workspace bytes of one call (mssm_workspace_size) on the current device."""
    n = ctypes.c_int64(0)
    check(lib().mssm_workspace_size(int(op), dims, int(headdim), ctypes.byref(n)))
    return int(n.value)


# One workspace per (device, stream), grown on demand from torch's caching
# allocator: calls on one stream run in order, so they can share it, and a
# grown buffer's old block returns to torch's pool on that same stream.
_WS = {}


def _workspace(op, dims, dev, stream, headdim=0):
    """(pointer, bytes) of a workspace for this call (None, 0 when none is needed)."""
    need = workspace_size(op, dims, headdim)
    if need <= 0:
        return None, 0
    key = (dev.index if dev.index is not None else torch.cuda.current_device(), stream)
    buf = _WS.get(key)
    if buf is None or buf.numel() < need:
        buf = torch.empty(need + 256, dtype=torch.uint8, device=dev)
        _WS[key] = buf
    ptr = buf.data_ptr()
    ptr += (-ptr) % 256
    return ptr, need


def scan_plan(batch, dim, dstate, seqlen, io_dtype=torch.bfloat16,
              time_segments=0, layout="bdl", ngroups=0) -> dict:
    """How the library splits a forward scan of this shape (no GPU needed)."""
    dims = Dims(batch, dim, dstate, seqlen, _IO[io_dtype], _layout(layout),
                time_segments, ngroups)
    plan = Plan()
    check(lib().mssm_selective_scan_fwd_plan(dims, plan))
    return plan.as_dict()


def selective_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                       softplus=True, last_state=None, load_state=False,
                       out=None, time_segments=0, layout="bdl", bc_layout="token"):
    """Forward selective scan.

    u, delta, z: (batch, dim, L); B, C: (batch, L, N) (bc_layout="state":
    (batch, N, L)), all fp32 or all bf16.
    A: (dim, N) fp32; D, delta_bias: (dim,) fp32 or None.
    last_state: (batch, dim, N) fp32 receiving the final state (and holding
    the initial state when load_state=True), or None.
    Returns out (batch, dim, L) in the io dtype.  layout="bld" takes and
    returns u, delta, z, out as (batch, L, dim).
    """
    if u.dtype not in _IO:
        raise ValueError("u must be float32 or bfloat16")
    io = u.dtype
    lay = _layout(layout)
    batch, dim, L = _dims_of(u, layout)
    es = _eshape(batch, dim, L, layout)
    N = A.shape[-1]
    dev = u.device
    _need(u, "u", io, es, dev)
    _need(delta, "delta", io, es, dev)
    _need(z, "z", io, es, dev)
    G = _groups(B, batch, L, N, bc_layout=bc_layout)
    _need(B, "B", io, _bc_shape(batch, L, G, N, B.dim() == 4, bc_layout), dev)
    _need(C, "C", io, tuple(B.shape), dev)
    _need(A, "A", torch.float32, (dim, N), dev)
    _need(D, "D", torch.float32, (dim,), dev)
    _need(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    _need(last_state, "last_state", torch.float32, (batch, dim, N), dev)
    if load_state and last_state is None:
        raise ValueError("load_state needs last_state")
    if out is None:
        out = torch.empty(es, dtype=io, device=dev)
    _need(out, "out", io, es, dev)
    dims = Dims(batch, dim, N, L, _IO[io],
                (MSSM_FLAG_LOAD_STATE if load_state else 0) | lay | _bc_flag(bc_layout),
                time_segments, G)
    with torch.cuda.device(dev):
        st = _stream(dev)
        ws, nws = _workspace(MSSM_OP_SCAN_FWD, dims, dev, st)
        check(lib().mssm_selective_scan_fwd_ws(
            _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(delta_bias), int(bool(softplus)), _ptr(out), _ptr(last_state),
            ws, nws, dims, st))
    return out


def causal_conv1d_fwd(x, weight, bias=None, init=None, silu=True, out=None,
                      layout="bdl"):
    """Causal depthwise convolution over time: x (batch, dim, L) fp32 or
    bf16, weight (dim, width) fp32 with width 2..4, bias (dim,) fp32 or None,
    init (batch, dim, width-1) in x's dtype (inputs before t = 0) or None.
    Returns silu(conv) (or conv with silu=False) in x's dtype; layout="bld"
    takes x and returns out as (batch, L, dim)."""
    if x.dtype not in _IO:
        raise ValueError("x must be float32 or bfloat16")
    lay = _layout(layout)
    batch, dim, L = _dims_of(x, layout)
    es = _eshape(batch, dim, L, layout)
    width = weight.shape[-1]
    dev = x.device
    _need(x, "x", x.dtype, es, dev)
    _need(weight, "weight", torch.float32, (dim, width), dev)
    _need(bias, "bias", torch.float32, (dim,), dev)
    _need(init, "init", x.dtype, (batch, dim, width - 1), dev)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", x.dtype, es, dev)
    dims = Dims(batch, dim, 0, L, _IO[x.dtype], lay, 0, 0)
    with torch.cuda.device(dev):
        check(lib().mssm_causal_conv1d_fwd(
            _ptr(x), _ptr(weight), _ptr(bias), _ptr(init), int(width),
            int(bool(silu)), _ptr(out), dims, _stream(dev)))
    return out


def causal_conv1d_bwd(x, weight, dout, bias=None, init=None, silu=True, dinit=False):
    """Gradients of causal_conv1d_fwd (same x, weight, bias, init, silu) for
    dout = dLoss/dout, all in the (batch, dim, L) layout.  Returns
    (dx in x's dtype, dweight (dim, width) fp32, dbias (dim,) fp32, dinit)
    where dinit is the (batch, dim, width-1) gradient of the values before
    t = 0 in x's dtype when `dinit` is true, else None."""
    if x.dtype not in _IO:
        raise ValueError("x must be float32 or bfloat16")
    if x.dim() != 3:
        raise ValueError("x must be (batch, dim, L)")
    batch, dim, L = x.shape
    width = weight.shape[-1]
    dev = x.device
    _need(x, "x", x.dtype, (batch, dim, L), dev)
    _need(dout, "dout", x.dtype, (batch, dim, L), dev)
    _need(weight, "weight", torch.float32, (dim, width), dev)
    _need(bias, "bias", torch.float32, (dim,), dev)
    _need(init, "init", x.dtype, (batch, dim, width - 1), dev)
    dx = torch.empty_like(x)
    dw = torch.empty(dim, width, dtype=torch.float32, device=dev)
    db = torch.empty(dim, dtype=torch.float32, device=dev)
    di = torch.empty(batch, dim, width - 1, dtype=x.dtype, device=dev) if dinit else None
    dims = Dims(batch, dim, 0, L, _IO[x.dtype], 0, 0, 0)
    with torch.cuda.device(dev):
        check(lib().mssm_causal_conv1d_bwd(
            _ptr(x), _ptr(weight), _ptr(bias), _ptr(init), int(width), int(bool(silu)),
            _ptr(dout), _ptr(dx), _ptr(dw), _ptr(db), _ptr(di), dims, _stream(dev)))
    return dx, dw, db, di


def selective_scan_fwd_conv(x, conv_weight, delta, A, B, C, conv_bias=None,
                            conv_init=None, D=None, z=None, delta_bias=None,
                            softplus=True, last_state=None, load_state=False,
                            out=None, u_out=None, time_segments=0, layout="bdl",
                            bc_layout="token"):
    """The forward scan whose input is u = silu(causal_conv(x)) (width 4),
    formed inside the scan kernel.  x: (batch, dim, L); conv_weight (dim, 4)
    fp32; conv_bias (dim,) fp32 or None; conv_init (batch, dim, 3) or None;
    the other arguments as in selective_scan_fwd.  u_out, if given, receives
    u.  Returns out."""
    if x.dtype not in _IO:
        raise ValueError("x must be float32 or bfloat16")
    io = x.dtype
    lay = _layout(layout)
    batch, dim, L = _dims_of(x, layout)
    es = _eshape(batch, dim, L, layout)
    N = A.shape[-1]
    dev = x.device
    _need(x, "x", io, es, dev)
    _need(conv_weight, "conv_weight", torch.float32, (dim, 4), dev)
    _need(conv_bias, "conv_bias", torch.float32, (dim,), dev)
    _need(conv_init, "conv_init", io, (batch, dim, 3), dev)
    _need(u_out, "u_out", io, es, dev)
    _need(delta, "delta", io, es, dev)
    _need(z, "z", io, es, dev)
    G = _groups(B, batch, L, N, bc_layout=bc_layout)
    _need(B, "B", io, _bc_shape(batch, L, G, N, B.dim() == 4, bc_layout), dev)
    _need(C, "C", io, tuple(B.shape), dev)
    _need(A, "A", torch.float32, (dim, N), dev)
    _need(D, "D", torch.float32, (dim,), dev)
    _need(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    _need(last_state, "last_state", torch.float32, (batch, dim, N), dev)
    if load_state and last_state is None:
        raise ValueError("load_state needs last_state")
    if out is None:
        out = torch.empty(es, dtype=io, device=dev)
    _need(out, "out", io, es, dev)
    dims = Dims(batch, dim, N, L, _IO[io],
                (MSSM_FLAG_LOAD_STATE if load_state else 0) | lay | _bc_flag(bc_layout),
                time_segments, G)
    with torch.cuda.device(dev):
        st = _stream(dev)
        ws, nws = _workspace(MSSM_OP_SCAN_FWD_CONV, dims, dev, st)
        check(lib().mssm_selective_scan_fwd_conv_ws(
            _ptr(x), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_init),
            _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(delta_bias), int(bool(softplus)), _ptr(out), _ptr(last_state),
            _ptr(u_out), ws, nws, dims, st))
    return out


def selective_scan_bwd(u, delta, A, B, C, dout, D=None, z=None,
                       delta_bias=None, softplus=True, h0=None, dlast=None,
                       want_dh0=False, time_segments=0, layout="bdl", bc_layout="token"):
    """Gradients of the forward scan for the loss
    sum(dout * out) + sum(dlast * last_state).

    Inputs as in selective_scan_fwd; h0 (batch, dim, N) fp32 is the initial
    state (None = zero), dout (batch, dim, L) in the io dtype, dlast
    (batch, dim, N) fp32 or None.  Returns a dict: du, ddelta, dz (io dtype,
    dz only with z), dA (dim, N), dB, dC (shaped as B), dD, ddelta_bias (dim,)
    and, with want_dh0, dh0 (batch, dim, N), all fp32 except the first three.
    time_segments: 0 = the library's split of rows into parallel time
    segments; k >= 1 asks for about k.
    """
    if u.dtype not in _IO:
        raise ValueError("u must be float32 or bfloat16")
    io = u.dtype
    lay = _layout(layout)
    batch, dim, L = _dims_of(u, layout)
    es = _eshape(batch, dim, L, layout)
    N = A.shape[-1]
    dev = u.device
    _need(u, "u", io, es, dev)
    _need(delta, "delta", io, es, dev)
    _need(z, "z", io, es, dev)
    _need(dout, "dout", io, es, dev)
    G = _groups(B, batch, L, N, bc_layout=bc_layout)
    _need(B, "B", io, _bc_shape(batch, L, G, N, B.dim() == 4, bc_layout), dev)
    _need(C, "C", io, tuple(B.shape), dev)
    _need(A, "A", torch.float32, (dim, N), dev)
    _need(D, "D", torch.float32, (dim,), dev)
    _need(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    _need(h0, "h0", torch.float32, (batch, dim, N), dev)
    _need(dlast, "dlast", torch.float32, (batch, dim, N), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(du=torch.empty(es, dtype=io, device=dev),
             ddelta=torch.empty(es, dtype=io, device=dev),
             dz=torch.empty(es, dtype=io, device=dev) if z is not None else None,
             dA=torch.empty((dim, N), **f32),
             dB=torch.empty(tuple(B.shape), **f32),
             dC=torch.empty(tuple(B.shape), **f32),
             dD=torch.empty((dim,), **f32),
             ddelta_bias=torch.empty((dim,), **f32),
             dh0=torch.empty((batch, dim, N), **f32) if want_dh0 else None)
    dims = Dims(batch, dim, N, L, _IO[io], lay | _bc_flag(bc_layout), time_segments, G)
    with torch.cuda.device(dev):
        st = _stream(dev)
        ws, nws = _workspace(MSSM_OP_SCAN_BWD, dims, dev, st)
        check(lib().mssm_selective_scan_bwd_ws(
            _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(delta_bias), int(bool(softplus)), _ptr(h0), _ptr(dout),
            _ptr(dlast), _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]),
            _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]),
            _ptr(g["ddelta_bias"]), _ptr(g["dh0"]), ws, nws, dims, st))
    return g


def selective_state_update(state, x, dt, A, B, C, D=None, z=None, dt_bias=None,
                           softplus=True, out=None, stream_state=False):
    """Single-token decode step; `state` (batch, dim, N) fp32 is updated in place.

    x, dt, z: (batch, dim); B, C: (batch, N), all fp32 or all bf16.
    stream_state: read and write the state with non-temporal hints
    (MSSM_FLAG_STATE_STREAM), for states that do not stay in the GPU's caches
    between steps; same results.
    Returns out (batch, dim) in the io dtype.
    """
    if x.dtype not in _IO:
        raise ValueError("x must be float32 or bfloat16")
    io = x.dtype
    batch, dim, N = state.shape
    dev = x.device
    _need(state, "state", torch.float32, (batch, dim, N), dev)
    _need(x, "x", io, (batch, dim), dev)
    _need(dt, "dt", io, (batch, dim), dev)
    _need(z, "z", io, (batch, dim), dev)
    G = _groups(B, batch, 1, N, token_dim=False)
    _need(B, "B", io, (batch, G, N) if B.dim() == 3 else (batch, N), dev)
    _need(C, "C", io, tuple(B.shape), dev)
    _need(A, "A", torch.float32, (dim, N), dev)
    _need(D, "D", torch.float32, (dim,), dev)
    _need(dt_bias, "dt_bias", torch.float32, (dim,), dev)
    if out is None:
        out = torch.empty((batch, dim), dtype=io, device=dev)
    _need(out, "out", io, (batch, dim), dev)
    dims = Dims(batch, dim, N, 1, _IO[io], MSSM_FLAG_STATE_STREAM if stream_state else 0, 0, G)
    with torch.cuda.device(dev):
        check(lib().mssm_selective_state_update(
            _ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
            _ptr(z), _ptr(dt_bias), int(bool(softplus)), _ptr(out), dims,
            _stream(dev)))
    return out


def mamba2_scan_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, softplus=True,
                    last_state=None, load_state=False, out=None, time_segments=0):
    """The Mamba-2 block's scan (mssm_mamba2_scan_fwd), bf16 activations.

    x, z: (batch, L, nheads, headdim) with headdim 64; dt: (batch, L, nheads);
    A, D, dt_bias: (nheads,) fp32; B, C: (batch, L, ngroups, N) with N 64 or
    128; last_state: (batch, nheads * headdim, N) fp32 receiving the final
    state (holding the initial one when load_state).  time_segments: 0 lets
    the library cut rows in time to fill the GPU, k >= 1 asks for k segments.
    Returns out, shaped as x.
    """
    if x.dim() != 4 or x.dtype != torch.bfloat16:
        raise ValueError("x must be a (batch, L, nheads, headdim) bfloat16 tensor")
    batch, L, H, P = x.shape
    dev = x.device
    if B.dim() != 4:
        raise ValueError("B must be (batch, L, ngroups, N)")
    G, N = B.shape[2], B.shape[3]
    _need(x, "x", torch.bfloat16, (batch, L, H, P), dev)
    _need(z, "z", torch.bfloat16, (batch, L, H, P), dev)
    _need(dt, "dt", torch.bfloat16, (batch, L, H), dev)
    _need(B, "B", torch.bfloat16, (batch, L, G, N), dev)
    _need(C, "C", torch.bfloat16, (batch, L, G, N), dev)
    _need(A, "A", torch.float32, (H,), dev)
    _need(D, "D", torch.float32, (H,), dev)
    _need(dt_bias, "dt_bias", torch.float32, (H,), dev)
    _need(last_state, "last_state", torch.float32, (batch, H * P, N), dev)
    if load_state and last_state is None:
        raise ValueError("load_state needs last_state")
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", torch.bfloat16, (batch, L, H, P), dev)
    dims = Dims(batch, H * P, N, L, _IO[torch.bfloat16], 1 if load_state else 0,
                int(time_segments), G)
    with torch.cuda.device(dev):
        st = _stream(dev)
        ws, nws = _workspace(MSSM_OP_MAMBA2_FWD, dims, dev, st, headdim=P)
        check(lib().mssm_mamba2_scan_fwd_ws(
            _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(dt_bias), int(bool(softplus)), P, _ptr(out), _ptr(last_state),
            ws, nws, dims, st))
    return out
