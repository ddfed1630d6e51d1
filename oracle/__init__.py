"""fp64 CPU oracle for the selective scan and the single-token decode step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``selective_state_space_52_amd``) never imports it and shares no code with it.

The arithmetic lives in ``mssm_oracle.c`` (plain C, fp64, sequential in time);
this module only compiles it with gcc and marshals numpy arrays through ctypes.
What the C code computes, and which passage of the pages each step follows, is
written at the top of that file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "mssm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmssm_oracle.so")
_D = ctypes.POINTER(ctypes.c_double)


def compile_source(src: str, out_path: str) -> str:
    """Compile an oracle C source with gcc (no fast-math, no FMA contraction)."""
    tmp = out_path + ".tmp"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-shared", "-fPIC", "-std=c99", src, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, out_path)
    return out_path


def build(force: bool = True) -> str:
    """Compile oracle/mssm_oracle.c into oracle/libmssm_oracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        compile_source(SOURCE, _LIB_PATH)
    return _LIB_PATH


def _open(path):
    lib = ctypes.CDLL(path)
    i64, cint = ctypes.c_int64, ctypes.c_int
    lib.mssm_oracle_scan.argtypes = [i64, i64, i64, i64, i64, _D, _D, _D, _D, _D,
                                     _D, _D, _D, cint, _D, _D, _D, cint]
    lib.mssm_oracle_scan.restype = cint
    lib.mssm_oracle_state_update.argtypes = [i64, i64, i64, i64, _D, _D, _D, _D, _D,
                                             _D, _D, _D, _D, cint, _D, cint]
    lib.mssm_oracle_state_update.restype = cint
    lib.mssm_oracle_scan_row.argtypes = [i64, i64, _D, _D, _D, _D, _D, _D,
                                         ctypes.c_double, ctypes.c_double,
                                         cint, _D, _D, _D]
    lib.mssm_oracle_scan_row.restype = None
    lib.mssm_oracle_scan_bwd.argtypes = [i64, i64, i64, i64, i64] + [_D] * 8 + [cint] + [_D] * 12
    lib.mssm_oracle_scan_bwd.restype = cint
    lib.mssm_oracle_causal_conv1d.argtypes = [i64, i64, i64, i64, _D, _D, _D,
                                              _D, cint, _D]
    lib.mssm_oracle_causal_conv1d.restype = cint
    lib.mssm_oracle_causal_conv1d_bwd.argtypes = [i64, i64, i64, i64, _D, _D, _D, _D,
                                                  cint, _D, _D, _D, _D, _D]
    lib.mssm_oracle_causal_conv1d_bwd.restype = cint
    return lib


def _f64(a):
    """Exact fp64 copy of a numpy array or a CPU torch tensor (bf16 included)."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_D)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


class Oracle:
    """The oracle's entry points bound to one compiled library."""

    def __init__(self, lib_path=None):
        if lib_path is None:
            lib_path = _LIB_PATH
            if not os.path.exists(lib_path):
                build(force=True)
        self.lib_path = lib_path
        self._lib = _open(lib_path)

    def scan(self, u, delta, A, B, C, D=None, z=None, delta_bias=None,
             softplus=True, h0=None, nthreads=None):
        """Selective scan in fp64.

        u, delta, z: (batch, dim, L); B, C: (batch, L, N), or (batch, L, G, N)
        for G groups of channels (channel d reads group d // (dim // G));
        A: (dim, N); D, delta_bias: (dim,); h0: (batch, dim, N) or None.
        Returns (out (batch, dim, L), last_state (batch, dim, N)), both fp64.
        """
        u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
        D, z, delta_bias, h0 = map(_f64, (D, z, delta_bias, h0))
        batch, dim, L = u.shape
        N = A.shape[1]
        G = B.shape[2] if B.ndim == 4 else 1
        assert delta.shape == u.shape and A.shape == (dim, N)
        assert B.shape == C.shape and B.shape in ((batch, L, N), (batch, L, G, N))
        assert z is None or z.shape == u.shape
        assert D is None or D.shape == (dim,)
        assert delta_bias is None or delta_bias.shape == (dim,)
        assert h0 is None or h0.shape == (batch, dim, N)
        out = np.empty((batch, dim, L), dtype=np.float64)
        last = np.empty((batch, dim, N), dtype=np.float64)
        rc = self._lib.mssm_oracle_scan(
            batch, dim, N, L, G, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
            _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(softplus)), _ptr(h0),
            _ptr(out), _ptr(last), int(nthreads or default_threads()))
        if rc != 0:
            raise ValueError("oracle: unsupported dstate %d or groups %d" % (N, G))
        return out, last

    def mamba2_scan(self, x, dt, A, B, C, D=None, z=None, dt_bias=None,
                    softplus=True, h0=None, nthreads=None):
        """The Mamba-2 block's scan in fp64, as the selective scan above with
        one A value, one step and one D per head (page "Mamba State Space
        Model", "Use the Mamba2 block", names the block and its state sizes;
        the per-head structure is the Mamba-2 architecture's).

        x, z: (batch, L, H, P) with headdim P; dt: (batch, L, H); A, D,
        dt_bias: (H,); B, C: (batch, L, G, N), heads h // (H // G) reading
        group g; h0: (batch, H * P, N) or None.  Channel d = h * P + p of the
        selective scan gets A[h] for every state, step dt[.., h] and D[h].
        Returns (out (batch, L, H, P), last_state (batch, H * P, N)), fp64.
        """
        x, dt, A, B, C = map(_f64, (x, dt, A, B, C))
        D, z, dt_bias, h0 = map(_f64, (D, z, dt_bias, h0))
        batch, L, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        assert dt.shape == (batch, L, H) and A.shape == (H,)
        assert B.shape == C.shape == (batch, L, G, N) and H % G == 0
        assert z is None or z.shape == x.shape
        dim = H * P

        def channels(a):   # (batch, L, H, P) -> (batch, dim, L)
            return np.ascontiguousarray(a.reshape(batch, L, dim).transpose(0, 2, 1))
        u = channels(x)
        delta = np.ascontiguousarray(np.repeat(dt, P, axis=2).transpose(0, 2, 1))
        A_full = np.repeat(A, P)[:, None] * np.ones((1, N))
        out, last = self.scan(
            u, delta, A_full, B, C,
            D=None if D is None else np.repeat(D, P), z=None if z is None else channels(z),
            delta_bias=None if dt_bias is None else np.repeat(dt_bias, P),
            softplus=softplus, h0=h0, nthreads=nthreads)
        return np.ascontiguousarray(out.transpose(0, 2, 1).reshape(batch, L, H, P)), last

    def scan_row(self, u, delta, A_row, B_b, C_b, D_d=0.0, z=None, bias_d=0.0,
                 softplus=True, h0=None):
        """One (batch, channel) row in fp64: u, delta, z of length L; A_row
        (N,); B_b, C_b (L, N).  Returns (out (L,), last_state (N,))."""
        u, delta, A_row, B_b, C_b, z, h0 = map(
            _f64, (u, delta, A_row, B_b, C_b, z, h0))
        L, N = u.shape[0], A_row.shape[0]
        assert B_b.shape == (L, N) and C_b.shape == (L, N)
        out = np.empty(L, dtype=np.float64)
        last = np.empty(N, dtype=np.float64)
        self._lib.mssm_oracle_scan_row(
            L, N, _ptr(u), _ptr(delta), _ptr(z), _ptr(A_row), _ptr(B_b),
            _ptr(C_b), float(D_d), float(bias_d), int(bool(softplus)),
            _ptr(h0), _ptr(out), _ptr(last))
        return out, last

    def scan_bwd(self, u, delta, A, B, C, dout, D=None, z=None,
                 delta_bias=None, softplus=True, h0=None, dlast=None):
        """Gradients of the scan for the loss sum(dout * out) +
        sum(dlast * last_state).  Returns a dict of fp64 arrays: du, ddelta
        (batch, dim, L), dA (dim, N), dB, dC (B's shape: (batch, L, N) or
        (batch, L, G, N)), dD, ddelta_bias (dim,), dz (batch, dim, L; None
        without z), dh0 (batch, dim, N)."""
        u, delta, A, B, C, dout = map(_f64, (u, delta, A, B, C, dout))
        D, z, delta_bias, h0, dlast = map(_f64, (D, z, delta_bias, h0, dlast))
        batch, dim, L = u.shape
        N = A.shape[1]
        G = B.shape[2] if B.ndim == 4 else 1
        assert dout.shape == u.shape and B.shape in ((batch, L, N), (batch, L, G, N))
        assert dlast is None or dlast.shape == (batch, dim, N)
        o = dict(du=np.empty_like(u), ddelta=np.empty_like(u),
                 dz=np.empty_like(u) if z is not None else None,
                 dA=np.empty((dim, N)), dB=np.empty(B.shape),
                 dC=np.empty(B.shape), dD=np.empty(dim),
                 ddelta_bias=np.empty(dim), dh0=np.empty((batch, dim, N)))
        rc = self._lib.mssm_oracle_scan_bwd(
            batch, dim, N, L, G, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
            _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(softplus)), _ptr(h0),
            _ptr(dout), _ptr(dlast), _ptr(o["du"]), _ptr(o["ddelta"]),
            _ptr(o["dz"]), _ptr(o["dA"]), _ptr(o["dB"]), _ptr(o["dC"]),
            _ptr(o["dD"]), _ptr(o["ddelta_bias"]), _ptr(o["dh0"]))
        if rc != 0:
            raise ValueError("oracle: scan_bwd failed (%d)" % rc)
        return o

    def causal_conv1d(self, x, w, bias=None, init=None, silu=True):
        """Causal depthwise convolution over time in fp64.

        x: (batch, dim, L); w: (dim, K); bias: (dim,) or None; init:
        (batch, dim, K-1) values of x before t = 0, or None for zeros.
        Returns (batch, dim, L) fp64: silu(conv) or, with silu=False, conv.
        """
        x, w, bias, init = map(_f64, (x, w, bias, init))
        batch, dim, L = x.shape
        K = w.shape[1]
        assert w.shape == (dim, K) and K >= 1
        assert bias is None or bias.shape == (dim,)
        assert init is None or init.shape == (batch, dim, K - 1)
        out = np.empty((batch, dim, L), dtype=np.float64)
        rc = self._lib.mssm_oracle_causal_conv1d(
            batch, dim, L, K, _ptr(x), _ptr(w), _ptr(bias), _ptr(init),
            int(bool(silu)), _ptr(out))
        if rc != 0:
            raise ValueError("oracle: bad conv width %d" % K)
        return out

    def causal_conv1d_bwd(self, x, w, dout, bias=None, init=None, silu=True):
        """Gradients of causal_conv1d (same arguments) for dout = dLoss/dout.

        Returns a dict of fp64 arrays: dx (batch, dim, L), dw (dim, K),
        dbias (dim,) and dinit (batch, dim, K-1), the gradient of the values
        before t = 0 (of the zeros when init is None).
        """
        x, w, bias, init, dout = map(_f64, (x, w, bias, init, dout))
        batch, dim, L = x.shape
        K = w.shape[1]
        assert w.shape == (dim, K) and K >= 1 and dout.shape == x.shape
        assert bias is None or bias.shape == (dim,)
        assert init is None or init.shape == (batch, dim, K - 1)
        o = {"dx": np.empty((batch, dim, L)), "dw": np.empty((dim, K)),
             "dbias": np.empty(dim), "dinit": np.empty((batch, dim, K - 1))}
        rc = self._lib.mssm_oracle_causal_conv1d_bwd(
            batch, dim, L, K, _ptr(x), _ptr(w), _ptr(bias), _ptr(init),
            int(bool(silu)), _ptr(dout), _ptr(o["dx"]), _ptr(o["dw"]),
            _ptr(o["dbias"]), _ptr(o["dinit"]))
        if rc != 0:
            raise ValueError("oracle: bad conv width %d" % K)
        return o

    def state_update(self, state, x, dt, A, B, C, D=None, z=None,
                     dt_bias=None, softplus=True, nthreads=None):
        """Single-token decode step in fp64.

        state: (batch, dim, N); x, dt, z: (batch, dim); B, C: (batch, N) or
        (batch, G, N) for G channel groups.
        Returns (out (batch, dim), new_state (batch, dim, N)); the inputs are
        left untouched.
        """
        st = _f64(state).copy()
        x, dt, A, B, C, D, z, dt_bias = map(
            _f64, (x, dt, A, B, C, D, z, dt_bias))
        batch, dim, N = st.shape
        G = B.shape[1] if B.ndim == 3 else 1
        assert x.shape == (batch, dim) and dt.shape == (batch, dim)
        assert A.shape == (dim, N) and B.shape in ((batch, N), (batch, G, N))
        assert C.shape == B.shape
        out = np.empty((batch, dim), dtype=np.float64)
        rc = self._lib.mssm_oracle_state_update(
            batch, dim, N, G, _ptr(st), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
            _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), int(bool(softplus)),
            _ptr(out), int(nthreads or default_threads()))
        if rc != 0:
            raise ValueError("oracle: unsupported dstate %d" % N)
        return out, st


_default = None


def _get():
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def scan(*args, **kwargs):
    """Selective scan in fp64 (see Oracle.scan)."""
    return _get().scan(*args, **kwargs)


def scan_row(*args, **kwargs):
    """One row of the scan in fp64 (see Oracle.scan_row)."""
    return _get().scan_row(*args, **kwargs)


def state_update(*args, **kwargs):
    """Single-token decode step in fp64 (see Oracle.state_update)."""
    return _get().state_update(*args, **kwargs)


def scan_bwd(*args, **kwargs):
    """Gradients of the scan in fp64 (see Oracle.scan_bwd)."""
    return _get().scan_bwd(*args, **kwargs)


def causal_conv1d(*args, **kwargs):
    """Causal depthwise convolution in fp64 (see Oracle.causal_conv1d)."""
    return _get().causal_conv1d(*args, **kwargs)


def causal_conv1d_bwd(*args, **kwargs):
    """Gradients of the causal convolution in fp64 (see Oracle.causal_conv1d_bwd)."""
    return _get().causal_conv1d_bwd(*args, **kwargs)


def mamba2_scan(*args, **kwargs):
    """The Mamba-2 block's scan in fp64 (see Oracle.mamba2_scan)."""
    return _get().mamba2_scan(*args, **kwargs)
