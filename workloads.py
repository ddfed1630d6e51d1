"""Seeded synthetic inputs for the selective scan and its decode step.

This module draws random numbers and rounds them to the storage dtype; it holds
none of the scan's arithmetic.  Both the oracle-side tests and the GPU path get
their inputs from here, so that they see bit-identical values.

Shapes follow the Mamba layer sizes the pages name: d_state = 16 and expand = 2
(page "Mamba: Selective State Space Models", "Quick Start"; page "Mamba State
Space Model", "Use the Mamba block"), so D_inner = 2 * d_model, with d_model
768 for the 130M model and 2560 for the 2.8B model (both named as Hugging Face
checkpoints on page "Mamba State Space Model", "Run zero-shot evaluations" and
"Benchmark Mamba generation latency and throughput").  Parameters that the
pages ask to keep in fp32 (page "Mamba State Space Model", "Troubleshoot model
instability with precision settings") -- A, D and the delta bias -- and the
recurrent state are fp32; activations are bf16 except in the tiny fp32 case.

Value recipe (all workloads):
  u, delta (raw, before bias and softplus), z, B, C ~ N(0, 1)
  dt ~ exp(U[ln 1e-3, ln 1e-1]) per channel; delta_bias = inv_softplus(dt)
      = log(expm1(dt)), so that softplus(0 + bias) = dt  (the bias init range
      of page "Mamba State Space Model", "Troubleshoot initialization issues")
  A[d, n] = -(n + 1)  (real, one N-vector per channel)
  D ~ N(0, 1) per channel
  decode state ~ 0.1 * N(0, 1)
Draw order from numpy.random.default_rng(seed): u, delta, z, B, C, D, log-dt,
then (decode only) the state.  The backward's incoming gradients use
default_rng([seed, 104729]): dout ~ N(0, 1) in the io dtype, then dlast ~
N(0, 1) fp32.  The causal conv ahead of the scan (width 4) draws from
default_rng([seed, 7717]): weight, bias ~ U(-1/2, 1/2) fp32 (a framework's
default Conv1d range 1/sqrt(width)), then the initial inputs ~ N(0, 1) in the
io dtype; the conv input x is the workload's u.  Decode tokens use default_rng([seed, 1 + k]) for
token k of a ring of ``tokens`` distinct tokens; step s uses token s % tokens.
bf16 values are fp32 draws rounded to nearest-even (torch's conversion).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class ScanSpec:
    name: str
    batch: int
    dim: int
    dstate: int
    seqlen: int
    io: str = "bf16"          # "f32" or "bf16": dtype of u, delta, z, B, C, out
    seed: int = 0
    softplus: bool = True
    has_z: bool = True
    has_D: bool = True
    has_bias: bool = True
    chunk: int = 0            # >0: the workload is also run as seqlen/chunk calls
    note: str = ""

    @property
    def elements(self) -> int:
        return self.batch * self.dim * self.seqlen

    @property
    def state_elements(self) -> int:
        return self.elements * self.dstate


@dataclass(frozen=True)
class DecodeSpec:
    name: str
    batch: int
    dim: int
    dstate: int
    steps: int = 1000
    tokens: int = 16          # ring of distinct seeded tokens
    io: str = "bf16"
    seed: int = 4
    softplus: bool = True
    state_std: float = 0.1
    note: str = ""


@dataclass(frozen=True)
class Mamba2Spec:
    """The Mamba-2 block's scan: heads of `headdim` channels, bf16 activations."""
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int = 1
    seed: int = 5
    softplus: bool = True
    has_z: bool = True
    has_D: bool = True
    has_bias: bool = True
    note: str = ""

    @property
    def dim(self) -> int:
        return self.nheads * self.headdim

    @property
    def elements(self) -> int:
        return self.batch * self.seqlen * self.dim

    @property
    def state_elements(self) -> int:
        return self.elements * self.dstate


WORKLOADS = {
    "tiny_f32": ScanSpec("tiny_f32", 1, 64, 16, 256, io="f32", seed=0,
                         note="tiny fp32 scan"),
    "mamba130m_layer": ScanSpec("mamba130m_layer", 8, 1536, 16, 2048, seed=1,
                                note="Mamba-130M-shaped layer scan, bf16 io, "
                                     "fp32 state, last_state out"),
    "mamba2p8b_layer": ScanSpec("mamba2p8b_layer", 4, 5120, 16, 2048, seed=2,
                                note="Mamba-2.8B-shaped layer scan, bf16 io"),
    "long_chunked": ScanSpec("long_chunked", 1, 1536, 16, 131072, seed=3,
                             chunk=2048,
                             note="long sequence, state carried across "
                                  "2048-step chunks"),
    "decode": DecodeSpec("decode", 256, 5120, 16, steps=1000, seed=4,
                         note="single-token state update, 256 sequences"),
    "mamba2_2p7b_layer": Mamba2Spec("mamba2_2p7b_layer", 4, 2048, 80, 64, 128, seed=5,
                                    note="Mamba-2-2.7B-shaped layer scan: 80 heads of "
                                         "64 channels (D_inner 5120), N 128, one group"),
}


def spec(name: str, **overrides):
    s = WORKLOADS[name]
    return replace(s, **overrides) if overrides else s


def _round_io(a: np.ndarray, io: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if io == "f32":
        return t
    if io == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError("io dtype must be 'f32' or 'bf16', got %r" % (io,))


def _params(rng: np.random.Generator, dim: int, dstate: int):
    D = rng.standard_normal(dim, dtype=np.float32)
    log_dt = rng.uniform(math.log(1e-3), math.log(1e-1), size=dim)
    dt = np.exp(log_dt)
    bias = np.log(np.expm1(dt)).astype(np.float32)
    A = np.broadcast_to(-(np.arange(dstate, dtype=np.float32) + 1.0),
                        (dim, dstate)).copy()
    return A, D, bias


def make_scan_inputs(s: ScanSpec) -> dict:
    """CPU tensors for one scan call: io-dtype u, delta, z, B, C and fp32 A, D,
    delta_bias (None where the spec switches them off)."""
    rng = np.random.default_rng(s.seed)
    shp = (s.batch, s.dim, s.seqlen)
    bshp = (s.batch, s.seqlen, s.dstate)
    u = _round_io(rng.standard_normal(shp, dtype=np.float32), s.io)
    delta = _round_io(rng.standard_normal(shp, dtype=np.float32), s.io)
    z = _round_io(rng.standard_normal(shp, dtype=np.float32), s.io)
    B = _round_io(rng.standard_normal(bshp, dtype=np.float32), s.io)
    C = _round_io(rng.standard_normal(bshp, dtype=np.float32), s.io)
    A, D, bias = _params(rng, s.dim, s.dstate)
    return dict(
        u=u, delta=delta, A=torch.from_numpy(A), B=B, C=C,
        D=torch.from_numpy(D) if s.has_D else None,
        z=z if s.has_z else None,
        delta_bias=torch.from_numpy(bias) if s.has_bias else None,
        softplus=s.softplus,
    )


def make_initial_state(s, seed_offset: int = 7919) -> torch.Tensor:
    """fp32 (batch, dim, N) state ~ state_std * N(0,1) for carried-state cases."""
    rng = np.random.default_rng([s.seed, seed_offset])
    std = getattr(s, "state_std", 0.1)
    return torch.from_numpy(
        (std * rng.standard_normal((s.batch, s.dim, s.dstate))).astype(np.float32))


def make_scan_grads(s: ScanSpec, seed_offset: int = 104729) -> dict:
    """Incoming gradients for the backward: io-dtype dout (batch, dim, L) and
    fp32 dlast (batch, dim, N), both ~ N(0, 1)."""
    rng = np.random.default_rng([s.seed, seed_offset])
    dout = _round_io(rng.standard_normal((s.batch, s.dim, s.seqlen),
                                         dtype=np.float32), s.io)
    dlast = torch.from_numpy(
        rng.standard_normal((s.batch, s.dim, s.dstate), dtype=np.float32))
    return dict(dout=dout, dlast=dlast)


def make_group_bc(s: ScanSpec, groups: int, seed_offset: int = 3571) -> dict:
    """io-dtype B, C (batch, L, groups, N) ~ N(0, 1) for G B/C groups (channel
    d reads group d // (dim // groups)); draws from default_rng([seed,
    seed_offset]), B then C."""
    rng = np.random.default_rng([s.seed, seed_offset])
    shp = (s.batch, s.seqlen, groups, s.dstate)
    B = _round_io(rng.standard_normal(shp, dtype=np.float32), s.io)
    C = _round_io(rng.standard_normal(shp, dtype=np.float32), s.io)
    return dict(B=B, C=C)


def make_conv_params(s: ScanSpec, width: int = 4, seed_offset: int = 7717) -> dict:
    """fp32 weight (dim, width) and bias (dim) ~ U(-1/2, 1/2), and io-dtype
    init (batch, dim, width - 1) ~ N(0, 1), for the causal conv."""
    rng = np.random.default_rng([s.seed, seed_offset])
    w = rng.uniform(-0.5, 0.5, size=(s.dim, width)).astype(np.float32)
    b = rng.uniform(-0.5, 0.5, size=s.dim).astype(np.float32)
    init = _round_io(rng.standard_normal((s.batch, s.dim, width - 1),
                                         dtype=np.float32), s.io)
    return dict(weight=torch.from_numpy(w), bias=torch.from_numpy(b), init=init)


def conv_bytes(s: ScanSpec, width: int = 4) -> int:
    """Algorithmic HBM bytes of the standalone conv: x read and the output
    written once, plus the weights."""
    io = 4 if s.io == "f32" else 2
    return 2 * s.elements * io + 4 * s.dim * (width + 1)


def conv_bwd_bytes(s: ScanSpec, width: int = 4) -> int:
    """Algorithmic HBM bytes of the conv's backward: x and dout read once, dx
    written once, the weights and bias read and their gradients written, the
    initial values read."""
    io = 4 if s.io == "f32" else 2
    return 3 * s.elements * io + 2 * 4 * s.dim * (width + 1) + s.batch * s.dim * (width - 1) * io


def scan_bwd_bytes(s: ScanSpec, has_h0: bool = False, has_dlast: bool = False,
                   want_dh0: bool = False) -> int:
    """Algorithmic HBM bytes of one backward call: the forward's operands and
    dout read once; du, ddelta, dz (io dtype) and dA, dB, dC, dD, dbias (fp32)
    written once."""
    io = 4 if s.io == "f32" else 2
    e = s.elements
    n_in = 3 + int(s.has_z)                             # u, delta, dout, z
    n_out = 2 + int(s.has_z)                            # du, ddelta, dz
    b = (n_in + n_out) * e * io
    b += 2 * s.batch * s.seqlen * s.dstate * io         # B, C in
    b += 2 * s.batch * s.seqlen * s.dstate * 4          # dB, dC out (fp32)
    b += 2 * 4 * s.dim * s.dstate                       # A in, dA out
    b += 2 * 4 * s.dim * (int(s.has_D) + int(s.has_bias))  # D, bias; dD, dbias
    rows = s.batch * s.dim
    b += 4 * rows * s.dstate * (int(has_h0) + int(has_dlast) + int(want_dh0))
    return b


def make_decode_params(s: DecodeSpec) -> dict:
    """fp32 A, D, dt_bias and the initial fp32 state for the decode workload."""
    rng = np.random.default_rng(s.seed)
    A, D, bias = _params(rng, s.dim, s.dstate)
    state = (s.state_std * rng.standard_normal((s.batch, s.dim, s.dstate))
             ).astype(np.float32)
    return dict(A=torch.from_numpy(A), D=torch.from_numpy(D),
                dt_bias=torch.from_numpy(bias), state=torch.from_numpy(state))


def make_large_decode_step(batch: int, dim: int, dstate: int, seed: int = 31,
                           device="cuda") -> dict:
    """One bf16 decode token and an fp32 state of N(0, 0.1^2) drawn directly on
    `device` (for sizes too large to draw on the host), with A, D and dt_bias
    as for the other workloads."""
    A, D, bias = _params(np.random.default_rng(seed), dim, dstate)
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def normal(*shape):
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return dict(state=normal(batch, dim, dstate).mul_(0.1),
                x=normal(batch, dim).to(torch.bfloat16),
                dt=normal(batch, dim).to(torch.bfloat16),
                z=normal(batch, dim).to(torch.bfloat16),
                B=normal(batch, dstate).to(torch.bfloat16),
                C=normal(batch, dstate).to(torch.bfloat16),
                A=torch.from_numpy(A).to(device), D=torch.from_numpy(D).to(device),
                dt_bias=torch.from_numpy(bias).to(device))


def make_large_scan_inputs(batch: int, dim: int, seqlen: int, dstate: int = 16,
                           seed: int = 33, device="cuda") -> dict:
    """bf16 u, delta, z (batch, dim, L) and B, C (batch, L, N) ~ N(0, 1) drawn
    directly on `device` (for sizes too large to draw on the host), one batch
    entry at a time, with A, D and delta_bias as for the other workloads."""
    A, D, bias = _params(np.random.default_rng(seed), dim, dstate)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = {}
    for name in ("u", "delta", "z"):
        t = torch.empty(batch, dim, seqlen, dtype=torch.bfloat16, device=device)
        for b in range(batch):
            t[b] = torch.randn(dim, seqlen, generator=g, device=device, dtype=torch.float32)
        out[name] = t
    for name in ("B", "C"):
        out[name] = torch.randn(batch, seqlen, dstate, generator=g, device=device,
                                dtype=torch.float32).to(torch.bfloat16)
    out.update(A=torch.from_numpy(A).to(device), D=torch.from_numpy(D).to(device),
               delta_bias=torch.from_numpy(bias).to(device))
    return out


def make_large_scan_dout(batch: int, dim: int, seqlen: int, seed: int = 34,
                         device="cuda") -> torch.Tensor:
    """bf16 incoming gradient dout (batch, dim, L) ~ N(0, 1), drawn on `device`
    one batch entry at a time."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.empty(batch, dim, seqlen, dtype=torch.bfloat16, device=device)
    for b in range(batch):
        t[b] = torch.randn(dim, seqlen, generator=g, device=device, dtype=torch.float32)
    return t


def make_large_mamba2_inputs(batch: int, seqlen: int, nheads: int, headdim: int = 64,
                             dstate: int = 128, ngroups: int = 1, seed: int = 36,
                             device="cuda") -> dict:
    """The Mamba-2 scan's inputs drawn on `device` (x, z, dt, B, C ~ N(0, 1) in
    bf16, one batch entry at a time) with the per-head A, D and dt_bias of
    make_mamba2_inputs drawn on the host."""
    rng = np.random.default_rng(seed)
    A = -rng.uniform(1.0, 16.0, nheads).astype(np.float32)
    D = rng.standard_normal(nheads, dtype=np.float32)
    log_dt = rng.uniform(math.log(1e-3), math.log(1e-1), size=nheads)
    bias = np.log(np.expm1(np.exp(log_dt))).astype(np.float32)
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def draw(*shape):
        t = torch.empty(shape, dtype=torch.bfloat16, device=device)
        for b in range(shape[0]):
            t[b] = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
        return t
    return dict(x=draw(batch, seqlen, nheads, headdim), dt=draw(batch, seqlen, nheads),
                z=draw(batch, seqlen, nheads, headdim),
                B=draw(batch, seqlen, ngroups, dstate), C=draw(batch, seqlen, ngroups, dstate),
                A=torch.from_numpy(A).to(device), D=torch.from_numpy(D).to(device),
                dt_bias=torch.from_numpy(bias).to(device), softplus=True)


def make_decode_token(s: DecodeSpec, k: int) -> dict:
    """Token k of the ring: io-dtype x, dt (raw), z (batch, dim) and B, C
    (batch, N)."""
    rng = np.random.default_rng([s.seed, 1 + k])
    shp = (s.batch, s.dim)
    x = _round_io(rng.standard_normal(shp, dtype=np.float32), s.io)
    dt = _round_io(rng.standard_normal(shp, dtype=np.float32), s.io)
    z = _round_io(rng.standard_normal(shp, dtype=np.float32), s.io)
    B = _round_io(rng.standard_normal((s.batch, s.dstate), dtype=np.float32), s.io)
    C = _round_io(rng.standard_normal((s.batch, s.dstate), dtype=np.float32), s.io)
    return dict(x=x, dt=dt, z=z, B=B, C=C)


def scan_bytes(s: ScanSpec, load_state: bool = False, write_state: bool = True) -> int:
    """Algorithmic HBM bytes of one scan call: every operand read once and every
    result written once."""
    io = 4 if s.io == "f32" else 2
    e = s.elements
    b = 3 * e * io if s.has_z else 2 * e * io          # u, delta, z in
    b += e * io                                         # out
    b += 2 * s.batch * s.seqlen * s.dstate * io         # B, C
    b += 4 * s.dim * s.dstate                           # A
    b += 4 * s.dim * (int(s.has_D) + int(s.has_bias))   # D, delta_bias
    rows = s.batch * s.dim
    if write_state:
        b += 4 * rows * s.dstate
    if load_state:
        b += 4 * rows * s.dstate
    return b


def decode_step_bytes(s: DecodeSpec) -> int:
    """Algorithmic HBM bytes of one decode step (state read and written once)."""
    io = 4 if s.io == "f32" else 2
    rows = s.batch * s.dim
    b = 2 * 4 * rows * s.dstate            # state in + out
    b += 4 * rows * io                     # x, dt, z in; out
    b += 2 * s.batch * s.dstate * io       # B, C
    b += 4 * s.dim * s.dstate + 2 * 4 * s.dim   # A, D, dt_bias
    return b


def make_mamba2_inputs(s: Mamba2Spec) -> dict:
    """Inputs of the Mamba-2 scan: x, z (batch, L, H, P), dt (batch, L, H), B, C
    (batch, L, G, N) ~ N(0, 1) in bf16; per head A = -U[1, 16], D ~ N(0, 1),
    dt_bias = inv_softplus(exp(U[ln 1e-3, ln 1e-1])), all fp32.  Draw order
    from default_rng(seed): x, dt, z, B, C, A, D, log-dt."""
    rng = np.random.default_rng(s.seed)
    b, L, H, P, N, G = s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups
    f32 = np.float32
    x = _round_io(rng.standard_normal((b, L, H, P), dtype=f32), "bf16")
    dt = _round_io(rng.standard_normal((b, L, H), dtype=f32), "bf16")
    z = _round_io(rng.standard_normal((b, L, H, P), dtype=f32), "bf16")
    B = _round_io(rng.standard_normal((b, L, G, N), dtype=f32), "bf16")
    C = _round_io(rng.standard_normal((b, L, G, N), dtype=f32), "bf16")
    A = -rng.uniform(1.0, 16.0, H).astype(f32)
    D = rng.standard_normal(H, dtype=f32)
    log_dt = rng.uniform(math.log(1e-3), math.log(1e-1), size=H)
    bias = np.log(np.expm1(np.exp(log_dt))).astype(f32)
    return dict(x=x, dt=dt, z=z if s.has_z else None, B=B, C=C, A=torch.from_numpy(A),
                D=torch.from_numpy(D) if s.has_D else None,
                dt_bias=torch.from_numpy(bias) if s.has_bias else None,
                softplus=s.softplus)


def mamba2_initial_state(s: Mamba2Spec, seed_offset: int = 7919) -> torch.Tensor:
    """(batch, H * P, N) fp32 initial state ~ 0.1 N(0, 1)."""
    rng = np.random.default_rng([s.seed, seed_offset])
    return torch.from_numpy(
        0.1 * rng.standard_normal((s.batch, s.dim, s.dstate), dtype=np.float32))


def mamba2_bytes(s: Mamba2Spec, load_state: bool = False) -> int:
    """Algorithmic bytes of one Mamba-2 scan call: x, z read and out written
    (bf16), dt (bf16), B, C (bf16), A, D, dt_bias (fp32), the final state
    written (fp32, and read when loaded)."""
    act = s.elements * 2 * (3 if s.has_z else 2)
    dt = s.batch * s.seqlen * s.nheads * 2
    bc = 2 * s.batch * s.seqlen * s.ngroups * s.dstate * 2
    par = 3 * s.nheads * 4
    st = s.batch * s.dim * s.dstate * 4 * (2 if load_state else 1)
    return act + dt + bc + par + st
