"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the fp64 oracle on the same seeded inputs.

Tolerances (the parity bar):
  fp32 io : |gpu - ref| <= 1e-4 * (1 + |ref|)   element-wise
  bf16 io : |gpu - ref| <= 2e-2 * (1 + |ref|)   element-wise (fp32 state)
  state   : |gpu - ref| <= 1e-4 * (1 + |ref|)   for last_state / decode state
A second, tighter bar records what a correct fp32 kernel achieves, so that a
regression far below the parity bar still shows: fp32 outputs within
2e-5 * (1 + |ref|); bf16 outputs within 2^-8 |ref| + 2e-5 (one rounding to
bf16 costs at most 2^-9 relative).
"""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda:0"

BAR = {"f32": 1e-4, "bf16": 2e-2}
STATE_BAR = 1e-4


def to_dev(x):
    return None if x is None else x.to(DEV)


def np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def gpu_scan(inp, h0=None, time_segments=0, want_state=True):
    """Run the product path.  Returns (out, last_state) as CPU tensors."""
    import selective_state_space_52_amd as m
    u = to_dev(inp["u"])
    batch, dim, _ = u.shape
    N = inp["A"].shape[1]
    last = None
    if want_state or h0 is not None:
        last = (to_dev(h0).clone() if h0 is not None else
                torch.full((batch, dim, N), float("nan"), device=DEV))
    out = m.selective_scan_fwd(u, to_dev(inp["delta"]), to_dev(inp["A"]),
                               to_dev(inp["B"]), to_dev(inp["C"]),
                               D=to_dev(inp["D"]), z=to_dev(inp["z"]),
                               delta_bias=to_dev(inp["delta_bias"]),
                               softplus=inp["softplus"], last_state=last,
                               load_state=h0 is not None,
                               time_segments=time_segments)
    torch.cuda.synchronize()
    return out.cpu(), (last.cpu() if last is not None else None)


def oracle_scan(inp, h0=None):
    import oracle
    return oracle.scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                       D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                       softplus=inp["softplus"], h0=h0)


def oracle_rows(inp, rows, h0=None):
    """Oracle outputs and final states of the listed (b, d) rows only."""
    import oracle
    outs, lasts = [], []
    for b, d in rows:
        o, l = oracle.scan_row(
            inp["u"][b, d], inp["delta"][b, d], inp["A"][d], inp["B"][b],
            inp["C"][b], D_d=float(inp["D"][d]) if inp["D"] is not None else 0.0,
            z=inp["z"][b, d] if inp["z"] is not None else None,
            bias_d=float(inp["delta_bias"][d]) if inp["delta_bias"] is not None else 0.0,
            softplus=inp["softplus"], h0=None if h0 is None else h0[b, d])
        outs.append(o)
        lasts.append(l)
    return np.stack(outs), np.stack(lasts)


def sample_rows(batch, dim, k=48, seed=0):
    """Rows at group edges, the ends, and random ones."""
    rng = np.random.default_rng(seed)
    rows = {(0, 0), (batch - 1, dim - 1), (0, min(63, dim - 1)),
            (batch - 1, min(64, dim - 1)), (batch // 2, dim // 2)}
    while len(rows) < k:
        rows.add((int(rng.integers(batch)), int(rng.integers(dim))))
    return sorted(rows)


def check_out(gpu, ref, io, what="", ref_rounded=False):
    """Parity bar plus the tighter bar; returns the worst ratio to each.
    ref_rounded: the reference is itself a bf16 result (two roundings apart,
    so one full bf16 ulp, 2^-7 relative, is allowed by the tight bar)."""
    g = np64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), "%s: non-finite output" % what
    err = np.abs(g - r)
    bar = BAR[io] * (1.0 + np.abs(r))
    worst = float((err / bar).max()) if err.size else 0.0
    assert worst <= 1.0, "%s: parity bar exceeded, worst err/bar %.3g, max err %.3g" % (
        what, worst, float(err.max()))
    rel = 2.0 ** -7 if ref_rounded else 2.0 ** -8
    tight = (2e-5 * (1.0 + np.abs(r))) if io == "f32" else ((rel + 2e-6) * np.abs(r) + 2e-5)
    worst_t = float((err / tight).max()) if err.size else 0.0
    assert worst_t <= 1.0, "%s: tight bar exceeded, worst err/bar %.3g, max err %.3g" % (
        what, worst_t, float(err.max()))
    return worst, worst_t


def check_state(gpu, ref, what=""):
    g = np64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape
    err = np.abs(g - r)
    worst = float((err / (STATE_BAR * (1.0 + np.abs(r)))).max()) if err.size else 0.0
    assert np.isfinite(g).all() and worst <= 1.0, \
        "%s: state bar exceeded, worst %.3g, max err %.3g" % (what, worst, float(err.max()))
    return worst
