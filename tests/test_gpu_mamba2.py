"""The Mamba-2 block's scan on the GPU (mssm_mamba2_scan_fwd, through the C
ABI) against the fp64 oracle's Mamba-2 scan (the pinned selective scan on
per-head expanded inputs).

Bars as for the forward scan (tests/gpu_common.py): bf16 outputs within the
parity bar of the fp64 result, the fp32 final state within 1e-4 (1 + |h|).
The kernel's chunked matrix form reassociates the recurrence; its fp32
operands enter the bf16 matrix products as hi + lo halves (16 mantissa bits).
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_common import DEV, check_out, check_state, to_dev

pytestmark = pytest.mark.gpu


def _report(what, worst):
    print("%-56s worst err/bar = %.3g (parity), %.3g (tight)" % (what, *worst), flush=True)


def _run(inp, h0=None, time_segments=0):
    import selective_state_space_52_amd as m
    x = to_dev(inp["x"])
    batch, L, H, P = x.shape
    N = inp["B"].shape[3]
    last = (to_dev(h0).clone() if h0 is not None else
            torch.full((batch, H * P, N), float("nan"), device=DEV))
    out = m.mamba2_scan_fwd(x, to_dev(inp["dt"]), to_dev(inp["A"]), to_dev(inp["B"]),
                            to_dev(inp["C"]), D=to_dev(inp["D"]), z=to_dev(inp["z"]),
                            dt_bias=to_dev(inp["dt_bias"]), softplus=inp["softplus"],
                            last_state=last, load_state=h0 is not None,
                            time_segments=time_segments)
    torch.cuda.synchronize()
    return out.cpu(), last.cpu()


def _oracle(inp, h0=None):
    import oracle
    return oracle.mamba2_scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                              D=inp["D"], z=inp["z"], dt_bias=inp["dt_bias"],
                              softplus=inp["softplus"], h0=h0)


CASES = [
    # batch, L, heads, N, groups -- several 64-step chunks, ragged tails
    (2, 200, 4, 64, 1),
    (1, 64, 2, 128, 1),      # exactly one chunk
    (2, 1, 2, 64, 1),        # one step
    (1, 333, 4, 128, 2),     # two groups of two heads
    (3, 129, 3, 64, 3),      # a group per head
    (1, 1000, 2, 128, 1),    # long row, 16 chunks
]


@pytest.mark.parametrize("batch,L,H,N,G", CASES,
                         ids=["b%d-l%d-h%d-n%d-g%d" % c for c in CASES])
def test_mamba2_shapes(batch, L, H, N, G):
    s = W.spec("mamba2_2p7b_layer", batch=batch, seqlen=L, nheads=H, dstate=N,
               ngroups=G, seed=900 + L + N)
    inp = W.make_mamba2_inputs(s)
    out, last = _run(inp)
    ro, rl = _oracle(inp)
    _report("mamba2 %s" % ((batch, L, H, N, G),), check_out(out, ro, "bf16", "out"))
    check_state(last, rl, "last_state")


VARIANTS = [dict(has_z=False), dict(has_D=False), dict(has_bias=False),
            dict(softplus=False, has_bias=False)]


@pytest.mark.parametrize("var", VARIANTS,
                         ids=lambda v: ",".join("%s=%s" % kv for kv in v.items()))
def test_mamba2_optional_operands(var):
    s = W.spec("mamba2_2p7b_layer", batch=2, seqlen=150, nheads=3, dstate=64, seed=31,
               **var)
    inp = W.make_mamba2_inputs(s)
    if not s.softplus:
        # raw steps must stay positive without softplus: use |dt| * 0.05
        inp["dt"] = (inp["dt"].float().abs() * 0.05).to(torch.bfloat16)
    out, last = _run(inp)
    ro, rl = _oracle(inp)
    _report("mamba2 variant %s" % var, check_out(out, ro, "bf16", "out"))
    check_state(last, rl, "last_state")


@pytest.mark.parametrize("N", [64, 128])
def test_mamba2_loaded_state_and_split(N):
    """A loaded initial state; and two calls over the halves of a sequence,
    the second loading the first's final state, equal one call."""
    s = W.spec("mamba2_2p7b_layer", batch=2, seqlen=300, nheads=2, dstate=N, seed=41)
    inp = W.make_mamba2_inputs(s)
    h0 = W.mamba2_initial_state(s)
    out, last = _run(inp, h0=h0)
    ro, rl = _oracle(inp, h0=h0)
    check_out(out, ro, "bf16", "loaded out")
    check_state(last, rl, "loaded last_state")
    cut = 100   # not a multiple of the chunk length
    first = {k: (v[:, :cut].contiguous() if k in ("x", "dt", "z", "B", "C") else v)
             for k, v in inp.items()}
    second = {k: (v[:, cut:].contiguous() if k in ("x", "dt", "z", "B", "C") else v)
              for k, v in inp.items()}
    o1, l1 = _run(first, h0=h0)
    o2, l2 = _run(second, h0=l1)
    check_out(torch.cat([o1, o2], dim=1), ro, "bf16", "split out")
    check_state(l2, rl, "split last_state")


SEGMENTS = [
    # batch, L, heads, N, segments -- 1: no split; ragged last segments
    (2, 200, 4, 64, 1),
    (1, 1000, 2, 128, 1),
    (2, 300, 3, 64, 2),
    (1, 333, 2, 128, 3),
    (1, 640, 2, 64, 10),   # one chunk per segment
]


@pytest.mark.parametrize("batch,L,H,N,P", SEGMENTS,
                         ids=["b%d-l%d-h%d-n%d-p%d" % c for c in SEGMENTS])
def test_mamba2_time_segments(batch, L, H, N, P):
    """Rows cut into forced time segments (a state-only pass, the combine and
    the segments from their entering states), with a loaded initial state."""
    s = W.spec("mamba2_2p7b_layer", batch=batch, seqlen=L, nheads=H, dstate=N, seed=950 + P)
    inp = W.make_mamba2_inputs(s)
    h0 = W.mamba2_initial_state(s)
    out, last = _run(inp, h0=h0, time_segments=P)
    ro, rl = _oracle(inp, h0=h0)
    _report("mamba2 segments %s" % ((batch, L, H, N, P),), check_out(out, ro, "bf16", "out"))
    check_state(last, rl, "last_state")


def test_mamba2_full_size_sampled_heads():
    """The Mamba-2-2.7B-shaped layer (batch 4, L 2048, 80 heads x 64, N 128)
    in one call; the oracle follows 6 sampled (batch, head) pairs whole."""
    import oracle
    s = W.spec("mamba2_2p7b_layer")
    inp = W.make_mamba2_inputs(s)
    out, last = _run(inp)
    pairs = [(0, 0), (3, 79), (1, 40), (2, 7), (0, 63), (3, 1)]
    P = s.headdim
    for b, h in pairs:
        sub = dict(x=inp["x"][b:b + 1, :, h:h + 1], dt=inp["dt"][b:b + 1, :, h:h + 1],
                   z=inp["z"][b:b + 1, :, h:h + 1], B=inp["B"][b:b + 1], C=inp["C"][b:b + 1],
                   A=inp["A"][h:h + 1], D=inp["D"][h:h + 1], dt_bias=inp["dt_bias"][h:h + 1])
        ro, rl = oracle.mamba2_scan(sub["x"], sub["dt"], sub["A"], sub["B"], sub["C"],
                                    D=sub["D"], z=sub["z"], dt_bias=sub["dt_bias"],
                                    softplus=True)
        _report("mamba2 full size (b %d, head %d)" % (b, h),
                check_out(out[b:b + 1, :, h:h + 1], ro, "bf16", "out b%d h%d" % (b, h)))
        check_state(last[b:b + 1, h * P:(h + 1) * P], rl, "state b%d h%d" % (b, h))
    assert torch.isfinite(out.float()).all()


def test_mamba2_64bit_element_offsets():
    """A Mamba-2 scan of more than 2^31 elements per tensor (batch 8 x L 32768
    x 160 heads x 64 channels): every step of (batch, head) pairs whose
    elements lie on both sides of element 2^31 (batch entry 6), and of the
    first and last pairs, against the oracle on each pair alone."""
    import oracle
    import selective_state_space_52_amd as m
    batch, L, H, P, N = 8, 32768, 160, 64, 128
    assert batch * L * H * P > 2 ** 31
    print("Mamba-2 64-bit offsets: batch %d L %d heads %d" % (batch, L, H), flush=True)
    d = W.make_large_mamba2_inputs(batch, L, H, P, N, device=DEV)
    last = torch.full((batch, H * P, N), float("nan"), device=DEV)
    out = m.mamba2_scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"],
                            dt_bias=d["dt_bias"], softplus=True, last_state=last)
    torch.cuda.synchronize()
    b6 = 2 ** 31 // (L * H * P)
    for b, h in [(0, 0), (b6, 0), (b6, 77), (b6, H - 1), (batch - 1, H - 1)]:
        hs = slice(h, h + 1)
        ro, rl = oracle.mamba2_scan(d["x"][b:b + 1, :, hs].cpu(), d["dt"][b:b + 1, :, hs].cpu(),
                                    d["A"][hs].cpu(), d["B"][b:b + 1].cpu(), d["C"][b:b + 1].cpu(),
                                    D=d["D"][hs].cpu(), z=d["z"][b:b + 1, :, hs].cpu(),
                                    dt_bias=d["dt_bias"][hs].cpu(), softplus=True)
        check_out(out[b:b + 1, :, hs].cpu(), ro, "bf16", "pair (%d, %d) out" % (b, h))
        check_state(last[b:b + 1, h * P:(h + 1) * P].cpu(), rl, "pair (%d, %d) state" % (b, h))
    del d, out, last
    torch.cuda.empty_cache()
