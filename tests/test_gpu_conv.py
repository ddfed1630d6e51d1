"""Causal conv (standalone) and the conv-fed forward scan on the GPU, through
the C ABI, against the fp64 oracle (conv, then scan of its output).

Bars as for the forward scan (tests/gpu_common.py): the GPU forms the conv in
fp32 from the exact io-dtype inputs and, in the fused path, feeds the scan the
fp32 conv output, while the oracle composes its fp64 conv and fp64 scan.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_common import (DEV, check_out, check_state, np64, oracle_rows,
                              sample_rows, to_dev)

pytestmark = pytest.mark.gpu


def _report(what, worst):
    print("%-52s worst err/bar = %.3g (parity), %.3g (tight)" % (what, *worst), flush=True)


def _case(name="mamba130m_layer", width=4, **over):
    s = W.spec(name, **over)
    return s, W.make_scan_inputs(s), W.make_conv_params(s, width)


CONV_SHAPES = [
    # io, batch, dim, L, width, silu, init, bias
    ("bf16", 2, 96, 256, 4, True, True, True),      # vector path
    ("bf16", 2, 70, 333, 4, True, False, True),     # element path, ragged
    ("f32", 1, 64, 264, 4, True, True, False),      # fp32 vector path
    ("f32", 2, 33, 77, 3, False, True, True),       # width 3, no activation
    ("bf16", 1, 40, 5, 2, True, True, True),        # shorter than a chunk
    ("bf16", 1, 8, 1, 4, True, True, True),         # one step: all init
]


@pytest.mark.parametrize("io,batch,dim,L,width,silu,use_init,use_bias", CONV_SHAPES,
                         ids=["%s-b%d-d%d-l%d-k%d-s%d-i%d-b%d" % c for c in CONV_SHAPES])
def test_conv_shapes(io, batch, dim, L, width, silu, use_init, use_bias):
    import oracle
    import selective_state_space_52_amd as m
    s, inp, cp = _case(io=io, batch=batch, dim=dim, seqlen=L, seed=600 + L + width)
    x = inp["u"]
    init = cp["init"] if use_init else None
    bias = cp["bias"] if use_bias else None
    out = m.causal_conv1d_fwd(to_dev(x), to_dev(cp["weight"]), to_dev(bias),
                              to_dev(init), silu=silu)
    torch.cuda.synchronize()
    ref = oracle.causal_conv1d(x, cp["weight"], bias, init, silu=silu)
    _report("conv %s" % ((io, batch, dim, L, width, silu, use_init, use_bias),),
            check_out(out.cpu(), ref, io, "conv"))


def _fused(inp, cp, use_init=True, h0=None, time_segments=0, want_u=False):
    import selective_state_space_52_amd as m
    u = to_dev(inp["u"])
    batch, dim, L = u.shape
    N = inp["A"].shape[1]
    last = (to_dev(h0).clone() if h0 is not None else
            torch.full((batch, dim, N), float("nan"), device=DEV))
    u_out = torch.empty_like(u) if want_u else None
    out = m.selective_scan_fwd_conv(
        u, to_dev(cp["weight"]), to_dev(inp["delta"]), to_dev(inp["A"]),
        to_dev(inp["B"]), to_dev(inp["C"]), conv_bias=to_dev(cp["bias"]),
        conv_init=to_dev(cp["init"]) if use_init else None, D=to_dev(inp["D"]),
        z=to_dev(inp["z"]), delta_bias=to_dev(inp["delta_bias"]),
        softplus=inp["softplus"], last_state=last, load_state=h0 is not None,
        u_out=u_out, time_segments=time_segments)
    torch.cuda.synchronize()
    return out.cpu(), last.cpu(), (u_out.cpu() if want_u else None)


def _oracle_fused(inp, cp, use_init=True, h0=None):
    import oracle
    u = oracle.causal_conv1d(inp["u"], cp["weight"], cp["bias"],
                             cp["init"] if use_init else None, silu=True)
    out, last = oracle.scan(u, inp["delta"], inp["A"], inp["B"], inp["C"],
                            D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                            softplus=inp["softplus"], h0=h0)
    return u, out, last


FUSED = [
    # io, batch, dim, N, L, segments, init
    ("f32", 1, 64, 16, 256, 0, True),
    ("bf16", 2, 96, 16, 512, 0, True),      # vector path
    ("bf16", 2, 70, 16, 333, 0, False),     # element path, ragged group/tile
    ("bf16", 1, 64, 16, 1000, 3, True),     # segments start inside the row
    ("f32", 2, 40, 8, 264, 2, True),
    ("bf16", 1, 64, 4, 37, 0, True),
    ("bf16", 1, 64, 64, 300, 2, True),
]


@pytest.mark.parametrize("io,batch,dim,N,L,P,use_init", FUSED,
                         ids=["%s-b%d-d%d-n%d-l%d-p%d-i%d" % c for c in FUSED])
def test_fused_scan_conv(io, batch, dim, N, L, P, use_init):
    s, inp, cp = _case(io=io, batch=batch, dim=dim, dstate=N, seqlen=L, seed=700 + L)
    out, last, u_gpu = _fused(inp, cp, use_init, time_segments=P, want_u=True)
    u, ro, rl = _oracle_fused(inp, cp, use_init)
    _report("fused %s" % ((io, batch, dim, N, L, P, use_init),), check_out(out, ro, io, "out"))
    check_state(last, rl, "last_state")
    check_out(u_gpu, u, io, "u_out")


def test_fused_scan_conv_chained():
    """Two calls over the halves of a sequence -- the second with the first
    half's last 3 inputs as conv_init and its final state loaded -- equal one
    call over the whole sequence."""
    s, inp, cp = _case(batch=2, dim=80, seqlen=512, seed=811)
    cut = 256
    whole, wlast, _ = _fused(inp, cp)
    first = {k: (v[:, :, :cut] if k in ("u", "delta", "z") else
                 v[:, :cut] if k in ("B", "C") else v) for k, v in inp.items()}
    second = {k: (v[:, :, cut:] if k in ("u", "delta", "z") else
                  v[:, cut:] if k in ("B", "C") else v) for k, v in inp.items()}
    for d in (first, second):
        for k in ("u", "delta", "z", "B", "C"):
            d[k] = d[k].contiguous()
    o1, l1, _ = _fused(first, cp)
    cp2 = dict(cp, init=inp["u"][:, :, cut - 3:cut].contiguous())
    o2, l2, _ = _fused(second, cp2, h0=l1)
    r_u, ro, rl = _oracle_fused(inp, cp)
    check_out(torch.cat([o1, o2], dim=2), ro, "bf16", "chained out")
    check_state(l2, rl, "chained last_state")
    check_out(whole, ro, "bf16", "whole out")


def test_fused_full_size_every_element():
    """The 2.8B-shaped layer with the conv, in the launch configuration the
    bench times: every output and final state against the oracle's conv then
    scan."""
    s, inp, cp = _case("mamba2p8b_layer")
    print("fused full size: batch %d dim %d L %d" % (s.batch, s.dim, s.seqlen), flush=True)
    out, last, _ = _fused(inp, cp)
    _, ro, rl = _oracle_fused(inp, cp)
    _report("fused full size every element", check_out(out, ro, "bf16", "out"))
    check_state(last, rl, "last_state")


def test_conv_64bit_element_offsets():
    """The standalone conv on more than 2^31 elements (batch 2 x 36864 x
    32768): rows on both sides of element 2^31, and the first and last rows,
    against the oracle."""
    import oracle
    import selective_state_space_52_amd as m
    batch, dim, L = 2, 36864, 32768
    assert batch * dim * L > 2 ** 31
    print("conv 64-bit offsets: batch %d dim %d L %d" % (batch, dim, L), flush=True)
    x = W.make_large_scan_inputs(batch, dim, L, device=DEV)["u"]
    cp = W.make_conv_params(W.spec("mamba130m_layer", batch=batch, dim=dim, seqlen=L, seed=37))
    w, bias, init = (to_dev(cp["weight"]), to_dev(cp["bias"]), to_dev(cp["init"]))
    out = m.causal_conv1d_fwd(x, w, bias=bias, init=init, silu=True)
    torch.cuda.synchronize()
    r0 = 2 ** 31 // L
    for r in sorted({0, r0 - 1, r0, r0 + 1, batch * dim - 1}):
        b, c = divmod(r, dim)
        ref = oracle.causal_conv1d(x[b:b + 1, c:c + 1].cpu(), cp["weight"][c:c + 1],
                                   bias=cp["bias"][c:c + 1], init=cp["init"][b:b + 1, c:c + 1],
                                   silu=True)
        check_out(out[b:b + 1, c:c + 1].cpu(), ref, "bf16", "conv row %d" % r)
    del x, out
    torch.cuda.empty_cache()
