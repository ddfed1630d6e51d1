"""Backward of the causal conv on the GPU, through the C ABI, against the
fp64 oracle's gradients (which central differences of the pinned forward
conv pin on the CPU).

Bar as for the scan's backward (tests/test_gpu_bwd.py): each gradient is a
sum of fp32 products (over the taps for dx and dinit, over batch and time for
dweight and dbias), so its rounding scales with the terms:
    |gpu - ref| <= 2e-4 * (|ref| + rms(ref)),
plus one bf16 rounding (2^-8 |ref|) for dx and dinit with bf16 io.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_common import np64, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-4


def _check(gpu, ref, io, name, rounded):
    g = np64(gpu)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.isfinite(g).all(), "%s: non-finite" % name
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    bar = TOL * (np.abs(r) + rms)
    if io == "bf16" and rounded:
        bar = bar + 2.0 ** -8 * np.abs(r)
    err = np.abs(g - r)
    worst = float((err / np.maximum(bar, 1e-30)).max())
    assert worst <= 1.0, "%s: bar exceeded, worst err/bar %.3g, max err %.3g, rms %.3g" % (
        name, worst, float(err.max()), rms)
    return worst


def _case(io, batch, dim, L, width, seed):
    s = W.spec("mamba130m_layer", io=io, batch=batch, dim=dim, seqlen=L, seed=seed)
    inp = W.make_scan_inputs(s)
    cp = W.make_conv_params(s, width)
    rng = np.random.default_rng([seed, 17])
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    dout = torch.from_numpy(rng.standard_normal((batch, dim, L), dtype=np.float32)).to(dt)
    return inp["u"], cp, dout


def _run(x, cp, dout, use_bias, use_init, silu, want_dinit=True):
    import selective_state_space_52_amd as m
    g = m.causal_conv1d_bwd(to_dev(x), to_dev(cp["weight"]), to_dev(dout),
                            bias=to_dev(cp["bias"]) if use_bias else None,
                            init=to_dev(cp["init"]) if use_init else None,
                            silu=silu, dinit=want_dinit)
    torch.cuda.synchronize()
    return [None if t is None else t.cpu() for t in g]


def _oracle(x, cp, dout, use_bias, use_init, silu):
    import oracle
    return oracle.causal_conv1d_bwd(x, cp["weight"], dout,
                                    bias=cp["bias"] if use_bias else None,
                                    init=cp["init"] if use_init else None, silu=silu)


def _compare(g, r, io, what):
    dx, dw, db, di = g
    worst = {"dx": _check(dx, r["dx"], io, what + " dx", True),
             "dw": _check(dw, r["dw"], io, what + " dweight", False),
             "db": _check(db, r["dbias"], io, what + " dbias", False)}
    if di is not None:
        worst["dinit"] = _check(di, r["dinit"], io, what + " dinit", True)
    print("%-48s %s" % (what, " ".join("%s=%.2g" % kv for kv in worst.items())), flush=True)


SHAPES = [
    # io, batch, dim, L, width, silu, init, bias
    ("bf16", 2, 96, 256, 4, True, True, True),       # vector path
    ("bf16", 2, 70, 333, 4, True, False, True),      # element path, ragged
    ("f32", 1, 64, 264, 4, True, True, False),       # fp32 vector path
    ("f32", 2, 33, 77, 3, False, True, True),        # width 3, no activation
    ("bf16", 3, 19, 4104, 2, True, True, True),      # rows longer than a stride of chunks
    ("bf16", 1, 40, 5, 2, True, True, True),         # shorter than a chunk
    ("bf16", 1, 8, 1, 4, True, True, True),          # one step
    ("f32", 2, 5, 3, 4, False, False, False),        # shorter than the width, no init
]


@pytest.mark.parametrize("io,batch,dim,L,width,silu,use_init,use_bias", SHAPES,
                         ids=["%s-b%d-d%d-l%d-k%d-s%d-i%d-b%d" % c for c in SHAPES])
def test_conv_bwd_shapes(io, batch, dim, L, width, silu, use_init, use_bias):
    x, cp, dout = _case(io, batch, dim, L, width, seed=700 + L + width)
    g = _run(x, cp, dout, use_bias, use_init, silu)
    r = _oracle(x, cp, dout, use_bias, use_init, silu)
    _compare(g, r, io, "conv bwd %s" % ((io, batch, dim, L, width, silu, use_init, use_bias),))


def test_conv_bwd_optional_outputs():
    """Without dinit (and with the binding's dbias always requested) the
    other gradients are unchanged."""
    x, cp, dout = _case("bf16", 2, 64, 128, 4, seed=733)
    a = _run(x, cp, dout, True, True, True, want_dinit=True)
    b = _run(x, cp, dout, True, True, True, want_dinit=False)
    assert b[3] is None
    for k in range(3):
        assert torch.equal(a[k], b[k])


def test_conv_bwd_full_size_every_element():
    """The 2.8B-shaped layer (batch 4, D 5120, L 2048, width 4, bf16): every
    dx and every channel's dweight and dbias against the oracle; repeated
    calls give the same bits."""
    s = W.spec("mamba2p8b_layer")
    print("conv bwd full size: batch %d dim %d L %d" % (s.batch, s.dim, s.seqlen), flush=True)
    x, cp, dout = _case("bf16", s.batch, s.dim, s.seqlen, 4, seed=s.seed)
    g = _run(x, cp, dout, True, True, True)
    r = _oracle(x, cp, dout, True, True, True)
    _compare(g, r, "bf16", "conv bwd 2.8B-shaped layer")
    g2 = _run(x, cp, dout, True, True, True)
    for a, b in zip(g, g2):
        assert torch.equal(a, b), "repeat differs"
