"""The (batch, length, dim) layout (MSSM_FLAG_LAYOUT_BLD) of the forward scan,
the conv-fed scan, the backward and the causal conv, on the GPU through the C
ABI.  Inputs are the workloads' (batch, dim, L) draws transposed on the host;
outputs are transposed back and compared with the fp64 oracle under the same
bars as the (batch, dim, L) tests."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_common import DEV, check_out, check_state, np64, to_dev

pytestmark = pytest.mark.gpu


def _bld(t):
    """(batch, dim, L) CPU tensor -> (batch, L, dim) device tensor."""
    return None if t is None else t.transpose(1, 2).contiguous().to(DEV)


def _bdl(t):
    """(batch, L, dim) device tensor -> (batch, dim, L) CPU tensor."""
    return None if t is None else t.transpose(1, 2).contiguous().cpu()


def _report(what, worst):
    print("%-52s worst err/bar = %.3g (parity), %.3g (tight)" % (what, *worst), flush=True)


FWD = [
    # io, batch, dim, N, L, segments.  dim % 4 == 0 takes the channel-quad
    # vector path (dim 70: one element at a time); a dim that is not a
    # multiple of 64 leaves out-of-range quads in the last group
    ("bf16", 2, 96, 16, 300, 0),
    ("f32", 1, 70, 16, 77, 0),
    ("bf16", 1, 64, 16, 1000, 3),
    ("bf16", 2, 40, 64, 130, 0),
    ("f32", 1, 68, 16, 77, 0),
    ("bf16", 2, 128, 4, 333, 0),
    ("bf16", 1, 64, 1, 700, 2),
    ("f32", 2, 72, 8, 96, 3),
    ("bf16", 1, 100, 128, 70, 0),
]


@pytest.mark.parametrize("io,batch,dim,N,L,P", FWD,
                         ids=["%s-b%d-d%d-n%d-l%d-p%d" % c for c in FWD])
def test_forward_bld(io, batch, dim, N, L, P):
    import oracle
    import selective_state_space_52_amd as m
    s = W.spec("mamba130m_layer", io=io, batch=batch, dim=dim, dstate=N, seqlen=L,
               seed=900 + L)
    inp = W.make_scan_inputs(s)
    h0 = W.make_initial_state(s)
    last = to_dev(h0).clone()
    out = m.selective_scan_fwd(_bld(inp["u"]), _bld(inp["delta"]), to_dev(inp["A"]),
                               to_dev(inp["B"]), to_dev(inp["C"]), D=to_dev(inp["D"]),
                               z=_bld(inp["z"]), delta_bias=to_dev(inp["delta_bias"]),
                               last_state=last, load_state=True, time_segments=P,
                               layout="bld")
    torch.cuda.synchronize()
    ro, rl = oracle.scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                         D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"], h0=h0)
    _report("bld fwd %s" % ((io, batch, dim, N, L, P),), check_out(_bdl(out), ro, io, "out"))
    check_state(last.cpu(), rl, "last_state")


# io, batch, dim, N, L, optional operands left out
SAME = [
    ("bf16", 2, 128, 16, 256, ()),
    ("f32", 1, 68, 16, 77, ()),
    ("bf16", 1, 100, 4, 300, ("z",)),
    ("bf16", 1, 64, 1, 64, ("D", "delta_bias")),
    ("f32", 2, 72, 8, 96, ("z", "D", "delta_bias")),
    ("bf16", 1, 40, 128, 40, ()),
    # more workgroups than CUs: the (batch, dim, L) forward stages its
    # outputs through LDS before storing them
    ("bf16", 5, 3328, 16, 64, ()),
    ("f32", 5, 3328, 16, 40, ("z",)),
]


@pytest.mark.parametrize("io,batch,dim,N,L,drop", SAME,
                         ids=["%s-b%d-d%d-n%d-l%d-%s" % (*c[:5], "-".join(c[5]) or "all")
                              for c in SAME])
def test_forward_bld_equals_bdl(io, batch, dim, N, L, drop):
    """Without time segments, the two layouts do the same arithmetic on every
    element in the same order (only the lanes that load and store differ), so
    out and last_state are equal bit for bit; so is the (batch, L, dim) call
    through the one-element-at-a-time path (u offset by one element, so not
    aligned to 4 values)."""
    import selective_state_space_52_amd as m
    s = W.spec("mamba130m_layer", io=io, batch=batch, dim=dim, dstate=N, seqlen=L,
               seed=950 + L + N)
    inp = W.make_scan_inputs(s)
    for k in drop:
        inp[k] = None
    dv = {k: (to_dev(v) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    print("bld == bdl %s %s" % ((io, batch, dim, N, L), drop), flush=True)

    def run(layout, u, delta, z):
        last = torch.full((batch, dim, N), float("nan"), device=DEV)
        o = m.selective_scan_fwd(u, delta, dv["A"], dv["B"], dv["C"], D=dv["D"], z=z,
                                 delta_bias=dv["delta_bias"], last_state=last,
                                 time_segments=1, layout=layout)
        torch.cuda.synchronize()
        return o, last.cpu()

    ref, ref_last = run("bdl", dv["u"], dv["delta"], dv["z"])
    ub, db, zb = _bld(inp["u"]), _bld(inp["delta"]), _bld(inp["z"])
    got, got_last = run("bld", ub, db, zb)
    assert torch.equal(_bdl(got), ref.cpu()), "quad path out differs"
    assert torch.equal(got_last, ref_last), "quad path last_state differs"
    # the same u one element into a larger buffer: aligned to its element only
    buf = torch.empty(ub.numel() + 1, dtype=ub.dtype, device=DEV)
    ue = buf[1:].view(ub.shape)
    ue.copy_(ub)
    got, got_last = run("bld", ue, db, zb)
    assert torch.equal(_bdl(got), ref.cpu()), "element path out differs"
    assert torch.equal(got_last, ref_last), "element path last_state differs"


def test_conv_and_fused_bld():
    import oracle
    import selective_state_space_52_amd as m
    s = W.spec("mamba130m_layer", batch=2, dim=80, seqlen=264, seed=911)
    inp = W.make_scan_inputs(s)
    cp = W.make_conv_params(s)
    u_ref = oracle.causal_conv1d(inp["u"], cp["weight"], cp["bias"], cp["init"])
    conv = m.causal_conv1d_fwd(_bld(inp["u"]), to_dev(cp["weight"]), to_dev(cp["bias"]),
                               to_dev(cp["init"]), layout="bld")
    torch.cuda.synchronize()
    _report("bld conv", check_out(_bdl(conv), u_ref, "bf16", "conv"))
    u_out = torch.empty_like(_bld(inp["u"]))
    out = m.selective_scan_fwd_conv(
        _bld(inp["u"]), to_dev(cp["weight"]), _bld(inp["delta"]), to_dev(inp["A"]),
        to_dev(inp["B"]), to_dev(inp["C"]), conv_bias=to_dev(cp["bias"]),
        conv_init=to_dev(cp["init"]), D=to_dev(inp["D"]), z=_bld(inp["z"]),
        delta_bias=to_dev(inp["delta_bias"]), u_out=u_out, layout="bld")
    torch.cuda.synchronize()
    ro, _ = oracle.scan(u_ref, inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                        z=inp["z"], delta_bias=inp["delta_bias"])
    _report("bld fused", check_out(_bdl(out), ro, "bf16", "fused out"))
    check_out(_bdl(u_out), u_ref, "bf16", "fused u_out")


@pytest.mark.parametrize("io,P", [("bf16", 0), ("f32", 3)])
def test_backward_bld(io, P):
    import oracle
    import selective_state_space_52_amd as m
    from tests.test_gpu_bwd import check_all
    s = W.spec("mamba130m_layer", io=io, batch=2, dim=70, seqlen=333, seed=920 + P)
    inp = W.make_scan_inputs(s)
    gr = W.make_scan_grads(s)
    g = m.selective_scan_bwd(_bld(inp["u"]), _bld(inp["delta"]), to_dev(inp["A"]),
                             to_dev(inp["B"]), to_dev(inp["C"]), _bld(gr["dout"]),
                             D=to_dev(inp["D"]), z=_bld(inp["z"]),
                             delta_bias=to_dev(inp["delta_bias"]),
                             dlast=to_dev(gr["dlast"]), want_dh0=True,
                             time_segments=P, layout="bld")
    torch.cuda.synchronize()
    g = {k: (None if v is None else (_bdl(v) if k in ("du", "ddelta", "dz") else v.cpu()))
         for k, v in g.items()}
    r = oracle.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], gr["dout"],
                        D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                        dlast=gr["dlast"])
    check_all(g, r, io, "bld bwd %s P=%d" % (io, P))
