"""B/C groups (mssm_dims.ngroups): B, C hold G vectors per token and channel
d reads group d // (dim // G).  Forward, conv-fed forward, backward and decode
on the GPU through the C ABI against the fp64 oracle (same bars as the
one-group tests)."""
import pytest
import torch

import workloads as W
from tests.gpu_common import DEV, check_out, check_state, np64, to_dev

pytestmark = pytest.mark.gpu


def _report(what, worst):
    print("%-52s worst err/bar = %.3g (parity), %.3g (tight)" % (what, *worst), flush=True)


def _case(G, **over):
    s = W.spec("mamba130m_layer", **over)
    inp = W.make_scan_inputs(s)
    inp.update(W.make_group_bc(s, G))
    return s, inp


FWD = [
    # io, batch, dim, N, L, G, segments, layout
    ("bf16", 2, 256, 16, 300, 2, 0, "bdl"),
    ("f32", 1, 192, 16, 77, 3, 0, "bdl"),
    ("bf16", 1, 256, 16, 1000, 4, 3, "bdl"),
    ("bf16", 2, 128, 64, 200, 2, 0, "bdl"),
    ("bf16", 2, 128, 16, 130, 2, 0, "bld"),
]


@pytest.mark.parametrize("io,batch,dim,N,L,G,P,layout", FWD,
                         ids=["%s-b%d-d%d-n%d-l%d-g%d-p%d-%s" % c for c in FWD])
def test_forward_groups(io, batch, dim, N, L, G, P, layout):
    import oracle
    import selective_state_space_52_amd as m
    s, inp = _case(G, io=io, batch=batch, dim=dim, dstate=N, seqlen=L, seed=1000 + L + G)
    h0 = W.make_initial_state(s)
    last = to_dev(h0).clone()
    tr = (lambda t: t.transpose(1, 2).contiguous()) if layout == "bld" else (lambda t: t)
    out = m.selective_scan_fwd(to_dev(tr(inp["u"])), to_dev(tr(inp["delta"])),
                               to_dev(inp["A"]), to_dev(inp["B"]), to_dev(inp["C"]),
                               D=to_dev(inp["D"]), z=to_dev(tr(inp["z"])),
                               delta_bias=to_dev(inp["delta_bias"]), last_state=last,
                               load_state=True, time_segments=P, layout=layout)
    torch.cuda.synchronize()
    ro, rl = oracle.scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                         D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"], h0=h0)
    _report("groups fwd %s" % ((io, batch, dim, N, L, G, P, layout),),
            check_out(tr(out.cpu()), ro, io, "out"))
    check_state(last.cpu(), rl, "last_state")


def test_fused_conv_groups():
    import oracle
    import selective_state_space_52_amd as m
    s, inp = _case(2, batch=2, dim=128, seqlen=264, seed=1111)
    cp = W.make_conv_params(s)
    out = m.selective_scan_fwd_conv(
        to_dev(inp["u"]), to_dev(cp["weight"]), to_dev(inp["delta"]), to_dev(inp["A"]),
        to_dev(inp["B"]), to_dev(inp["C"]), conv_bias=to_dev(cp["bias"]),
        conv_init=to_dev(cp["init"]), D=to_dev(inp["D"]), z=to_dev(inp["z"]),
        delta_bias=to_dev(inp["delta_bias"]))
    torch.cuda.synchronize()
    u = oracle.causal_conv1d(inp["u"], cp["weight"], cp["bias"], cp["init"])
    ro, _ = oracle.scan(u, inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                        z=inp["z"], delta_bias=inp["delta_bias"])
    _report("groups fused conv", check_out(out.cpu(), ro, "bf16", "out"))


@pytest.mark.parametrize("io,dim,G,P", [("bf16", 256, 4, 0), ("f32", 128, 2, 3)])
def test_backward_groups(io, dim, G, P):
    import oracle
    import selective_state_space_52_amd as m
    from tests.test_gpu_bwd import check_all
    s, inp = _case(G, io=io, batch=2, dim=dim, seqlen=200, seed=1200 + G)
    gr = W.make_scan_grads(s)
    g = m.selective_scan_bwd(to_dev(inp["u"]), to_dev(inp["delta"]), to_dev(inp["A"]),
                             to_dev(inp["B"]), to_dev(inp["C"]), to_dev(gr["dout"]),
                             D=to_dev(inp["D"]), z=to_dev(inp["z"]),
                             delta_bias=to_dev(inp["delta_bias"]),
                             dlast=to_dev(gr["dlast"]), want_dh0=True, time_segments=P)
    torch.cuda.synchronize()
    g = {k: (None if v is None else v.cpu()) for k, v in g.items()}
    r = oracle.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], gr["dout"],
                        D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                        dlast=gr["dlast"])
    check_all(g, r, io, "groups bwd %s G=%d P=%d" % (io, G, P))


@pytest.mark.parametrize("io,batch,dim,N,G", [("bf16", 3, 96, 16, 4), ("f32", 2, 40, 64, 2)])
def test_decode_groups(io, batch, dim, N, G):
    import oracle
    import selective_state_space_52_amd as m
    s = W.spec("decode", io=io, batch=batch, dim=dim, dstate=N, tokens=1)
    par = W.make_decode_params(s)
    tok = W.make_decode_token(s, 0)
    gs = W.spec("mamba130m_layer", io=io, batch=batch, dim=dim, dstate=N, seqlen=1)
    bc = W.make_group_bc(gs, G)
    B, C = bc["B"][:, 0], bc["C"][:, 0]          # (batch, G, N)
    state = to_dev(par["state"]).clone()
    out = m.selective_state_update(state, to_dev(tok["x"]), to_dev(tok["dt"]),
                                   to_dev(par["A"]), to_dev(B), to_dev(C),
                                   D=to_dev(par["D"]), z=to_dev(tok["z"]),
                                   dt_bias=to_dev(par["dt_bias"]))
    torch.cuda.synchronize()
    ro, rs = oracle.state_update(par["state"], tok["x"], tok["dt"], par["A"], B, C,
                                 D=par["D"], z=tok["z"], dt_bias=par["dt_bias"])
    _report("groups decode %s" % ((io, batch, dim, N, G),), check_out(out.cpu(), ro, io, "out"))
    check_state(state.cpu(), rs, "state")


@pytest.mark.parametrize("groups", [1, 2])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_state_major_bc_layout(io, groups):
    """B and C given state-major, (batch, [G,] N, L), give bit for bit the
    token-major call's forward outputs and final state, and the backward's
    gradients with dB and dC in the state-major layout; both against the
    oracle."""
    import oracle
    import selective_state_space_52_amd as m
    s = W.spec("mamba130m_layer", io=io, batch=2, dim=128 * groups, seqlen=300, seed=61 + groups)
    inp = W.make_scan_inputs(s)
    if groups > 1:
        inp.update(W.make_group_bc(s, groups))
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    if groups > 1:
        Bs = d["B"].permute(0, 2, 3, 1).contiguous()    # (batch, G, N, L)
        Cs = d["C"].permute(0, 2, 3, 1).contiguous()
    else:
        Bs = d["B"].transpose(1, 2).contiguous()        # (batch, N, L)
        Cs = d["C"].transpose(1, 2).contiguous()
    outs = {}
    for lay, Bx, Cx in (("token", d["B"], d["C"]), ("state", Bs, Cs)):
        last = torch.empty(s.batch, s.dim, s.dstate, device=DEV)
        o = m.selective_scan_fwd(d["u"], d["delta"], d["A"], Bx, Cx, D=d["D"], z=d["z"],
                                 delta_bias=d["delta_bias"], last_state=last,
                                 bc_layout=lay)
        g = m.selective_scan_bwd(d["u"], d["delta"], d["A"], Bx, Cx, d["u"], D=d["D"],
                                 z=d["z"], delta_bias=d["delta_bias"], bc_layout=lay)
        torch.cuda.synchronize()
        outs[lay] = (o.cpu(), last.cpu(), {k: v.cpu() for k, v in g.items() if v is not None})
    (o_t, l_t, g_t), (o_s, l_s, g_s) = outs["token"], outs["state"]
    assert torch.equal(o_t, o_s) and torch.equal(l_t, l_s)
    for k in g_t:
        if k in ("dB", "dC"):
            back = g_s[k].permute(0, 3, 1, 2) if groups > 1 else g_s[k].transpose(1, 2)
            assert torch.equal(g_t[k], back.contiguous()), k
        else:
            assert torch.equal(g_t[k], g_s[k]), k
    ro, rl = oracle.scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                         z=inp["z"], delta_bias=inp["delta_bias"])
    check_out(o_s, ro, io, "state-major out")
    check_state(l_s, rl, "state-major last_state")
