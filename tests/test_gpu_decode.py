"""Single-token decode step on the GPU (through the C ABI) against the oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_common import (DEV, check_out, check_state, gpu_scan, np64,
                              to_dev)

pytestmark = pytest.mark.gpu


def _run_steps(s, steps, rows=None):
    """Run `steps` decode steps on the GPU (token ring of the spec) and the
    oracle on all rows (rows=None) or the listed (b, d) rows."""
    import oracle
    import selective_state_space_52_amd as m
    par = W.make_decode_params(s)
    toks = [W.make_decode_token(s, k) for k in range(min(s.tokens, steps))]
    dtoks = [{k: to_dev(v) for k, v in t.items()} for t in toks]
    toks64 = [{k: np64(v) for k, v in t.items()} for t in toks]
    par64 = {k: np64(v) for k, v in par.items()}
    state = to_dev(par["state"]).clone()
    A, D, bias = to_dev(par["A"]), to_dev(par["D"]), to_dev(par["dt_bias"])
    ref_state = np64(par["state"])
    if rows is not None:
        bi = np.array([r[0] for r in rows])
        di = np.array([r[1] for r in rows])
        ref_state = ref_state[bi, di][:, None, :]          # (R, 1, N)
    outs_g, outs_r = [], []
    for step in range(steps):
        t, dt_ = toks[step % len(toks)], dtoks[step % len(toks)]
        out = m.selective_state_update(state, dt_["x"], dt_["dt"], A, dt_["B"],
                                       dt_["C"], D=D, z=dt_["z"], dt_bias=bias,
                                       softplus=s.softplus)
        if rows is None:
            ro, ref_state = oracle.state_update(
                ref_state, t["x"], t["dt"], par["A"], t["B"], t["C"], D=par["D"],
                z=t["z"], dt_bias=par["dt_bias"], softplus=s.softplus)
            outs_g.append(out.cpu())
            outs_r.append(ro)
        else:
            # each sampled row as its own (batch 1, dim 1) problem
            t = toks64[step % len(toks)]
            ro = np.empty(len(rows))
            for i, (b, d) in enumerate(rows):
                o1, st1 = oracle.state_update(
                    ref_state[i:i + 1], t["x"][b:b + 1, d:d + 1],
                    t["dt"][b:b + 1, d:d + 1], par64["A"][d:d + 1], t["B"][b:b + 1],
                    t["C"][b:b + 1], D=par64["D"][d:d + 1], z=t["z"][b:b + 1, d:d + 1],
                    dt_bias=par64["dt_bias"][d:d + 1], softplus=s.softplus, nthreads=1)
                ro[i] = o1[0, 0]
                ref_state[i:i + 1] = st1
            if step in (0, steps // 2, steps - 1):
                oc = out.cpu()
                outs_g.append(torch.stack([oc[b, d] for b, d in rows]))
                outs_r.append(ro.copy())
    torch.cuda.synchronize()
    return state.cpu(), ref_state, outs_g, outs_r


@pytest.mark.parametrize("io,batch,dim,N", [("bf16", 3, 200, 16), ("f32", 2, 70, 16),
                                             ("bf16", 2, 64, 1), ("bf16", 2, 64, 4),
                                             ("f32", 5, 33, 8), ("bf16", 3, 100, 32),
                                             ("f32", 2, 70, 64), ("bf16", 2, 66, 128),
                                             # the row -> (batch, channel) split at
                                             # dim 1, just above a power of two, odd
                                             ("bf16", 7, 1, 16), ("bf16", 4, 4097, 16),
                                             ("f32", 3, 7777, 8)])
def test_decode_small(io, batch, dim, N):
    s = W.spec("decode", io=io, batch=batch, dim=dim, dstate=N, tokens=5)
    state, ref_state, og, orf = _run_steps(s, steps=12)
    for k, (g, r) in enumerate(zip(og, orf)):
        check_out(g, r, io, "decode out step %d" % k)
    check_state(state, ref_state, "decode state")


@pytest.mark.parametrize("N", [16, 64])
def test_decode_iterated_equals_gpu_scan(N):
    """L decode steps reproduce the forward scan's outputs and final state."""
    import selective_state_space_52_amd as m
    s = W.spec("mamba130m_layer", batch=2, dim=96, dstate=N, seqlen=40, seed=9)
    inp = W.make_scan_inputs(s)
    h0 = W.make_initial_state(s)
    out, last = gpu_scan(inp, h0=h0)
    state = to_dev(h0).clone()
    d = {k: to_dev(v) if isinstance(v, torch.Tensor) else v for k, v in inp.items()}
    ys = []
    for t in range(s.seqlen):
        ys.append(m.selective_state_update(
            state, d["u"][..., t].contiguous(), d["delta"][..., t].contiguous(),
            d["A"], d["B"][:, t].contiguous(), d["C"][:, t].contiguous(), D=d["D"],
            z=d["z"][..., t].contiguous(), dt_bias=d["delta_bias"]).cpu())
    torch.cuda.synchronize()
    dec = torch.stack(ys, dim=-1)
    check_out(dec, np64(out), "bf16", "decode vs scan", ref_rounded=True)
    check_state(state.cpu(), np64(last), "decode vs scan state")


def test_decode_full_size_1000_steps():
    """The decode workload (256 sequences x D 5120, N 16) for 1000 steps, each
    on one in-place state; the oracle follows every row, and every output and
    every state element is compared after steps 1, 500 and 1000."""
    import oracle
    import selective_state_space_52_amd as m
    s = W.spec("decode")
    print("decode full size: %d x %d, N %d, %d steps" % (s.batch, s.dim, s.dstate,
                                                         s.steps), flush=True)
    par = W.make_decode_params(s)
    toks = [W.make_decode_token(s, k) for k in range(s.tokens)]
    dtoks = [{k: to_dev(v) for k, v in t.items()} for t in toks]
    toks64 = [{k: np64(v) for k, v in t.items()} for t in toks]
    par64 = {k: np64(v) for k, v in par.items()}
    state = to_dev(par["state"]).clone()
    A, D, bias = to_dev(par["A"]), to_dev(par["D"]), to_dev(par["dt_bias"])
    ref_state = par64["state"]
    checks = {1, s.steps // 2, s.steps}
    done = 0
    for step in range(1, s.steps + 1):
        t, dt_ = toks64[(step - 1) % len(toks)], dtoks[(step - 1) % len(toks)]
        out = m.selective_state_update(state, dt_["x"], dt_["dt"], A, dt_["B"], dt_["C"],
                                       D=D, z=dt_["z"], dt_bias=bias, softplus=s.softplus)
        ro, ref_state = oracle.state_update(
            ref_state, t["x"], t["dt"], par64["A"], t["B"], t["C"], D=par64["D"],
            z=t["z"], dt_bias=par64["dt_bias"], softplus=s.softplus)
        if step in checks:
            check_out(out.cpu(), ro, "bf16", "decode out after step %d" % step)
            check_state(state.cpu(), ref_state, "decode state after step %d" % step)
            done += 1
            print("decode step %d: every row within the bars" % step, flush=True)
    assert done == 3


def test_decode_64bit_indices():
    """4100 x 4096 rows of 128 states: 2.15e9 state elements (8.6 GB), past
    2^31, so the launch takes 64-bit indices.  Rows on both sides of element
    2^31 and at the ends follow the oracle."""
    import oracle
    import selective_state_space_52_amd as m
    batch, dim, N = 4100, 4096, 128
    assert batch * dim * N > 2 ** 31
    print("decode 64-bit indices: batch %d dim %d N %d" % (batch, dim, N), flush=True)
    t = W.make_large_decode_step(batch, dim, N, device=DEV)
    rng = np.random.default_rng(12)
    rows = [(0, 0), (0, 4095), (4095, 4095), (4096, 0), (4096, 1), (4097, 17),
            (4099, 4095)] + [(int(b), int(d)) for b, d in
                             zip(rng.integers(4090, 4100, 9), rng.integers(0, 4096, 9))]
    bi = torch.tensor([b for b, _ in rows], device=DEV)
    di = torch.tensor([d for _, d in rows], device=DEV)
    h_before = np64(t["state"][bi, di].cpu())
    out = m.selective_state_update(t["state"], t["x"], t["dt"], t["A"], t["B"], t["C"],
                                   D=t["D"], z=t["z"], dt_bias=t["dt_bias"])
    torch.cuda.synchronize()
    got_out = out[bi, di].cpu()
    got_state = t["state"][bi, di].cpu()
    A, D, bias = np64(t["A"].cpu()), np64(t["D"].cpu()), np64(t["dt_bias"].cpu())
    tok = {k: np64(t[k][bi, di].cpu()) for k in ("x", "dt", "z")}
    Bs, Cs = np64(t["B"][bi].cpu()), np64(t["C"][bi].cpu())
    ref_out = np.empty(len(rows))
    ref_state = np.empty((len(rows), N))
    for i, (b, d) in enumerate(rows):
        o1, st1 = oracle.state_update(
            h_before[i:i + 1, None, :], tok["x"][i:i + 1, None], tok["dt"][i:i + 1, None],
            A[d:d + 1], Bs[i:i + 1], Cs[i:i + 1], D=D[d:d + 1], z=tok["z"][i:i + 1, None],
            dt_bias=bias[d:d + 1], softplus=True, nthreads=1)
        ref_out[i] = o1[0, 0]
        ref_state[i] = st1[0, 0]
    del t
    check_out(got_out, ref_out, "bf16", "decode 64-bit indices out")
    check_state(got_state, ref_state, "decode 64-bit indices state")


def test_decode_graph_replays_match_eager():
    """Decode steps captured in one HIP graph (as the bench replays its
    rotating loop): each of several replays, with eager launches and
    synchronisations between them, gives the bit-identical outputs and states
    of the same steps run eagerly from the same starting states."""
    import selective_state_space_52_amd as m
    s = W.spec("decode", batch=8, dim=640, tokens=3)
    par = W.make_decode_params(s)
    toks = [{k: to_dev(v) for k, v in W.make_decode_token(s, k).items()}
            for k in range(s.tokens)]
    A, D, bias = to_dev(par["A"]), to_dev(par["D"]), to_dev(par["dt_bias"])
    states = [to_dev(par["state"]).clone() for _ in range(2)]
    outs = [torch.empty(s.batch, s.dim, dtype=torch.bfloat16, device=DEV) for _ in range(6)]
    steps = 6

    def run():
        for i in range(steps):
            t = toks[i % len(toks)]
            m.selective_state_update(states[i % 2], t["x"], t["dt"], A, t["B"], t["C"], D=D,
                                     z=t["z"], dt_bias=bias, out=outs[i])

    graph = torch.cuda.CUDAGraph()
    start = [st.clone() for st in states]
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        begin = [st.clone() for st in states]
        graph.replay()
        torch.cuda.synchronize()
        g_outs = [o.clone() for o in outs]
        g_states = [st.clone() for st in states]
        # the same steps eagerly from the same starting states
        for st, b0 in zip(states, begin):
            st.copy_(b0)
        run()
        torch.cuda.synchronize()
        for k in range(steps):
            assert torch.equal(g_outs[k], outs[k]), "replay %d, step %d out" % (rep, k)
        for k in range(2):
            assert torch.equal(g_states[k], states[k]), "replay %d, state %d" % (rep, k)
        # eager work between replays: a plain call on another state
        scratch_state = start[0].clone()
        t = toks[0]
        m.selective_state_update(scratch_state, t["x"], t["dt"], A, t["B"], t["C"], D=D,
                                 z=t["z"], dt_bias=bias)
        torch.cuda.synchronize()
    del graph


@pytest.mark.parametrize("io,batch,dim,N", [("bf16", 3, 200, 16), ("f32", 2, 70, 4),
                                             ("bf16", 2, 66, 128), ("f32", 5, 33, 8)])
def test_decode_stream_state_hint(io, batch, dim, N):
    """The streaming hint (MSSM_FLAG_STATE_STREAM: non-temporal loads and
    stores of the state) gives the same bits as the default, step after step,
    and both match the oracle."""
    import oracle
    import selective_state_space_52_amd as m
    s = W.spec("decode", io=io, batch=batch, dim=dim, dstate=N, tokens=4, seed=61)
    par = W.make_decode_params(s)
    toks = [W.make_decode_token(s, k) for k in range(s.tokens)]
    dtoks = [{k: to_dev(v) for k, v in t.items()} for t in toks]
    A, D, bias = to_dev(par["A"]), to_dev(par["D"]), to_dev(par["dt_bias"])
    st_a = to_dev(par["state"]).clone()
    st_b = to_dev(par["state"]).clone()
    ref_state = np64(par["state"])
    print("stream hint %s batch %d dim %d N %d" % (io, batch, dim, N), flush=True)
    for step in range(6):
        t, d = toks[step % len(toks)], dtoks[step % len(toks)]
        oa = m.selective_state_update(st_a, d["x"], d["dt"], A, d["B"], d["C"], D=D,
                                      z=d["z"], dt_bias=bias)
        ob = m.selective_state_update(st_b, d["x"], d["dt"], A, d["B"], d["C"], D=D,
                                      z=d["z"], dt_bias=bias, stream_state=True)
        ro, ref_state = oracle.state_update(
            ref_state, t["x"], t["dt"], par["A"], t["B"], t["C"], D=par["D"],
            z=t["z"], dt_bias=par["dt_bias"], softplus=s.softplus)
        torch.cuda.synchronize()
        assert torch.equal(oa.cpu(), ob.cpu()), "step %d out differs" % step
        assert torch.equal(st_a.cpu(), st_b.cpu()), "step %d state differs" % step
        check_out(ob.cpu(), ro, io, "decode stream out step %d" % step)
    check_state(st_b.cpu(), ref_state, "decode stream state")
