"""Forward scan on the GPU (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_common import (DEV, check_out, check_state, gpu_scan, np64,
                              oracle_scan)

pytestmark = pytest.mark.gpu


def _inputs(name, **over):
    return W.make_scan_inputs(W.spec(name, **over))


def _report(what, worst):
    print("%-48s worst err/bar = %.3g (parity), %.3g (tight)" % (what, *worst), flush=True)


def test_tiny_fp32_full():
    """The tiny fp32 workload (batch 1, D 64, N 16, L 256), every output."""
    inp = _inputs("tiny_f32")
    out, last = gpu_scan(inp)
    ro, rl = oracle_scan(inp)
    _report("tiny_f32 out", check_out(out, ro, "f32", "tiny out"))
    check_state(last, rl, "tiny last_state")


SHAPES = [
    # io, batch, dim, N, L   -- several tiles, ragged channel groups and tails
    ("bf16", 3, 128, 16, 256),    # vector path, whole tiles
    ("bf16", 2, 100, 16, 333),    # element path, ragged group and tile
    ("bf16", 2, 130, 16, 1000),   # vector path, ragged last tile
    ("f32", 1, 64, 16, 257),      # fp32 element path
    ("f32", 2, 70, 16, 264),      # fp32 vector path
    ("bf16", 1, 64, 16, 1),
    ("bf16", 1, 64, 16, 7),
    ("bf16", 1, 64, 16, 63),
    ("bf16", 1, 64, 16, 64),
    ("bf16", 1, 64, 16, 65),
    ("bf16", 1, 5, 16, 40),       # fewer channels than a wave
    ("bf16", 1, 64, 16, 8),       # shortest vector-path row: one ragged tile
    ("bf16", 2, 64, 8, 8),        # the same with 8-step chunks
    ("bf16", 2, 96, 32, 296),     # N = 32 on the vector path, ragged last tile
    ("bf16", 2, 96, 1, 200),
    ("bf16", 2, 96, 2, 200),
    ("bf16", 2, 96, 4, 200),
    ("bf16", 2, 96, 8, 200),
    ("f32", 2, 33, 8, 77),
    # larger states (Mamba-2 sizes): 8 waves, N / 8 states per wave
    ("bf16", 2, 96, 32, 300),
    ("f32", 1, 64, 64, 264),
    ("bf16", 2, 64, 64, 1000),
    ("bf16", 1, 70, 128, 200),
    ("f32", 1, 40, 128, 77),      # fp32 N = 128: a token's B/C run spans 2 batches
]


@pytest.mark.parametrize("io,batch,dim,N,L", SHAPES,
                         ids=["%s-b%d-d%d-n%d-l%d" % s for s in SHAPES])
def test_shapes(io, batch, dim, N, L):
    inp = _inputs("mamba130m_layer", io=io, batch=batch, dim=dim, dstate=N,
                  seqlen=L, seed=100 + L + N)
    out, last = gpu_scan(inp)
    ro, rl = oracle_scan(inp)
    _report("shape %s" % ((io, batch, dim, N, L),), check_out(out, ro, io, "out"))
    check_state(last, rl, "last_state")


VARIANTS = [
    dict(has_z=False), dict(has_D=False), dict(has_bias=False),
    dict(softplus=False, has_bias=False), dict(has_z=False, has_D=False, has_bias=False),
]


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("var", VARIANTS, ids=lambda v: ",".join("%s=%s" % kv for kv in v.items()))
def test_optional_operands(io, var):
    inp = _inputs("mamba130m_layer", io=io, batch=2, dim=80, seqlen=136, seed=7, **var)
    if not var.get("softplus", True):
        # raw steps must stay positive without softplus: use |delta| * 0.05
        inp["delta"] = (inp["delta"].float().abs() * 0.05).to(inp["delta"].dtype)
    out, last = gpu_scan(inp)
    ro, rl = oracle_scan(inp)
    _report("variant %s %s" % (io, var), check_out(out, ro, io, "out"))
    check_state(last, rl, "last_state")


@pytest.mark.parametrize("L,ts", [(1000, 2), (1000, 3), (999, 7), (2048, 5), (200, 9)])
def test_forced_time_segments(L, ts):
    """Rows cut into time segments joined by the carried state (aggregate
    tasks publish each segment's summary, later segments fold them into
    their entering state) give the oracle's result."""
    inp = _inputs("mamba130m_layer", batch=2, dim=72, seqlen=L, seed=L + ts)
    h0 = W.make_initial_state(W.spec("mamba130m_layer", batch=2, dim=72))
    out, last = gpu_scan(inp, h0=h0, time_segments=ts)
    ro, rl = oracle_scan(inp, h0=h0.double().numpy())
    _report("segments L=%d ts=%d" % (L, ts), check_out(out, ro, "bf16", "out"))
    check_state(last, rl, "last_state")


@pytest.mark.parametrize("io,N", [("bf16", 64), ("f32", 128)])
def test_forced_time_segments_large_state(io, N):
    """The segment carry with 8 states (16) per wave."""
    s = W.spec("mamba130m_layer", io=io, batch=1, dim=72, dstate=N, seqlen=700, seed=N)
    inp = W.make_scan_inputs(s)
    h0 = W.make_initial_state(s)
    out, last = gpu_scan(inp, h0=h0, time_segments=3)
    ro, rl = oracle_scan(inp, h0=h0.double().numpy())
    _report("segments N=%d %s" % (N, io), check_out(out, ro, io, "out"))
    check_state(last, rl, "last_state")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_load_state_chaining(io):
    """Consecutive calls carrying last_state reproduce one call (the resume
    path), and both match the oracle."""
    inp = _inputs("mamba130m_layer", io=io, batch=2, dim=64, seqlen=600, seed=3)
    full, full_last = gpu_scan(inp)
    cuts = [0, 1, 97, 352, 600]
    state = torch.zeros(2, 64, 16)
    pieces = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        part = dict(inp, u=inp["u"][..., a:b].contiguous(),
                    delta=inp["delta"][..., a:b].contiguous(),
                    z=inp["z"][..., a:b].contiguous(),
                    B=inp["B"][:, a:b].contiguous(), C=inp["C"][:, a:b].contiguous())
        o, state = gpu_scan(part, h0=state)
        pieces.append(o)
    chained = torch.cat(pieces, dim=-1)
    ro, rl = oracle_scan(inp)
    check_out(chained, ro, io, "chained out")
    check_state(state, rl, "chained last_state")
    check_out(full, ro, io, "full out")
    check_state(full_last, rl, "full last_state")


def test_determinism():
    inp = _inputs("mamba130m_layer", batch=2, dim=192, seqlen=512, seed=5)
    o1, l1 = gpu_scan(inp)
    o2, l2 = gpu_scan(inp)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["mamba130m_layer", "mamba2p8b_layer"])
def test_full_size_every_element(name):
    """Full-size layer workloads in the launch configuration the bench times
    (at the 2.8B-shaped layer on 256 CUs: 256 whole channel groups and 64
    groups cut into time segments, all in one launch),
    every output and every final state against the oracle; then a second and
    a third call must reproduce the first bit for bit."""
    import selective_state_space_52_amd as m
    s = W.spec(name)
    print("full size %s: batch %d dim %d N %d L %d" % (name, s.batch, s.dim, s.dstate,
                                                    s.seqlen), flush=True)
    plan = m.scan_plan(s.batch, s.dim, s.dstate, s.seqlen)
    print("plan", plan, flush=True)
    if name == "mamba2p8b_layer" and torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert plan["whole_groups"] == 256 and plan["split_groups"] == 64
    inp = W.make_scan_inputs(s)
    out, last = gpu_scan(inp)
    ro, rl = oracle_scan(inp)
    _report("%s every element" % name, check_out(out, ro, "bf16", name))
    check_state(last, rl, name + " last_state")
    for k in range(2):
        o2, l2 = gpu_scan(inp)
        assert torch.equal(o2, out) and torch.equal(l2, last), "repeat %d differs" % (k + 1)


def test_split_plan_small():
    """A shape small enough for the oracle in a second that still takes the
    bench's kind of plan: 5 x 3328 channels = 260 groups of 64, so on 256
    CUs 256 groups run whole and 4 are cut into time segments whose
    aggregates publish summaries that the later segments wait for, in the
    same launch.  Every element against the oracle, a loaded initial state
    (read by the first aggregate and the first segment), and repeat calls
    bit for bit."""
    import selective_state_space_52_amd as m
    batch, dim, N, L = 5, 3328, 16, 1024
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = m.scan_plan(batch, dim, N, L)
    print("split plan on %d CUs: %s" % (cus, plan), flush=True)
    if cus == 256:
        assert plan["whole_groups"] == 256 and plan["split_groups"] == 4
        assert plan["segments"] >= 2
    s = W.spec("mamba130m_layer", batch=batch, dim=dim, seqlen=L, seed=260)
    inp = W.make_scan_inputs(s)
    h0 = W.make_initial_state(s)
    out, last = gpu_scan(inp, h0=h0)
    ro, rl = oracle_scan(inp, h0=h0.double().numpy())
    _report("split plan every element", check_out(out, ro, "bf16", "out"))
    check_state(last, rl, "last_state")
    for k in range(3):
        o2, l2 = gpu_scan(inp, h0=h0)
        assert torch.equal(o2, out) and torch.equal(l2, last), "repeat %d differs" % (k + 1)


def test_long_sequence_split_vs_unsplit():
    """Long sequence (batch 1, D 1536, N 16, L 131072): one call (rows cut into
    time segments inside the library) against 64 chained calls of 2048 steps
    carrying last_state, both against the oracle on every element."""
    s = W.spec("long_chunked")
    print("long sequence: dim %d L %d" % (s.dim, s.seqlen), flush=True)
    inp = W.make_scan_inputs(s)
    out, last = gpu_scan(inp)
    state = torch.zeros(1, s.dim, s.dstate)
    pieces = []
    for a in range(0, s.seqlen, s.chunk):
        b = a + s.chunk
        part = dict(inp, u=inp["u"][..., a:b].contiguous(),
                    delta=inp["delta"][..., a:b].contiguous(),
                    z=inp["z"][..., a:b].contiguous(),
                    B=inp["B"][:, a:b].contiguous(), C=inp["C"][:, a:b].contiguous())
        o, state = gpu_scan(part, h0=state)
        pieces.append(o)
    chunked = torch.cat(pieces, dim=-1)
    ro, rl = oracle_scan(inp)
    for got, lab in ((out, "one call"), (chunked, "chunked")):
        _report("long %s every element" % lab, check_out(got, ro, "bf16", lab))
    check_state(last, rl, "one-call last_state")
    check_state(state, rl, "chunked last_state")
    # split vs unsplit over every row
    check_state(last, np64(state), "split vs unsplit last_state")
    diff = (out.float() - chunked.float()).abs()
    assert float((diff / (2e-2 * (1 + chunked.float().abs()))).max()) <= 1.0


def test_softplus_relative_accuracy():
    """Delta itself, through the scan and the decode step: with A = 0, one
    state, B = C = u = 1 and no skip or gate, out = softplus(delta).  Checks
    the relative error of the kernels' softplus over delta in [-80, 40],
    where the absolute parity bar would not see errors on tiny Delta.  The
    bound allows the fp32 rounding of -|x| log2(e) (about 6e-8 |x| relative
    in e^-|x|) plus a few units of the last place."""
    import oracle
    import selective_state_space_52_amd as m
    n = 8192
    x = torch.linspace(-80.0, 40.0, n, dtype=torch.float32)
    one = torch.ones(1, n, 1, dtype=torch.float32)
    A = torch.zeros(n, 1, dtype=torch.float32)
    inp = {"u": one.clone(), "delta": x.reshape(1, n, 1), "A": A,
           "B": torch.ones(1, 1, 1), "C": torch.ones(1, 1, 1), "D": None, "z": None,
           "delta_bias": None, "softplus": True}
    ref, _ = oracle_scan(inp)
    ref = np.asarray(ref, dtype=np.float64).reshape(n)
    bound = (5e-7 + 1e-7 * np.abs(np64(x))) * ref
    out, _ = gpu_scan(inp, want_state=False)
    err = np.abs(np64(out).reshape(n) - ref)
    _report("softplus via scan, rel err/bound", (float((err / bound).max()), 0.0))
    assert (err <= bound).all(), "scan softplus off at delta=%g" % float(x[int(np.argmax(err / bound))])
    # the decode step: state 0 -> state = out = Delta
    state = torch.zeros(1, n, 1, device=DEV)
    out = m.selective_state_update(state, torch.ones(1, n, device=DEV), x.reshape(1, n).to(DEV),
                                   A.to(DEV), torch.ones(1, 1, device=DEV),
                                   torch.ones(1, 1, device=DEV), softplus=True)
    torch.cuda.synchronize()
    for what, got in (("out", out), ("state", state)):
        err = np.abs(np64(got).reshape(n) - ref)
        assert (err <= bound).all(), "decode softplus (%s) off at delta=%g" % (
            what, float(x[int(np.argmax(err / bound))]))


def test_forward_64bit_element_offsets():
    """A forward call of more than 2^31 elements (batch 2 x 36864 channels x
    32768 steps), so row offsets pass 2^31: every step of sampled rows on both
    sides of element 2^31 -- which are also the first rows of the groups the
    plan cuts in time -- the first and last rows, against the oracle."""
    import oracle
    import selective_state_space_52_amd as m
    batch, dim, L, N = 2, 36864, 32768, 16
    assert batch * dim * L > 2 ** 31
    plan = m.scan_plan(batch, dim, N, L)
    print("forward 64-bit offsets: batch %d dim %d L %d plan %s" % (batch, dim, L, plan),
          flush=True)
    d = W.make_large_scan_inputs(batch, dim, L, N, device=DEV)
    last = torch.full((batch, dim, N), float("nan"), device=DEV)
    out = m.selective_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                               z=d["z"], delta_bias=d["delta_bias"], last_state=last)
    torch.cuda.synchronize()
    r0 = 2 ** 31 // L                     # first row past element 2^31
    rows = sorted({0, r0 - 65, r0 - 1, r0, r0 + 1, r0 + 63, r0 + 64, r0 + 4000,
                   batch * dim - 1})
    for r in rows:
        b, c = divmod(r, dim)
        ro, rl = oracle.scan(d["u"][b:b + 1, c:c + 1].cpu(), d["delta"][b:b + 1, c:c + 1].cpu(),
                             d["A"][c:c + 1].cpu(), d["B"][b:b + 1].cpu(), d["C"][b:b + 1].cpu(),
                             D=d["D"][c:c + 1].cpu(), z=d["z"][b:b + 1, c:c + 1].cpu(),
                             delta_bias=d["delta_bias"][c:c + 1].cpu(), softplus=True)
        check_out(out[b:b + 1, c:c + 1].cpu(), ro, "bf16", "row %d out" % r)
        check_state(last[b:b + 1, c:c + 1].cpu(), rl, "row %d last_state" % r)
    del d, out, last
    torch.cuda.empty_cache()
