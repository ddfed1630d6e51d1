"""The ALU issue-rate probes (mssm_valu_probe) compute the chains they claim
to time: every kind launches through the C-ABI and writes finite values, and
the fma and exp chains (kinds 0, 1 and 4) match a float64 emulation of the
same iterations.  The probes feed the ALU ceiling the bench reports, so a
probe whose loop did other work than described would mislead it."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

BLOCKS, ITERS = 4, 64


def seeds():
    lane = (np.arange(BLOCKS * 256) & 63).astype(np.float32)
    return (np.float32(0.5) + np.float32(1e-3) * lane).astype(np.float64)


def fma_chains(s0):
    c = s0[:, None] + np.arange(8, dtype=np.float64)
    for _ in range(ITERS):
        c = c * np.float64(np.float32(0.999)) + np.float64(np.float32(1e-3))
    return c.sum(axis=1)


def exp_chains(x):
    for _ in range(ITERS):
        x = np.exp2(-np.abs(x))
    return x


def run(kind):
    import selective_state_space_52_amd as m
    sink = torch.full((BLOCKS * 256,), float("nan"), device="cuda")
    print("valu probe kind %d, %d blocks, %d iterations" % (kind, BLOCKS, ITERS), flush=True)
    m.valu_probe(kind, BLOCKS, ITERS, sink)
    torch.cuda.synchronize()
    return sink.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("kind", [0, 1, 2, 3, 4])
def test_probe_writes_finite_values(kind):
    assert np.isfinite(run(kind)).all()


def test_probe_chains_match_emulation():
    s0 = seeds()
    np.testing.assert_allclose(run(0), fma_chains(s0), rtol=1e-5)
    e = exp_chains(s0[:, None] + np.arange(8, dtype=np.float64)).sum(axis=1)
    np.testing.assert_allclose(run(1), e, rtol=1e-5)
    both = fma_chains(s0) + exp_chains(s0) + exp_chains(s0 + 0.5)
    np.testing.assert_allclose(run(4), both, rtol=1e-5)
