"""Seeded input generator: determinism, rounding and value ranges (CPU)."""
import math

import numpy as np
import torch

import workloads as W


def test_same_seed_same_bytes():
    s = W.spec("tiny_f32")
    a, b = W.make_scan_inputs(s), W.make_scan_inputs(s)
    for k in ("u", "delta", "z", "B", "C", "A", "D", "delta_bias"):
        assert torch.equal(a[k], b[k]), k


def test_shapes_and_dtypes():
    s = W.spec("mamba130m_layer", batch=2, dim=16, seqlen=40)
    x = W.make_scan_inputs(s)
    assert x["u"].shape == (2, 16, 40) and x["u"].dtype == torch.bfloat16
    assert x["B"].shape == (2, 40, 16) and x["C"].dtype == torch.bfloat16
    assert x["A"].shape == (16, 16) and x["A"].dtype == torch.float32
    assert x["D"].dtype == torch.float32 and x["delta_bias"].shape == (16,)


def test_bf16_is_round_to_nearest_even_of_the_fp32_draw():
    s = W.spec("mamba130m_layer", batch=1, dim=8, seqlen=64)
    x = W.make_scan_inputs(s)
    rng = np.random.default_rng(s.seed)
    u32 = rng.standard_normal((1, 8, 64), dtype=np.float32)
    # round to nearest even on the bit pattern, written out independently
    bits = u32.view(np.uint32).astype(np.uint64)
    rnd = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    want = rnd.astype(np.uint32).view(np.float32)
    assert np.array_equal(x["u"].float().numpy(), want)


def test_parameter_recipe():
    s = W.spec("mamba2p8b_layer", batch=1, dim=512, seqlen=8)
    x = W.make_scan_inputs(s)
    A = x["A"].numpy()
    assert np.array_equal(A, -(np.arange(16) + 1.0)[None, :].repeat(512, 0))
    # softplus(bias) lands in the dt range [1e-3, 1e-1]
    dt = np.logaddexp(0.0, x["delta_bias"].double().numpy())
    assert dt.min() >= 1e-3 * (1 - 1e-5) and dt.max() <= 1e-1 * (1 + 1e-5)
    assert math.log(dt.max() / dt.min()) > 3.5   # spans the log-uniform range


def test_decode_tokens_distinct_and_deterministic():
    s = W.spec("decode", batch=4, dim=64)
    t0, t1 = W.make_decode_token(s, 0), W.make_decode_token(s, 1)
    assert not torch.equal(t0["x"], t1["x"])
    assert torch.equal(t0["x"], W.make_decode_token(s, 0)["x"])
    p = W.make_decode_params(s)
    assert p["state"].shape == (4, 64, 16)
    assert 0.08 < float(p["state"].std()) < 0.12


def test_algorithmic_bytes():
    # (batch 4, D 5120, N 16, L 2048, bf16): 8 B per element plus B, C,
    # parameters and the fp32 final state
    assert W.scan_bytes(W.spec("mamba2p8b_layer")) == 337747968
    assert W.scan_bytes(W.spec("tiny_f32")) == 303616
    assert W.decode_step_bytes(W.spec("decode")) == 178642944
