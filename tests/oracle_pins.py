"""Pins that tie the fp64 oracle to something other than itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with a value fixed by mathematics: a hand-evaluated tiny case, a
closed form (geometric series, convolution, step response), a library routine
(numpy.convolve, numpy.logaddexp, scipy.special.expit), a brute-force
"materialised" evaluation that sums every path through the recurrence
explicitly, or an invariant (split/carry, linearity, causality, permutation).

The method being pinned (the reading the oracle follows):
  Delta_t = softplus(delta_t + bias)          (or delta_t + bias, softplus off)
  h_t[n]  = exp(Delta_t A[n]) h_{t-1}[n] + Delta_t B_t[n] u_t
  out_t   = (sum_n C_t[n] h_t[n] + D u_t) * silu(z_t)
from page "Mamba: Selective State Space Models", "Mathematical Foundation"
(continuous model, selective mechanism, sequential scan) and "Architecture"
(Delta as the discretisation step).

The pins are written so that each plausible slip in the oracle -- a dropped
skip term, the readout taken before the update, the bias added after the
softplus, a flipped sign on A, B and C swapped, a transposed B index, a missing
or misplaced gate, an ignored initial state, another discretisation rule, a
wrong activation, a lost last_state, decode wiring mistakes -- fails at least
one of them; ``test_oracle_mutants.py`` checks exactly that by compiling such
variants of the oracle.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import expit

LN2 = math.log(2.0)


def _close(got, want, rtol=1e-13, atol=1e-13, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    err = np.abs(got - want)
    bound = atol + rtol * np.abs(want)
    bad = err > bound
    assert not bad.any(), "%s: max err %.3e (worst got %r want %r)" % (
        what, float(err.max()), got[bad].ravel()[:3], want[bad].ravel()[:3])


def _row_inputs(L, N, delta, A, B, C, u, D=0.0, bias=0.0):
    """Build a batch=1, dim=1 problem from per-row values."""
    u = np.asarray(u, dtype=np.float64).reshape(1, 1, L)
    delta = np.asarray(delta, dtype=np.float64).reshape(1, 1, L)
    A = np.asarray(A, dtype=np.float64).reshape(1, N)
    B = np.asarray(B, dtype=np.float64).reshape(1, L, N)
    C = np.asarray(C, dtype=np.float64).reshape(1, L, N)
    return dict(u=u, delta=delta, A=A, B=B, C=C, D=np.array([D]),
                delta_bias=np.array([bias]))


# ---------------------------------------------------------------- hand cases

def pin_h1_time_varying_delta(orc):
    """Delta = (1, 0.5, 0.25, 2) given directly, A = -1, B = C = u = 1, D = 0.
    Hand evaluation of the state after each token."""
    d = [1.0, 0.5, 0.25, 2.0]
    args = _row_inputs(4, 1, d, [-1.0], np.ones((4, 1)), np.ones((4, 1)),
                       np.ones(4))
    out, last = orc.scan(**args, softplus=False)
    h1 = 1.0                               # 0 * e^-1 + 1
    h2 = math.exp(-0.5) * h1 + 0.5
    h3 = math.exp(-0.25) * h2 + 0.25
    h4 = math.exp(-2.0) * h3 + 2.0
    _close(out.ravel(), [h1, h2, h3, h4], what="h1 out")
    _close(last.ravel(), [h4], what="h1 last_state")


def pin_h2_softplus_gate_skip(orc):
    """softplus(0) = ln 2 so exp(Delta A) = 1/2 for A = -1; B = 2, u = 1 gives
    a drive of 2 ln 2 per token and the state is the geometric series
    h_t = 4 ln2 (1 - 2^-(t+1)).  C = 1, D = 0.5, z = 2:
    out_t = (h_t + 0.5) * 2 / (1 + e^-2)."""
    L = 6
    args = _row_inputs(L, 1, np.zeros(L), [-1.0], 2 * np.ones((L, 1)),
                       np.ones((L, 1)), np.ones(L), D=0.5)
    z = 2.0 * np.ones((1, 1, L))
    out, last = orc.scan(**args, z=z, softplus=True)
    t = np.arange(L)
    h = 4 * LN2 * (1 - 0.5 ** (t + 1))
    gate = 2.0 / (1.0 + math.exp(-2.0))
    _close(out.ravel(), (h + 0.5) * gate, what="h2 out")
    _close(last.ravel(), [h[-1]], what="h2 last_state")


def pin_h3_zero_b_loaded_state(orc):
    """B = 0 with a loaded state h0 = (1, -2), A = (-1, -3), C = (1, 1),
    Delta = (0.5, 0.25, 0.25), u = (1, 2, 3), D = 0.5, softplus off:
    y_t = e^-S_t - 2 e^-3S_t + 0.5 u_t with S_t the running sum of Delta."""
    args = _row_inputs(3, 2, [0.5, 0.25, 0.25], [-1.0, -3.0],
                       np.zeros((3, 2)), np.ones((3, 2)), [1.0, 2.0, 3.0],
                       D=0.5)
    h0 = np.array([1.0, -2.0]).reshape(1, 1, 2)
    out, last = orc.scan(**args, softplus=False, h0=h0)
    S = np.array([0.5, 0.75, 1.0])
    y = np.exp(-S) - 2 * np.exp(-3 * S) + 0.5 * np.array([1.0, 2.0, 3.0])
    _close(out.ravel(), y, what="h3 out")
    _close(last.ravel(), [math.exp(-1.0), -2 * math.exp(-3.0)],
           what="h3 last_state")


def pin_h4_bias_inside_softplus(orc):
    """One token, A = -1, B = C = u = 1, D = 0, no gate, so y = Delta.
    delta = 0.5 with bias -0.5 must give softplus(0) = ln 2 (the bias is added
    before the activation); delta = -30 gives log(1 + e^-30), evaluated from
    its series e^-30 - e^-60/2; delta = 30 gives 30 + e^-30 - e^-60/2."""
    for delta, bias, want in [
            (0.5, -0.5, LN2),
            (-30.0, 0.0, math.exp(-30) - math.exp(-60) / 2),
            (30.0, 0.0, 30.0 + math.exp(-30) - math.exp(-60) / 2)]:
        args = _row_inputs(1, 1, [delta], [-1.0], [[1.0]], [[1.0]], [1.0],
                           bias=bias)
        out, _ = orc.scan(**args, softplus=True)
        _close(out.ravel(), [want], rtol=1e-14, atol=0.0,
               what="softplus(%g%+g)" % (delta, bias))


# ------------------------------------------------------------ closed forms

def pin_lti_convolution(orc):
    """Constant Delta, B, C over time make the scan time-invariant: the output
    is D u plus the causal convolution of u with the kernel
    K_k = sum_n C[n] exp(k Delta A[n]) Delta B[n]  (numpy.convolve).
    Run with Delta given directly and with Delta = softplus(x + bias), the
    latter evaluated with numpy.logaddexp(0, .)."""
    rng = np.random.default_rng(11)
    L, N = 50, 5
    A = -rng.uniform(0.2, 3.0, N)
    Bv = rng.standard_normal(N)
    Cv = rng.standard_normal(N)
    u = rng.standard_normal(L)
    D = 0.7
    for softplus, raw, bias in [(False, 0.3, 0.0), (True, -0.4, -1.1)]:
        dt = float(np.logaddexp(0.0, raw + bias)) if softplus else raw + bias
        args = _row_inputs(L, N, raw * np.ones(L), A, np.tile(Bv, (L, 1)),
                           np.tile(Cv, (L, 1)), u, D=D, bias=bias)
        out, _ = orc.scan(**args, softplus=softplus)
        k = np.arange(L)
        K = (Cv[None, :] * np.exp(np.outer(k, dt * A)) * dt * Bv[None, :]).sum(1)
        want = D * u + np.convolve(u, K)[:L]
        _close(out.ravel(), want, rtol=1e-12, atol=1e-12,
               what="lti conv softplus=%s" % softplus)


def pin_step_response(orc):
    """Constant u as well: every state component follows the geometric step
    response h_t[n] = Delta B[n] u (1 - a^(t+1)) / (1 - a), a = exp(Delta A[n])."""
    rng = np.random.default_rng(12)
    L, N = 37, 6
    A = -rng.uniform(0.1, 2.0, N)
    Bv = rng.standard_normal(N)
    dt, u = 0.45, 1.3
    args = _row_inputs(L, N, dt * np.ones(L), A, np.tile(Bv, (L, 1)),
                       np.ones((L, N)), u * np.ones(L))
    _, last = orc.scan(**args, softplus=False)
    a = np.exp(dt * A)
    want = dt * Bv * u * (1 - a ** L) / (1 - a)
    _close(last.ravel(), want, rtol=1e-12, atol=1e-14, what="step response")


def pin_zero_b(orc):
    """B = 0 and a zero initial state: the state stays exactly 0 and
    out = D u silu(z), silu via scipy.special.expit."""
    rng = np.random.default_rng(13)
    batch, dim, L, N = 2, 3, 17, 4
    u = rng.standard_normal((batch, dim, L))
    z = rng.standard_normal((batch, dim, L))
    D = rng.standard_normal(dim)
    out, last = orc.scan(u=u, delta=rng.standard_normal((batch, dim, L)),
                         A=-rng.uniform(0.5, 2, (dim, N)),
                         B=np.zeros((batch, L, N)),
                         C=rng.standard_normal((batch, L, N)), D=D, z=z,
                         delta_bias=rng.standard_normal(dim), softplus=True)
    want = D[None, :, None] * u * z * expit(z)
    _close(out, want, rtol=1e-14, atol=0.0, what="zero-B out")
    assert np.all(last == 0.0), "zero-B last_state not exactly 0"


def materialised(u, delta, A, B, C, D, z, bias, softplus, h0):
    """Brute force: every output as an explicit sum over all earlier tokens,
    h_t[n] = exp(A[n] S_t) h0[n] + sum_{s<=t} exp(A[n](S_t - S_s)) Delta_s
    B_s[n] u_s with S_t the running sum of Delta.  O(L^2 N) per row."""
    batch, dim, L = u.shape
    N = A.shape[1]
    x = delta + bias[None, :, None]
    dts = np.logaddexp(0.0, x) if softplus else x
    out = np.empty_like(u)
    last = np.empty((batch, dim, N))
    for b in range(batch):
        for d in range(dim):
            dt = dts[b, d]
            S = np.cumsum(dt)
            for t in range(L):
                h = np.exp(A[d] * S[t]) * h0[b, d]
                for s in range(t + 1):
                    h = h + np.exp(A[d] * (S[t] - S[s])) * dt[s] * B[b, s] * u[b, d, s]
                y = float(C[b, t] @ h) + D[d] * u[b, d, t]
                out[b, d, t] = y * z[b, d, t] * expit(z[b, d, t])
                if t == L - 1:
                    last[b, d] = h
    return out, last


def random_case(seed, batch=2, dim=3, L=24, N=4):
    rng = np.random.default_rng(seed)
    return dict(
        u=rng.standard_normal((batch, dim, L)),
        delta=rng.standard_normal((batch, dim, L)) - 1.0,
        A=-rng.uniform(0.2, 4.0, (dim, N)),
        B=rng.standard_normal((batch, L, N)),
        C=rng.standard_normal((batch, L, N)),
        D=rng.standard_normal(dim),
        z=rng.standard_normal((batch, dim, L)),
        delta_bias=rng.uniform(-2.0, 0.5, dim),
    ), 0.5 * rng.standard_normal((batch, dim, N))


def pin_materialised(orc):
    """The general case (softplus, bias, gate, skip, loaded state, batch > 1
    with a different B and C per batch entry) against the brute-force sum."""
    for softplus in (True, False):
        args, h0 = random_case(21 + softplus)
        out, last = orc.scan(**args, softplus=softplus, h0=h0)
        w_out, w_last = materialised(args["u"], args["delta"], args["A"],
                                     args["B"], args["C"], args["D"],
                                     args["z"], args["delta_bias"], softplus,
                                     h0)
        _close(out, w_out, rtol=1e-11, atol=1e-12, what="materialised out")
        _close(last, w_last, rtol=1e-11, atol=1e-12, what="materialised last")
    # the larger state sizes (up to 128 states per row)
    args, h0 = random_case(23, batch=1, dim=2, L=10, N=128)
    out, last = orc.scan(**args, softplus=True, h0=h0)
    w_out, w_last = materialised(args["u"], args["delta"], args["A"], args["B"],
                                 args["C"], args["D"], args["z"],
                                 args["delta_bias"], True, h0)
    _close(out, w_out, rtol=1e-11, atol=1e-12, what="materialised out N=128")
    _close(last, w_last, rtol=1e-11, atol=1e-12, what="materialised last N=128")


# -------------------------------------------------------------- invariants

def pin_split_carry(orc):
    """Scanning tokens [0, s) and then [s, L) from the carried last_state
    reproduces the unsplit scan, for every split point s."""
    args, h0 = random_case(31, batch=1, dim=2, L=40, N=3)
    out, last = orc.scan(**args, softplus=True, h0=h0)
    for s in range(1, 40):
        a1 = dict(args, u=args["u"][..., :s], delta=args["delta"][..., :s],
                  z=args["z"][..., :s], B=args["B"][:, :s], C=args["C"][:, :s])
        a2 = dict(args, u=args["u"][..., s:], delta=args["delta"][..., s:],
                  z=args["z"][..., s:], B=args["B"][:, s:], C=args["C"][:, s:])
        o1, l1 = orc.scan(**a1, softplus=True, h0=h0)
        o2, l2 = orc.scan(**a2, softplus=True, h0=l1)
        _close(np.concatenate([o1, o2], axis=-1), out, rtol=1e-13, atol=1e-14,
               what="split at %d" % s)
        _close(l2, last, rtol=1e-13, atol=1e-14, what="split last at %d" % s)


def pin_limits(orc):
    """Delta = 0 freezes the state: y = C_t . h0 + D u.  A = -1e4 makes
    exp(Delta A) underflow to 0: y = Delta u (C_t . B_t) + D u."""
    args, h0 = random_case(41, batch=1, dim=2, L=9, N=3)
    a0 = dict(args, delta=np.zeros_like(args["delta"]),
              delta_bias=np.zeros(2), z=None)
    out, last = orc.scan(**a0, softplus=False, h0=h0)
    want = (np.einsum("tn,dn->dt", args["C"][0], h0[0])
            + args["D"][:, None] * args["u"][0])
    _close(out[0], want, rtol=1e-14, atol=1e-14, what="Delta=0 out")
    _close(last, h0, rtol=0, atol=0, what="Delta=0 last")
    a1 = dict(args, A=-1e4 * np.ones_like(args["A"]), z=None,
              delta=np.abs(args["delta"]) + 0.1, delta_bias=np.zeros(2))
    out, _ = orc.scan(**a1, softplus=False, h0=h0)
    dt = a1["delta"][0]
    cb = np.einsum("tn,tn->t", args["C"][0], args["B"][0])
    want = dt * args["u"][0] * cb[None, :] + args["D"][:, None] * args["u"][0]
    _close(out[0], want, rtol=1e-13, atol=1e-14, what="A=-1e4 out")


def pin_linearity_causality(orc):
    """u -> out is linear for fixed delta, B, C, z (zero initial state), and a
    change of u at token t0 leaves every earlier output untouched."""
    args, _ = random_case(51, L=20)
    rng = np.random.default_rng(52)
    u1, u2 = args["u"], rng.standard_normal(args["u"].shape)
    o1, _ = orc.scan(**args, softplus=True)
    o2, _ = orc.scan(**dict(args, u=u2), softplus=True)
    o3, _ = orc.scan(**dict(args, u=2.5 * u1 - 1.5 * u2), softplus=True)
    _close(o3, 2.5 * o1 - 1.5 * o2, rtol=1e-12, atol=1e-12, what="linearity")
    u4 = u1.copy()
    u4[..., 11] += 3.0
    o4, _ = orc.scan(**dict(args, u=u4), softplus=True)
    assert np.array_equal(o4[..., :11], o1[..., :11]), "causality"
    assert not np.allclose(o4[..., 11:], o1[..., 11:]), "u change had no effect"


def pin_channel_permutation(orc):
    """Permuting channels together with A, D and the bias permutes the output."""
    args, h0 = random_case(61, dim=5, L=12)
    out, last = orc.scan(**args, softplus=True, h0=h0)
    p = np.array([3, 0, 4, 1, 2])
    pa = dict(args, u=args["u"][:, p], delta=args["delta"][:, p],
              z=args["z"][:, p], A=args["A"][p], D=args["D"][p],
              delta_bias=args["delta_bias"][p])
    o2, l2 = orc.scan(**pa, softplus=True, h0=h0[:, p])
    assert np.array_equal(o2, out[:, p]) and np.array_equal(l2, last[:, p])


def pin_decode_equals_scan(orc):
    """L single-token decode steps from h0 reproduce the scan's outputs and
    last_state: the sequential inference form of the same recurrence."""
    args, h0 = random_case(71, batch=2, dim=3, L=15, N=4)
    out, last = orc.scan(**args, softplus=True, h0=h0)
    state = h0.copy()
    for t in range(15):
        y, state = orc.state_update(
            state, args["u"][..., t], args["delta"][..., t], args["A"],
            args["B"][:, t], args["C"][:, t], D=args["D"],
            z=args["z"][..., t], dt_bias=args["delta_bias"], softplus=True)
        _close(y, out[..., t], rtol=1e-15, atol=1e-15, what="decode t=%d" % t)
    _close(state, last, rtol=1e-15, atol=1e-15, what="decode state")


PINS = [
    pin_h1_time_varying_delta,
    pin_h2_softplus_gate_skip,
    pin_h3_zero_b_loaded_state,
    pin_h4_bias_inside_softplus,
    pin_lti_convolution,
    pin_step_response,
    pin_zero_b,
    pin_materialised,
    pin_split_carry,
    pin_limits,
    pin_linearity_causality,
    pin_channel_permutation,
    pin_decode_equals_scan,
]


# ------------------------------------------------------------- gradients

def _loss(orc, args, softplus, h0, dout, dlast):
    out, last = orc.scan(**args, softplus=softplus, h0=h0)
    return float((dout * out).sum() + (dlast * last).sum())


def pin_bwd_finite_differences(orc):
    """Every gradient of the oracle's backward against central differences of
    the (pinned) forward oracle, loss = sum(dout*out) + sum(dlast*last_state),
    step 1e-6 (truncation error O(1e-12) relative)."""
    for softplus in (True, False):
        args, h0 = random_case(91 + softplus, batch=2, dim=3, L=9, N=3)
        if not softplus:
            args = dict(args, delta=np.abs(args["delta"]) * 0.3 + 0.05,
                        delta_bias=np.abs(args["delta_bias"]) * 0.1)
        rng = np.random.default_rng(93)
        dout = rng.standard_normal(args["u"].shape)
        dlast = rng.standard_normal(h0.shape)
        g = orc.scan_bwd(args["u"], args["delta"], args["A"], args["B"], args["C"],
                         dout, D=args["D"], z=args["z"],
                         delta_bias=args["delta_bias"], softplus=softplus, h0=h0,
                         dlast=dlast)
        eps = 1e-6
        pairs = [("u", "du"), ("delta", "ddelta"), ("z", "dz"), ("A", "dA"),
                 ("B", "dB"), ("C", "dC"), ("D", "dD"),
                 ("delta_bias", "ddelta_bias"), ("h0", "dh0")]
        for name, gname in pairs:
            base = h0 if name == "h0" else args[name]
            fd = np.empty_like(base)
            for idx in np.ndindex(base.shape):
                p, m = base.copy(), base.copy()
                p[idx] += eps
                m[idx] -= eps
                if name == "h0":
                    lp = _loss(orc, args, softplus, p, dout, dlast)
                    lm = _loss(orc, args, softplus, m, dout, dlast)
                else:
                    lp = _loss(orc, dict(args, **{name: p}), softplus, h0, dout, dlast)
                    lm = _loss(orc, dict(args, **{name: m}), softplus, h0, dout, dlast)
                fd[idx] = (lp - lm) / (2 * eps)
            _close(g[gname], fd, rtol=1e-6, atol=1e-7,
                   what="d%s softplus=%s" % (name, softplus))


def pin_bwd_zero_b_closed_form(orc):
    """B = 0, no gate, D = 0: out_t = sum_n C_t[n] exp(A[n] S_t) h0[n] with
    S_t the running sum of Delta, so dC_t[n] = dout_t exp(A[n] S_t) h0[n] and
    dh0[n] = sum_t dout_t C_t[n] exp(A[n] S_t) exactly; du = dB * 0 terms
    vanish except du_t = sum_n g_t[n] Delta_t B_t[n] = 0."""
    rng = np.random.default_rng(97)
    L, N = 11, 4
    dt = np.abs(rng.standard_normal(L)) * 0.2 + 0.01
    A = -rng.uniform(0.3, 2.0, N)
    C = rng.standard_normal((L, N))
    h0 = rng.standard_normal(N)
    dout = rng.standard_normal(L)
    args = _row_inputs(L, N, dt, A, np.zeros((L, N)), C, rng.standard_normal(L))
    g = orc.scan_bwd(args["u"], args["delta"], args["A"], args["B"], args["C"],
                     dout.reshape(1, 1, L), D=np.zeros(1), z=None,
                     delta_bias=np.zeros(1), softplus=False,
                     h0=h0.reshape(1, 1, N), dlast=None)
    S = np.cumsum(dt)
    E = np.exp(np.outer(S, A))                       # (L, N)
    _close(g["dC"][0], dout[:, None] * E * h0[None, :], rtol=1e-13, atol=1e-15,
           what="zero-B dC")
    _close(g["dh0"][0, 0], (dout[:, None] * C * E).sum(0), rtol=1e-13, atol=1e-15,
           what="zero-B dh0")
    _close(g["du"][0, 0], np.zeros(L), rtol=0, atol=1e-15, what="zero-B du")


PINS += [pin_bwd_finite_differences, pin_bwd_zero_b_closed_form]


# ------------------------------------------------ causal conv ahead of the scan
# Reading pinned here (width K = 4, page "Mamba State Space Model" d_conv):
#   v[t] = bias + sum_k w[k] x[t-(K-1)+k],  x[t<0] = init or 0;  out = silu(v)

def pin_conv_numpy_convolve(orc):
    """Equals numpy.convolve's full causal convolution truncated to L (the
    library routine flips the kernel, so w[K-1] weighs the current step),
    plus the bias, for every channel; with silu, expit(v) * v."""
    rng = np.random.default_rng(41)
    batch, dim, L, K = 2, 3, 29, 4
    x = rng.standard_normal((batch, dim, L))
    w = rng.standard_normal((dim, K))
    bias = rng.standard_normal(dim)
    v = orc.causal_conv1d(x, w, bias, silu=False)
    s = orc.causal_conv1d(x, w, bias, silu=True)
    for b in range(batch):
        for d in range(dim):
            want = np.convolve(x[b, d], w[d, ::-1])[:L] + bias[d]
            _close(v[b, d], want, 1e-13, 1e-13, "conv vs numpy.convolve")
            _close(s[b, d], want * expit(want), 1e-13, 1e-13, "silu(conv)")


def pin_conv_impulse_and_constant(orc):
    """A unit impulse at step 5 reproduces the taps in reverse time order
    (out[5 + j] = w[K-1-j]) and nothing before step 5; a constant input c
    gives bias + c * sum(w) once the window is full, and partial sums of
    the newest taps before that (zero history)."""
    L, K = 14, 4
    w = np.array([[0.5, -1.25, 2.0, 3.5]])
    x = np.zeros((1, 1, L))
    x[0, 0, 5] = 1.0
    v = orc.causal_conv1d(x, w, None, silu=False)[0, 0]
    want = np.zeros(L)
    for j in range(K):
        want[5 + j] = w[0, K - 1 - j]
    _close(v, want, 0, 0, "impulse response")
    c = 0.75
    v = orc.causal_conv1d(np.full((1, 1, L), c), w, np.array([0.3]), silu=False)[0, 0]
    for t in range(L):
        taps = w[0, K - 1 - min(t, K - 1):]      # the newest min(t+1, K) taps
        _close(v[t], 0.3 + c * taps.sum(), 1e-15, 1e-15, "constant input")


def pin_conv_initial_values_split(orc):
    """Splitting a sequence in two and passing the last K-1 inputs of the first
    part as the second part's initial values reproduces the whole run; a
    nonzero init changes exactly the first K-1 outputs."""
    rng = np.random.default_rng(43)
    batch, dim, L, K, cut = 2, 2, 20, 4, 9
    x = rng.standard_normal((batch, dim, L))
    w = rng.standard_normal((dim, K))
    bias = rng.standard_normal(dim)
    full = orc.causal_conv1d(x, w, bias)
    first = orc.causal_conv1d(x[:, :, :cut], w, bias)
    second = orc.causal_conv1d(x[:, :, cut:], w, bias, init=x[:, :, cut - K + 1:cut])
    _close(np.concatenate([first, second], axis=2), full, 0, 0, "conv split")
    init = rng.standard_normal((batch, dim, K - 1))
    a = orc.causal_conv1d(x, w, bias, init=init, silu=False)
    b = orc.causal_conv1d(x, w, bias, silu=False)
    _close(a[:, :, K - 1:], b[:, :, K - 1:], 0, 0, "init affects only the first K-1")
    for t in range(K - 1):
        want = b[:, :, t] + sum(w[None, :, k] * init[:, :, t + k]
                                for k in range(K - 1 - t))
        _close(a[:, :, t], want, 1e-14, 1e-14, "init step %d" % t)


def pin_conv_then_scan_equals_scan_of_conv(orc):
    """The fused block step is the composition: scanning silu(conv(x)) is the
    oracle scan applied to the conv output (a wiring check the GPU's fused
    path is compared against)."""
    rng = np.random.default_rng(47)
    batch, dim, L, N = 1, 2, 12, 4
    x = rng.standard_normal((batch, dim, L))
    w = rng.standard_normal((dim, 4))
    cb = rng.standard_normal(dim)
    u = orc.causal_conv1d(x, w, cb)
    assert np.isfinite(u).all()
    # brute-force silu(conv) at one point
    t = 7
    v = cb[1] + sum(w[1, k] * x[0, 1, t - 3 + k] for k in range(4))
    _close(u[0, 1, t], v / (1.0 + math.exp(-v)), 1e-14, 1e-14, "silu(conv) point")


PINS += [pin_conv_numpy_convolve, pin_conv_impulse_and_constant,
         pin_conv_initial_values_split, pin_conv_then_scan_equals_scan_of_conv]


def pin_conv_bwd_finite_differences(orc):
    """Every gradient of the conv's backward (x, w, bias and the values before
    t = 0, given or zero) against central differences of the pinned forward
    conv, loss = sum(dout * out), for widths 1..4 with and without silu;
    step 1e-6 (truncation error O(1e-12) relative)."""
    rng = np.random.default_rng(51)
    batch, dim, L = 2, 2, 6
    for K in (1, 2, 3, 4):
        for silu in (True, False):
            for with_init in (True, False):
                x = rng.standard_normal((batch, dim, L))
                w = rng.standard_normal((dim, K))
                bias = rng.standard_normal(dim)
                init = rng.standard_normal((batch, dim, K - 1)) if with_init else None
                dout = rng.standard_normal((batch, dim, L))
                g = orc.causal_conv1d_bwd(x, w, dout, bias=bias, init=init, silu=silu)
                base = {"x": x, "w": w, "bias": bias,
                        "init": init if with_init else np.zeros((batch, dim, K - 1))}

                def loss(**over):
                    a = dict(base, **over)
                    return float((dout * orc.causal_conv1d(a["x"], a["w"], a["bias"],
                                                           init=a["init"],
                                                           silu=silu)).sum())
                eps = 1e-6
                for name, gname in (("x", "dx"), ("w", "dw"), ("bias", "dbias"),
                                    ("init", "dinit")):
                    arr = base[name]
                    fd = np.empty_like(arr)
                    for idx in np.ndindex(arr.shape):
                        p, m = arr.copy(), arr.copy()
                        p[idx] += eps
                        m[idx] -= eps
                        fd[idx] = (loss(**{name: p}) - loss(**{name: m})) / (2 * eps)
                    _close(g[gname], fd, rtol=1e-6, atol=1e-8,
                           what="conv d%s K=%d silu=%s init=%s" % (name, K, silu, with_init))


def pin_conv_bwd_width1_closed_form(orc):
    """Width 1 without silu is out = w x + bias per channel, so exactly
    dx = w dout, dw = sum(dout x), dbias = sum(dout) over batch and time, and
    no values before t = 0 are read (dinit is empty)."""
    rng = np.random.default_rng(53)
    batch, dim, L = 3, 4, 10
    x = rng.standard_normal((batch, dim, L))
    w = rng.standard_normal((dim, 1))
    dout = rng.standard_normal((batch, dim, L))
    g = orc.causal_conv1d_bwd(x, w, dout, bias=rng.standard_normal(dim), silu=False)
    _close(g["dx"], w[None, :, 0:1] * dout, 1e-15, 1e-15, "width-1 dx")
    _close(g["dw"][:, 0], (dout * x).sum(axis=(0, 2)), 1e-13, 1e-13, "width-1 dw")
    _close(g["dbias"], dout.sum(axis=(0, 2)), 1e-13, 1e-13, "width-1 dbias")
    assert g["dinit"].shape == (batch, dim, 0)


PINS += [pin_conv_bwd_finite_differences, pin_conv_bwd_width1_closed_form]


# --------------------------------------------------------------- B/C groups
# Reading: with G groups, B, C are (batch, L, G, N) and channel d reads group
# d // (dim // G) (contiguous channel blocks).

def pin_groups_reduce_to_one_group(orc):
    """G groups holding identical B and C give exactly the one-group result;
    and each group's channels equal a one-group scan of just those channels
    with just that group's B and C (forward, decode and backward)."""
    rng = np.random.default_rng(61)
    batch, dim, L, N, G = 2, 6, 9, 3, 3
    args, h0 = random_case(62, batch=batch, dim=dim, L=L, N=N)
    Bg = rng.standard_normal((batch, L, G, N))
    Cg = rng.standard_normal((batch, L, G, N))
    same = dict(args, B=np.repeat(args["B"][:, :, None, :], G, axis=2),
                C=np.repeat(args["C"][:, :, None, :], G, axis=2))
    o1, l1 = orc.scan(**args, softplus=True, h0=h0)
    oG, lG = orc.scan(**same, softplus=True, h0=h0)
    _close(oG, o1, 0, 0, "identical groups = one group")
    _close(lG, l1, 0, 0, "identical groups = one group (state)")
    gargs = dict(args, B=Bg, C=Cg)
    out, last = orc.scan(**gargs, softplus=True, h0=h0)
    dout = rng.standard_normal(args["u"].shape)
    dlast = rng.standard_normal(h0.shape)
    gb = orc.scan_bwd(gargs["u"], gargs["delta"], gargs["A"], Bg, Cg, dout,
                      D=gargs["D"], z=gargs["z"], delta_bias=gargs["delta_bias"],
                      h0=h0, dlast=dlast)
    per = dim // G
    for g in range(G):
        ch = slice(g * per, (g + 1) * per)
        sub = dict(u=args["u"][:, ch], delta=args["delta"][:, ch], A=args["A"][ch],
                   B=Bg[:, :, g], C=Cg[:, :, g], D=args["D"][ch], z=args["z"][:, ch],
                   delta_bias=args["delta_bias"][ch])
        o, l = orc.scan(**sub, softplus=True, h0=h0[:, ch])
        _close(out[:, ch], o, 0, 0, "group %d channels" % g)
        _close(last[:, ch], l, 0, 0, "group %d state" % g)
        sb = orc.scan_bwd(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"],
                          dout[:, ch], D=sub["D"], z=sub["z"],
                          delta_bias=sub["delta_bias"], h0=h0[:, ch],
                          dlast=dlast[:, ch])
        _close(gb["dB"][:, :, g], sb["dB"], 1e-13, 1e-13, "group %d dB" % g)
        _close(gb["dC"][:, :, g], sb["dC"], 1e-13, 1e-13, "group %d dC" % g)
        _close(gb["du"][:, ch], sb["du"], 0, 0, "group %d du" % g)
        # decode of the first token against the group's one-group decode
        o1s, s1s = orc.state_update(h0[:, ch], sub["u"][:, :, 0], sub["delta"][:, :, 0],
                                    sub["A"], sub["B"][:, 0], sub["C"][:, 0], D=sub["D"],
                                    z=sub["z"][:, :, 0], dt_bias=sub["delta_bias"])
        oGs, sGs = orc.state_update(h0, args["u"][:, :, 0], args["delta"][:, :, 0],
                                    args["A"], Bg[:, 0], Cg[:, 0], D=args["D"],
                                    z=args["z"][:, :, 0], dt_bias=args["delta_bias"])
        _close(oGs[:, ch], o1s, 0, 0, "group %d decode" % g)
        _close(sGs[:, ch], s1s, 0, 0, "group %d decode state" % g)


PINS += [pin_groups_reduce_to_one_group]


# ------------------------------------------------------------ Mamba-2 scan
# Reading: the Mamba-2 block's scan is the selective recurrence with one A,
# one step Delta and one D per head of P channels, B and C per group of
# heads, x and out laid out (batch, L, heads, P), the state (batch, heads * P,
# N) with channel h * P + p.

def _softplus_inv(v):
    return math.log(math.expm1(v))


def pin_mamba2_per_head_closed_form(orc):
    """Constant inputs per head: every (head, channel, state) follows the
    geometric series h_t = s (1 - e^(t+1)) / (1 - e), e = exp(Delta_h A_h),
    s = Delta_h B_g[n] x_hp, with Delta_h from dt_bias through softplus, the
    head's own D and the channel's own gate."""
    batch, L, H, P, N, G = 2, 7, 4, 3, 2, 2
    A = np.array([-0.5, -1.0, -2.0, -0.25])
    Dh = np.array([0.5, -1.0, 2.0, 0.0])
    step = np.array([0.3, 0.05, 0.7, 1.1])              # Delta per head
    bias = np.array([_softplus_inv(v) for v in step])
    Bg = np.array([[1.0, 2.0], [-0.5, 3.0]])            # per group, constant in t
    Cg = np.array([[1.0, -1.0], [0.25, 2.0]])
    xv = np.arange(1, batch * H * P + 1, dtype=np.float64).reshape(batch, H, P) / 7.0
    zv = np.linspace(-2.0, 2.0, batch * H * P).reshape(batch, H, P)
    x = np.broadcast_to(xv[:, None], (batch, L, H, P)).copy()
    z = np.broadcast_to(zv[:, None], (batch, L, H, P)).copy()
    dt = np.zeros((batch, L, H))
    B = np.broadcast_to(Bg, (batch, L, G, N)).copy()
    C = np.broadcast_to(Cg, (batch, L, G, N)).copy()
    out, last = orc.mamba2_scan(x, dt, A, B, C, D=Dh, z=z, dt_bias=bias, softplus=True)
    want = np.empty_like(out)
    want_last = np.empty_like(last)
    for b in range(batch):
        for h in range(H):
            g = h // (H // G)
            e = math.exp(step[h] * A[h])
            for p in range(P):
                for t in range(L):
                    hs = step[h] * Bg[g] * xv[b, h, p] * (1.0 - e ** (t + 1)) / (1.0 - e)
                    y = float(np.dot(Cg[g], hs)) + Dh[h] * xv[b, h, p]
                    want[b, t, h, p] = y * zv[b, h, p] * expit(zv[b, h, p])
                want_last[b, h * P + p] = hs
    _close(out, want, 1e-12, 1e-12, "mamba2 closed form out")
    _close(last, want_last, 1e-12, 1e-12, "mamba2 closed form state")


def pin_mamba2_brute_force(orc):
    """Random tiny case, time-varying everything, loaded state, softplus off
    and on: the recurrence evaluated with plain loops over (b, t, h, p, n)."""
    rng = np.random.default_rng(71)
    batch, L, H, P, N, G = 2, 5, 4, 2, 3, 2
    x = rng.standard_normal((batch, L, H, P))
    z = rng.standard_normal((batch, L, H, P))
    dt = rng.uniform(0.05, 0.6, (batch, L, H))
    A = -rng.uniform(0.2, 2.0, H)
    B = rng.standard_normal((batch, L, G, N))
    C = rng.standard_normal((batch, L, G, N))
    Dh = rng.standard_normal(H)
    bias = rng.uniform(-0.5, 0.5, H)
    h0 = rng.standard_normal((batch, H * P, N))
    for softplus in (False, True):
        out, last = orc.mamba2_scan(x, dt, A, B, C, D=Dh, z=z, dt_bias=bias,
                                    softplus=softplus, h0=h0)
        want = np.empty((batch, L, H, P))
        state = h0.copy()
        for b in range(batch):
            for h in range(H):
                g = h // (H // G)
                for t in range(L):
                    v = dt[b, t, h] + bias[h]
                    step = math.log1p(math.exp(v)) if softplus else v
                    for p in range(P):
                        d = h * P + p
                        y = 0.0
                        for n in range(N):
                            state[b, d, n] = (math.exp(step * A[h]) * state[b, d, n]
                                              + step * B[b, t, g, n] * x[b, t, h, p])
                            y += C[b, t, g, n] * state[b, d, n]
                        y += Dh[h] * x[b, t, h, p]
                        want[b, t, h, p] = y * z[b, t, h, p] / (1.0 + math.exp(-z[b, t, h, p]))
        _close(out, want, 1e-12, 1e-12, "mamba2 brute force out (softplus %s)" % softplus)
        _close(last, state, 1e-12, 1e-12, "mamba2 brute force state (softplus %s)" % softplus)


PINS += [pin_mamba2_per_head_closed_form, pin_mamba2_brute_force]
