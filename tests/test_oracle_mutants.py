"""Plants plausible mistakes in copies of the oracle (on the CPU) and checks
that the pins catch every one of them."""
import os

import pytest

import oracle
from tests.oracle_pins import PINS

# (name, original text, mutated text) applied to oracle/mssm_oracle.c
MUTANTS = [
    ("drop_skip", "y += D_d * u[t];", "y += 0.0 * D_d * u[t];"),
    ("readout_before_update",
     "h[n] = decay * h[n] + drive;\n            y += C_b[t * dstate + n] * h[n];",
     "y += C_b[t * dstate + n] * h[n];\n            h[n] = decay * h[n] + drive;"),
    ("bias_after_softplus",
     "double x = delta[t] + bias_d;\n        double dt = softplus ? oracle_softplus(x) : x;",
     "double x = delta[t];\n        double dt = (softplus ? oracle_softplus(x) : x) + bias_d;"),
    ("flipped_A_sign", "exp(dt * A_row[n])", "exp(-dt * A_row[n])"),
    ("B_C_swapped", ["dt * B_b[t * dstate + n] * u[t]", "y += C_b[t * dstate + n]"],
     ["dt * C_b[t * dstate + n] * u[t]", "y += B_b[t * dstate + n]"]),
    ("B_transposed_index", "dt * B_b[t * dstate + n]", "dt * B_b[n * seqlen + t]"),
    ("no_gate", "out[t] = z ? y * oracle_silu(z[t]) : y;", "out[t] = y;"),
    ("skip_outside_gate",
     "y += D_d * u[t];\n        out[t] = z ? y * oracle_silu(z[t]) : y;",
     "out[t] = (z ? y * oracle_silu(z[t]) : y) + D_d * u[t];"),
    ("h0_ignored", "h[n] = h0 ? h0[n] : 0.0;", "h[n] = 0.0;"),
    ("euler_on_A", "double decay = exp(dt * A_row[n]);",
     "double decay = 1.0 + dt * A_row[n];"),
    ("full_zoh_on_B", "double drive = dt * B_b[t * dstate + n] * u[t];",
     "double drive = (exp(dt * A_row[n]) - 1.0) / A_row[n] * B_b[t * dstate + n] * u[t];"),
    ("sigmoid_gate", "return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    ("softplus_without_log", "return log1p(exp(x));", "return exp(x);"),
    ("softplus_naive_large_x", "return x + log1p(exp(-x));", "return x;"),
    ("last_state_lost", "last_state[n] = h[n];", "last_state[n] = 0.0;"),
    ("decode_B_of_batch0", "A + d * dstate, B + bg, C + bg,", "A + d * dstate, B, C,"),
    ("decode_state_not_written", "softplus, h, out + r, h);", "softplus, h, out + r, NULL);"),
    ("decode_x_dt_swapped", "x + r, dt + r", "dt + r, x + r"),
    # backward
    ("bwd_dy_without_gate", "dy = dout[t] * z[t] * sg;", "dy = dout[t];"),
    ("bwd_state_grad_not_decayed", "g[n] *= e;", "g[n] *= 1.0;"),
    ("bwd_dA_uses_new_state", "dA_row[n] += g[n] * DT[t] * e * prev;",
     "dA_row[n] += g[n] * DT[t] * H[t * dstate + n];"),
    ("bwd_softplus_derivative", "ddt *= 1.0 / (1.0 + exp(-X[t]));", "ddt *= exp(X[t]);"),
    ("bwd_dC_uses_state_grad", "dC_b[t * dstate + n] += dy * H[t * dstate + n];",
     "dC_b[t * dstate + n] += g[n] * H[t * dstate + n];"),
    ("bwd_dB_without_delta", "dB_b[t * dstate + n] += g[n] * DT[t] * u[t];",
     "dB_b[t * dstate + n] += g[n] * u[t];"),
    ("bwd_dz_without_silu_derivative", "dz[t] = dout[t] * Y[t] * sg * (1.0 + z[t] * (1.0 - sg));",
     "dz[t] = dout[t] * Y[t] * sg;"),
    ("bwd_readout_grad_after_use",
     "g[n] += dy * C_b[t * dstate + n];\n            dC_b[t * dstate + n] += dy * H[t * dstate + n];\n            dB_b[t * dstate + n] += g[n] * DT[t] * u[t];",
     "dC_b[t * dstate + n] += dy * H[t * dstate + n];\n            dB_b[t * dstate + n] += g[n] * DT[t] * u[t];\n            g[n] += dy * C_b[t * dstate + n];"),
    ("bwd_dh0_dropped", "dh0[n] = g[n];", "dh0[n] = 0.0;"),
    ("bwd_dD_missing", "*dD += dy * u[t];", "*dD += 0.0 * u[t];"),
    # B/C groups
    ("group_index_modulo", "return d / (dim / ngroups);", "return d % ngroups;"),
    ("group_gather_transposed",
     "X[((b * seqlen + t) * ngroups + g) * dstate + n];",
     "X[((b * ngroups + g) * seqlen + t) * dstate + n];"),
    ("bwd_dB_group_scatter_wrong_group", "dB[dst] = dBg[src];",
     "dB[dst] = dBg[((b * ngroups + 0) * seqlen + t) * dstate + n];"),
    # causal conv
    ("conv_kernel_not_flipped", "v += wr[k] * xv;", "v += wr[K - 1 - k] * xv;"),
    ("conv_window_off_by_one", "const int64_t s = t - (K - 1) + k;",
     "const int64_t s = t - K + k;"),
    ("conv_bias_dropped", "double v = bias ? bias[d] : 0.0;", "double v = 0.0;"),
    ("conv_silu_missing", "o[t] = silu ? oracle_silu(v) : v;", "o[t] = v;"),
    ("conv_init_ignored", "else if (ir)", "else if (0 && ir)"),
    ("conv_init_misaligned", "xv = ir[(K - 1) + s];", "xv = ir[-s - 1];"),
    # causal conv backward
    ("conv_bwd_silu_derivative_is_sigmoid", "g *= sg * (1.0 + v * (1.0 - sg));", "g *= sg;"),
    ("conv_bwd_dx_kernel_not_flipped", "dxr[s] += wr[k] * g;", "dxr[s] += wr[K - 1 - k] * g;"),
    ("conv_bwd_dw_uses_dout", "dw[d * K + k] += g * xv;", "dw[d * K + k] += gr[t] * xv;"),
    ("conv_bwd_dinit_dropped", "dir[(K - 1) + s] += wr[k] * g;", "dir[(K - 1) + s] += 0.0 * g;"),
    ("conv_bwd_dbias_ungated", "dbias[d] += g;", "dbias[d] += gr[t];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    olds = old if isinstance(old, list) else [old]
    news = new if isinstance(new, list) else [new]
    for o, n in zip(olds, news):
        # the first occurrence: the forward scan's own code comes before the
        # backward's recomputation of it
        assert src.count(o) >= 1, "mutation site for %s not found" % name
        src = src.replace(o, n, 1)
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(src)
    lib = oracle.compile_source(path, os.path.join(tmp_path, "libmutant.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "no pin caught mutant %s" % name
