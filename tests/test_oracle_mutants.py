"""Plant plausible mistakes in copies of the oracle (forward and backward) and
check the pins catch each.

Every mutant is a textual edit of oracle/flce_oracle.c compiled to a private
library on the CPU; the real oracle is never modified. A mutant that passes
every pin would mean the pins cannot tell that mistake from the definition.
"""
import os
import tempfile

import pytest

import oracle
from oracle_pins import ALL_PINS, BWD_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "flce_oracle.c")

MUTANTS = {
    "drop_last_word": ("for (int64_t v = 0; v < V; ++v) S += exp(z[v] - M);",
                       "for (int64_t v = 0; v < V - 1; ++v) S += exp(z[v] - M);"),
    "drop_first_word": ("for (int64_t v = 0; v < V; ++v) S += exp(z[v] - M);",
                        "for (int64_t v = 1; v < V; ++v) S += exp(z[v] - M);"),
    "lse_sign": ("double l = M + log(S);", "double l = M - log(S);"),
    "log_base2": ("double l = M + log(S);", "double l = M + log2(S);"),
    "loss_sign": ("loss[r] = l - z[t];", "loss[r] = z[t] - l;"),
    "no_max_shift": ("S += exp(z[v] - M);\n  double l = M + log(S);",
                     "S += exp(z[v]);\n  double l = log(S);"),
    "zero_init_max": ("double M = z[0];", "double M = 0.0;"),
    "transposed_W": ("acc += widen(H, dtype, i * D + d) * widen(W, dtype, v * D + d);",
                     "acc += widen(H, dtype, i * D + d) * widen(W, dtype, d * V + v);"),
    "reversed_features_H": ("acc += widen(H, dtype, i * D + d) * widen(W, dtype, v * D + d);",
                            "acc += widen(H, dtype, i * D + (D - 1 - d)) * widen(W, dtype, v * D + d);"),
    "drop_first_feature": ("for (int64_t d = 0; d < D; ++d)\n      acc += widen(H",
                           "for (int64_t d = 1; d < D; ++d)\n      acc += widen(H"),
    "neighbour_target": ("loss[r] = l - z[t];", "loss[r] = l - z[(t + 1) % V];"),
    "lse_minus_target_twice": ("lse[r] = l;", "lse[r] = l - z[0];"),
    "bf16_high_half_wrong": ("(uint32_t)((const uint16_t*)base)[idx] << 16",
                             "(uint32_t)((const uint16_t*)base)[idx] << 15"),
    # backward
    "bwd_onehot_sign": ("dz[v] = g[i] * (p - hit);", "dz[v] = g[i] * (p + hit);"),
    "bwd_no_upstream": ("dz[v] = g[i] * (p - hit);", "dz[v] = (p - hit);"),
    "bwd_neighbour_target": ("const double hit = v == t ? 1.0 : 0.0;", "const double hit = v == (t + 1) % V ? 1.0 : 0.0;"),
    "bwd_unnormalised_softmax": ("const double p = exp(dz[v] - l);", "const double p = exp(dz[v]);"),
    "bwd_dH_transposed_W": ("const double w = widen(W, dtype, v * D + d);", "const double w = widen(W, dtype, d * V + v);"),
    "bwd_dW_reversed_rows": ("const double h = widen(H, dtype, i * D + d);",
                             "const double h = widen(H, dtype, (N - 1 - i) * D + d);"),
    "bwd_dW_drop_last_row": ("for (int64_t i = 0; i < N; ++i) {\n          const double h",
                             "for (int64_t i = 0; i < N - 1; ++i) {\n          const double h"),
    # backward: the sums of |terms| that scale the GPU tolerance (inflated, dropped, signed)
    "bwd_abs_inflate_hit": ("dzabs[v] = fabs(g[i]) * (p + hit);", "dzabs[v] = fabs(g[i]) * (p + 2.0 * hit);"),
    "bwd_abs_inflate_p": ("dzabs[v] = fabs(g[i]) * (p + hit);", "dzabs[v] = fabs(g[i]) * (2.0 * p + hit);"),
    "bwd_abs_drop_hit": ("dzabs[v] = fabs(g[i]) * (p + hit);", "dzabs[v] = fabs(g[i]) * p;"),
    "bwd_abs_drop_p": ("dzabs[v] = fabs(g[i]) * (p + hit);", "dzabs[v] = fabs(g[i]) * hit;"),
    "bwd_abs_signed_g": ("dzabs[v] = fabs(g[i]) * (p + hit);", "dzabs[v] = g[i] * (p + hit);"),
    "bwd_dH_abs_signed_w": ("aabs += dzabs[v] * fabs(w);", "aabs += dzabs[v] * w;"),
    "bwd_dW_abs_signed_h": ("aabs += dzabs_all[i * V + v] * fabs(h);", "aabs += dzabs_all[i * V + v] * h;"),
    "bwd_dW_abs_squared_h": ("aabs += dzabs_all[i * V + v] * fabs(h);", "aabs += dzabs_all[i * V + v] * h * h;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "mutant.c")
        with open(src, "w") as f:
            f.write(text.replace(old, new))
        lib = oracle.load(oracle.build(src=src, out=os.path.join(d, "libmutant.so")))

        def fwd(H, W, y, rows=None):
            return oracle.forward(H, W, y, rows=rows, lib=lib)

        def bwd(H, W, y, g, rows=None, want_dW=True):
            return oracle.backward(H, W, y, g, rows=rows, want_dW=want_dW, lib=lib)

        caught = []
        for pin in ALL_PINS:
            try:
                pin(fwd)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(pin.__name__)
        for pin in BWD_PINS:
            try:
                pin(fwd, bwd)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(pin.__name__)
        assert caught, f"no pin catches mutant {name}"
