"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one: a transposed index, a wrong sign, a dropped
term, the wrong state in a gradient, a seed that ignores dsT."""
import os

import numpy as np
import pytest

import oracle
from oracle import build as obuild
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "wkv7_oracle.c")

MUTANTS = {
    "sa_transposed": ("acc += S[i * N + j] * J->a[vix(J, b, t, h, j)];",
                      "acc += S[j * N + i] * J->a[vix(J, b, t, h, j)];"),
    "update_sign": ("vi * J->k[q] + sa[i] * J->b[q];\n            yy",
                    "vi * J->k[q] - sa[i] * J->b[q];\n            yy"),
    "update_drops_vk": ("S[i * N + j] * J->w[q] + vi * J->k[q] + sa[i] * J->b[q];\n            yy",
                        "S[i * N + j] * J->w[q] + sa[i] * J->b[q];\n            yy"),
    "readout_pre_update": ("yy += S[i * N + j] * J->r[q];",
                           "yy += (S[i * N + j] - vi * J->k[q]) * J->r[q];"),
    "dr_uses_pre_state": ("acc += St[i * N + j] * J->dy[vix(J, b, t, h, i)];",
                          "acc += P[i * N + j] * J->dy[vix(J, b, t, h, i)];"),
    "dw_uses_post_state": ("gw += g * P[i * N + j];", "gw += g * St[i * N + j];"),
    "db_uses_v": ("gb += g * sa[i];", "gb += g * J->v[vix(J, b, t, h, i)];"),
    "dv_uses_b": ("gv += G[i * N + j] * J->k[q];", "gv += G[i * N + j] * J->b[q];"),
    "da_transposed": ("acc += dsa[i] * P[i * N + j];", "acc += dsa[i] * P[j * N + i];"),
    "carry_uses_b": ("G[i * N + j] * J->w[q] + dsa[i] * J->a[q];",
                     "G[i * N + j] * J->w[q] + dsa[i] * J->b[q];"),
    "carry_drops_decay": ("G[i * N + j] * J->w[q] + dsa[i] * J->a[q];",
                          "G[i * N + j] + dsa[i] * J->a[q];"),
    "dy_r_not_folded": ("G[i * N + j] += dyi * J->r[vix(J, b, t, h, j)];",
                        "G[i * N + j] += 0.0 * dyi * J->r[vix(J, b, t, h, j)];"),
    "seed_ignores_dsT": ("J->dsT ? J->dsT[six(J, b, h, i, j)] : 0.0",
                         "0.0 * (J->dsT ? J->dsT[six(J, b, h, i, j)] : 0.0)"),
    "s0_transposed": ("S[i * N + j] = J->s0 ? J->s0[six(J, b, h, i, j)] : 0.0;",
                      "S[i * N + j] = J->s0 ? J->s0[six(J, b, h, j, i)] : 0.0;"),
}

# The cheap pins: enough to kill every mutant above.
QUICK = ("golden_n1", "golden_n2", "matrix_form", "identities", "split_sequence",
         "torch_autograd")


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    p = tmp_path / "mut.c"
    p.write_text(src.replace(old, new))
    lib = oracle.load(obuild.build(str(p), str(tmp_path / "libmut.so")))
    try:
        caught = []
        for pin in QUICK:
            fn, tol = P.ALL_PINS[pin]
            err = fn(np.random.default_rng(11), lib)
            if not err <= tol:
                caught.append(pin)
        assert caught, f"no pin caught mutant {name}"
    finally:
        oracle.load()  # restore the real oracle as the default
