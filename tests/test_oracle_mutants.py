"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one: a transposed index, a wrong sign, a dropped
term, the wrong state in a gradient, a seed that ignores dsT, a slip in the
backward's replay of the forward from kept states."""
import os

import numpy as np
import pytest

import oracle
from oracle import build as obuild
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "wkv7_oracle.c")

MUTANTS = {
    "sa_transposed": ("mat_vec(S, J->a + o, sa, N);", "mat_t_vec(S, J->a + o, sa, N);"),
    "update_sign": ("add_outer(S, sa, J->b + o, N);",
                    "for (int64_t i = 0; i < N; i++) sa[i] = -sa[i]; add_outer(S, sa, J->b + o, N);"),
    "update_drops_vk": ("    add_outer(S, J->v + o, J->k + o, N);\n", ""),
    "readout_pre_update": ("step(J, o, S, sa);\n            if (J->y) mat_vec(S, J->r + o, J->y + o, N);",
                           "if (J->y) mat_vec(S, J->r + o, J->y + o, N);\n            step(J, o, S, sa);"),
    "dr_uses_pre_state": ("mat_t_vec(Scur, J->dy + o, J->dr + o, N);",
                          "mat_t_vec(Sprev, J->dy + o, J->dr + o, N);"),
    "dw_uses_post_state": ("diag_t_prod(Sprev, G, J->dw + o, N);",
                           "diag_t_prod(Scur, G, J->dw + o, N);"),
    "db_uses_v": ("mat_t_vec(G, sa, J->db + o, N);", "mat_t_vec(G, J->v + o, J->db + o, N);"),
    "dv_uses_b": ("mat_vec(G, J->k + o, J->dv + o, N);", "mat_vec(G, J->b + o, J->dv + o, N);"),
    "dk_transposed": ("mat_t_vec(G, J->v + o, J->dk + o, N);",
                      "mat_vec(G, J->v + o, J->dk + o, N);"),
    "da_transposed": ("mat_t_vec(Sprev, u, J->da + o, N);", "mat_vec(Sprev, u, J->da + o, N);"),
    "carry_uses_b": ("add_outer(G, u, J->a + o, N);", "add_outer(G, u, J->b + o, N);"),
    "carry_drops_decay": ("scale_cols(G, J->w + o, N);", "(void)0;"),
    "dy_r_not_folded": ("add_outer(G, J->dy + o, J->r + o, N);", "(void)0;"),
    "seed_ignores_dsT": ("copy_or_zero(G, J->dsT ? J->dsT + state_at(J, b, h) : NULL, N);",
                         "copy_or_zero(G, NULL, N);"),
    "state_transposed": ("if (src) memcpy(dst, src, (size_t)(N * N) * sizeof(double));",
                         "if (src) { for (int64_t i = 0; i < N; i++) for (int64_t j = 0; j < N; j++) "
                         "dst[i * N + j] = src[j * N + i]; }"),
    "replay_keeps_post_state": (
        "if (t % REPLAY == 0) memcpy(keep + (t / REPLAY) * NN, S, (size_t)NN * sizeof(double));\n"
        "            step(J, vec_at(J, b, t, h), S, sa);",
        "step(J, vec_at(J, b, t, h), S, sa);\n"
        "            if (t % REPLAY == 0) memcpy(keep + (t / REPLAY) * NN, S, (size_t)NN * sizeof(double));"),
    "replay_skips_last_step": ("for (int64_t t = t0; t < t1; t++) {\n                double *next",
                               "for (int64_t t = t0; t < t1 - 1; t++) {\n                double *next"),
}

# The cheap pins: enough to kill every mutant above.
QUICK = ("golden_n1", "golden_n2", "matrix_form", "identities", "split_sequence",
         "torch_autograd", "torch_autograd_long")


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
