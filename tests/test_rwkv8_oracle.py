"""The RWKV-8 rho oracle against facts that do not come from the oracle
itself (tests/rwkv8_pins.py), its degenerate cases, and planted mistakes in
copies of its source that the pins must catch."""
import os
import zlib

import numpy as np
import pytest

import oracle.rwkv8 as R8
from oracle import build as obuild
import rwkv8_pins as P


@pytest.mark.parametrize("name", list(P.ALL_PINS))
def test_rwkv8_oracle_pin(name):
    fn, tol = P.ALL_PINS[name]
    err = fn(np.random.default_rng(zlib.crc32(name.encode())), None)
    assert err <= tol, f"{name}: rel err {err:.3e} > {tol:.0e}"


def test_rwkv8_oracle_degenerate():
    rng = np.random.default_rng(5)
    # T = 0: final states are the carry-in states, their gradients the final ones
    d = P.rand_inputs(rng, 2, 3, 0, 4, 5)
    y, RT, nT = P.run_fwd(d)
    g = P.run_bwd(d)
    assert y.shape == (2, 3, 0, 5)
    np.testing.assert_array_equal(RT, d["R0"])
    np.testing.assert_array_equal(nT, d["n0"])
    np.testing.assert_array_equal(g["dR0"], d["dRT"])
    np.testing.assert_array_equal(g["dn0"], d["dnT"])
    assert not g["ddecay"].any()
    # absent states and final gradients are zeros
    d = P.rand_inputs(rng, 1, 2, 6, 3, 4, states=False, final_grads=False)
    z = dict(d, R0=np.zeros((1, 2, 3, 4)), n0=np.zeros((1, 2, 3)), dRT=np.zeros((1, 2, 3, 4)),
             dnT=np.zeros((1, 2, 3)))
    for a, b in zip(P.run_fwd(d), P.run_fwd(z)):
        np.testing.assert_array_equal(a, b)
    ga, gb = P.run_bwd(d), P.run_bwd(z)
    for n in ga:
        np.testing.assert_array_equal(ga[n], gb[n])
    # threads do not change any bit
    d = P.rand_inputs(rng, 3, 4, 9, 3, 4)
    g1 = R8.backward(d["q"], d["v"], d["decay"], d["dy"], d["R0"], d["n0"], d["dRT"], d["dnT"],
                     threads=1)
    g7 = R8.backward(d["q"], d["v"], d["decay"], d["dy"], d["R0"], d["n0"], d["dRT"], d["dnT"],
                     threads=7)
    for n in g1:
        np.testing.assert_array_equal(g1[n], g7[n])


SRC = os.path.join(os.path.dirname(R8.__file__), "rwkv8_oracle.c")

MUTANTS = {
    "sigma_drops_eps": ("const double sigma = s + EPS;", "const double sigma = s;"),
    "weights_use_post_norm": ("if (J->y) readout(R, c, J->y + y_at(J, b, h, t), L, E);\n            update(R, n, d, q, v, L, E);",
                              "update(R, n, d, q, v, L, E);\n            if (J->y) readout(R, c, J->y + y_at(J, b, h, t), L, E);"),
    "update_decays_after_add": ("R[l * E + e] = d[l] * R[l * E + e] + q[l] * v[e];",
                                "R[l * E + e] = d[l] * (R[l * E + e] + q[l] * v[e]);"),
    "norm_misses_decay": ("n[l] = d[l] * n[l] + q[l];", "n[l] = n[l] + q[l];"),
    "dv_transposed_sum": ("acc += GR[l * E + e] * q[l];", "acc += GR[l * E + e] * q[e % L];"),
    "dq_drops_norm_carry": ("dq[l] = acc + Gn[l];", "dq[l] = acc;"),
    "decay_grad_post_state": ("dacc += GR[l * E + e] * Rt[l * E + e];",
                              "dacc += GR[l * E + e] * (Rt[l * E + e] * d[l] + q[l] * v[e]);"),
    "carry_misses_decay": ("for (int64_t e = 0; e < E; e++) GR[l * E + e] *= d[l];", "(void)0;"),
    "weights_grad_sign": ("dq[l] += (gc[l] - wq) / sigma;", "dq[l] += (gc[l] + wq) / sigma;"),
    "norm_grad_missing": ("Gn[l] -= gc[l] * c[l];", "(void)0;"),
    "context_grad_missing": ("GR[l * E + e] += c[l] * dy[e];", "(void)0;"),
    "final_grad_ignored": ("if (J->dRT) memcpy(GR, J->dRT + u * LE, (size_t)LE * sizeof(double));",
                           "if (0) memcpy(GR, J->dRT + u * LE, (size_t)LE * sizeof(double));"),
    "replay_keeps_post_state": ("update(hR, hn, d, J->q + q_at(J, b, h, t), J->v + v_at(J, b, h, t), L, E);\n        }\n        if (J->dRT)",
                                "update(hR, hn, d, J->q + q_at(J, b, h, t), J->v + v_at(J, b, h, t), L, E);\n            if (t % REPLAY == 0) { memcpy(kR + (t / REPLAY) * LE, hR, (size_t)LE * sizeof(double)); memcpy(kn + (t / REPLAY) * L, hn, (size_t)L * sizeof(double)); }\n        }\n        if (J->dRT)"),
}
QUICK = ("unit_decay_closed_form", "decay_brute_force", "identities", "torch_autograd",
         "torch_autograd_long", "split_sequence")


@pytest.mark.parametrize("name", list(MUTANTS))
def test_rwkv8_pins_catch_mutant(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    p = tmp_path / "mut.c"
    p.write_text(src.replace(old, new))
    lib = R8.load(obuild.build(str(p), str(tmp_path / "libmut.so")))
    try:
        caught = []
        for pin in QUICK:
            fn, tol = P.ALL_PINS[pin]
            if not fn(np.random.default_rng(13), lib) <= tol:
                caught.append(pin)
        assert caught, f"no pin caught mutant {name}"
    finally:
        R8.load()
