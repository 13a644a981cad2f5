"""The fp64 oracle against facts that do not come from the oracle itself."""
import zlib

import numpy as np
import pytest

import oracle_pins as P


@pytest.mark.parametrize("name", list(P.ALL_PINS))
def test_oracle_pin(name):
    fn, tol = P.ALL_PINS[name]
    err = fn(np.random.default_rng(zlib.crc32(name.encode())), None)
    assert err <= tol, f"{name}: rel err {err:.3e} > {tol:.0e}"


def test_oracle_empty_and_degenerate():
    import oracle
    rng = np.random.default_rng(3)
    # T = 0: sT = s0, ds0 = dsT
    d = P.rand_inputs(rng, 2, 0, 3, 4)
    y, sT = P.run_fwd(d)
    g = P.run_bwd(d)
    assert y.shape == (2, 0, 3, 4)
    np.testing.assert_array_equal(sT, d["s0"])
    np.testing.assert_array_equal(g["ds0"], d["dsT"])
    # no s0 / no dsT: zeros
    d = P.rand_inputs(rng, 1, 6, 2, 4, s0=False, dsT=False)
    y, sT = P.run_fwd(d)
    d0 = dict(d, s0=np.zeros((1, 2, 4, 4)), dsT=np.zeros((1, 2, 4, 4)))
    y0, sT0 = P.run_fwd(d0)
    np.testing.assert_array_equal(y, y0)
    g, g0 = P.run_bwd(d), P.run_bwd(d0)
    for n in P.NAMES_GRAD + ("ds0",):
        np.testing.assert_array_equal(g[n], g0[n])
    # B = 0
    d = P.rand_inputs(rng, 0, 5, 2, 4)
    y, sT = oracle.forward(*(d[n] for n in P.NAMES_IN), s0=d["s0"])
    assert y.shape == (0, 5, 2, 4)


def test_oracle_threads_agree():
    """Spreading (b, h) over threads changes nothing (bitwise)."""
    import oracle
    rng = np.random.default_rng(4)
    d = P.rand_inputs(rng, 3, 9, 5, 6)
    args = [d[n] for n in P.NAMES_IN]
    y1, s1 = oracle.forward(*args, s0=d["s0"], threads=1)
    y8, s8 = oracle.forward(*args, s0=d["s0"], threads=8)
    np.testing.assert_array_equal(y1, y8)
    np.testing.assert_array_equal(s1, s8)
    g1 = oracle.backward(*args, d["dy"], s0=d["s0"], dsT=d["dsT"], threads=1)
    g8 = oracle.backward(*args, d["dy"], s0=d["s0"], dsT=d["dsT"], threads=7)
    for n in g1:
        np.testing.assert_array_equal(g1[n], g8[n])
