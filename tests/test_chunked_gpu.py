"""The chunk-form reverse scan (WKV7_ALGO_CHUNKED) against the oracle and the
step scan, and its per-head fallback, through the C ABI (MI355X only)."""
import pytest
import torch

from linear_attention_rnn_wkv7_amd.synthetic import custom, make_inputs

import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _check(out, ref, tau, label):
    errs, bad = H.compare(out, ref, tau)
    _say(f"{label}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    assert not bad, f"{label}: over {tau:g}*RMS: {bad} {errs}"


# (B, T, H, dtype, s0, dsT): one and several chunks, ragged last chunks
CASES = [
    (1, 1, 1, "f32", False, False),
    (1, 5, 2, "f32", True, True),
    (2, 63, 3, "f32", True, False),
    (1, 64, 2, "f32", False, True),
    (2, 65, 2, "f32", True, True),
    (1, 130, 4, "f32", False, False),
    (3, 200, 2, "f32", True, True),
    (2, 273, 3, "bf16", True, True),
    (1, 640, 2, "f32", True, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}_t{}_h{}_{}_s0{}_dsT{}".format(*c))
def test_chunked_parity(case):
    B, T, Hh, dt, s0, dsT = case
    wl = custom(B, T, Hh, 64, dtype=dt, has_s0=s0, has_dsT=dsT, seed=11 + T)
    _say(f"case chunked {wl.name}")
    inp = make_inputs(wl, device="cuda")
    out = H.gpu_run(inp, chunk=64, algo="chunked")
    torch.cuda.synchronize()
    ref = H.oracle_run(inp)
    _check(out, ref, H.TAU[inp["r"].dtype], wl.name)


def test_chunked_agrees_with_scan():
    wl = custom(2, 512, 4, 64, has_s0=True, has_dsT=True, seed=5)
    _say(f"case chunked-vs-scan {wl.name}")
    inp = make_inputs(wl, device="cuda")
    a = H.gpu_run(inp, chunk=64, algo="chunked")
    b = H.gpu_run(inp, chunk=64, algo="scan")
    torch.cuda.synchronize()
    ref = {n: H.to64(x) for n, x in b.items() if x is not None}
    _check(a, ref, 2e-4, "chunked vs scan")


def test_chunked_falls_back_per_head():
    """Heads whose decays leave the chunk form's range are recomputed by the
    step scan (bitwise equal to it); the other heads keep the chunk form."""
    wl = custom(2, 200, 3, 64, has_s0=True, has_dsT=True, seed=17)
    _say(f"case fallback {wl.name}")
    inp = make_inputs(wl, device="cuda")
    w = inp["w"]
    w[1, 150, 2, 7] = 0.0          # a decay of exactly 0
    w[0, 10:30, 1, :] = 0.02       # decays below 1/16
    w[1, 64:128, 0, 3] = 0.3       # cumulative decay 0.3^64 < 2^-60
    flagged = [(1, 2), (0, 1), (1, 0)]
    a = H.gpu_run(inp, chunk=64, algo="chunked")
    s = H.gpu_run(inp, chunk=64, algo="scan")
    torch.cuda.synchronize()
    ref = H.oracle_run(inp)
    _check(a, ref, 2e-4, "fallback")
    for b in range(wl.B):
        for h in range(wl.H):
            same = all(torch.equal(a[n][b, :, h], s[n][b, :, h]) for n in H.GRADS) and \
                torch.equal(a["ds0"][b, h], s["ds0"][b, h])
            assert same == ((b, h) in flagged), (b, h, same)
