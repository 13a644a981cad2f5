"""The time-mix epilogue (group norm, bonus, gate) after the scan, forward
and backward, against the fp64 oracle (oracle.epilogue), through the C ABI
(MI355X only)."""
import numpy as np
import pytest
import torch

import oracle.epilogue as OE
from linear_attention_rnn_wkv7_amd import api
from linear_attention_rnn_wkv7_amd.synthetic import custom, make_inputs

import gpu_helpers as H

pytestmark = pytest.mark.gpu

OUTS = ("dy", "dg", "dr", "dk", "dv", "dln_w", "dln_b", "dr_k")


def _say(msg):
    print(msg, flush=True)


def _inputs(B, T, Hh, dt, seed):
    """The scan's r, k, v and a scan-like y from the seeded generator of the
    workloads; gate = sigmoid(N(0,1)); per-channel parameters ~ N(1, 0.1^2),
    N(0, 0.1^2), N(0, 0.5^2)."""
    inp = make_inputs(custom(B, T, Hh, 64, dt, False, False, seed=seed), device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed + 1)
    shp = (B, T, Hh, 64)
    d = {"r": inp["r"], "k": inp["k"], "v": inp["v"],
         "y": 4.0 * torch.randn(shp, generator=gen, device="cuda") + 0.3,
         "g": torch.sigmoid(torch.randn(shp, generator=gen, device="cuda")).to(inp["r"].dtype),
         "dz": torch.randn(shp, generator=gen, device="cuda"),
         "ln_w": 1.0 + 0.1 * torch.randn((Hh, 64), generator=gen, device="cuda"),
         "ln_b": 0.1 * torch.randn((Hh, 64), generator=gen, device="cuda"),
         "r_k": 0.5 * torch.randn((Hh, 64), generator=gen, device="cuda")}
    return d


ARGS = ("y", "r", "k", "v", "g", "ln_w", "ln_b", "r_k")


def _check(got, ref, tau, label, names):
    errs, bad = H.compare(got, ref, tau, names=names)
    _say(f"{label}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    assert not bad, f"{label}: over {tau:g}*RMS: {bad} {errs}"


CASES = [(2, 37, 3, "f32"), (1, 100, 4, "bf16"), (3, 1, 2, "f32"), (4, 1024, 32, "f32")]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}_t{}_h{}_{}".format(*c))
def test_epilogue_parity(case):
    B, T, Hh, dt = case
    _say(f"case epilogue {case}")
    d = _inputs(B, T, Hh, dt, seed=900 + T)
    z = api.wkv7_epilogue_forward(*(d[n] for n in ARGS))
    g = api.wkv7_epilogue_backward(d["dz"], *(d[n] for n in ARGS))
    torch.cuda.synchronize()
    host = {n: H.to64(x) for n, x in d.items()}
    ref = OE.backward(host["dz"], *(host[n] for n in ARGS))
    ref["z"] = OE.forward(*(host[n] for n in ARGS))
    got = dict(g)
    got["z"] = z
    _check(got, ref, H.TAU[d["r"].dtype], f"epilogue{case}", ("z",) + OUTS)


def test_epilogue_deterministic():
    d = _inputs(2, 300, 8, "f32", seed=5)
    a = api.wkv7_epilogue_backward(d["dz"], *(d[n] for n in ARGS))
    b = api.wkv7_epilogue_backward(d["dz"], *(d[n] for n in ARGS))
    for n in OUTS:
        assert torch.equal(a[n], b[n]), n


def test_epilogue_around_the_scan():
    """scan -> epilogue forward; epilogue backward -> reverse scan with its dy,
    the bonus shares added to the scan's dr, dk, dv: against the two oracles
    chained the same way."""
    wl = custom(2, 100, 3, 64, "f32", True, True, seed=44)
    inp = make_inputs(wl, device="cuda")
    d = _inputs(2, 100, 3, "f32", seed=45)
    y, sT, ck = api.wkv7_forward(*(inp[n] for n in H.IN), inp["s0"], want_ckpt=True)
    z = api.wkv7_epilogue_forward(y, inp["r"], inp["k"], inp["v"], d["g"], d["ln_w"], d["ln_b"], d["r_k"])
    e = api.wkv7_epilogue_backward(d["dz"], y, inp["r"], inp["k"], inp["v"], d["g"], d["ln_w"],
                                   d["ln_b"], d["r_k"])
    s = api.wkv7_backward(*(inp[n] for n in H.IN), e["dy"], inp["s0"], inp["dsT"], ck)
    torch.cuda.synchronize()
    got = {"z": z, "dr": s["dr"] + e["dr"], "dk": s["dk"] + e["dk"], "dv": s["dv"] + e["dv"],
           "dw": s["dw"], "da": s["da"], "db": s["db"], "ds0": s["ds0"], "dg": e["dg"]}
    import oracle
    h = {n: H.to64(inp[n]) for n in H.IN}
    yo, _ = oracle.forward(*(h[n] for n in H.IN), s0=H.to64(inp["s0"]))
    pe = {n: H.to64(d[n]) for n in ("g", "ln_w", "ln_b", "r_k", "dz")}
    zo = OE.forward(yo, h["r"], h["k"], h["v"], pe["g"], pe["ln_w"], pe["ln_b"], pe["r_k"])
    eo = OE.backward(pe["dz"], yo, h["r"], h["k"], h["v"], pe["g"], pe["ln_w"], pe["ln_b"], pe["r_k"])
    so = oracle.backward(*(h[n] for n in H.IN), eo["dy"], s0=H.to64(inp["s0"]), dsT=H.to64(inp["dsT"]))
    ref = {"z": zo, "dr": so["dr"] + eo["dr"], "dk": so["dk"] + eo["dk"], "dv": so["dv"] + eo["dv"],
           "dw": so["dw"], "da": so["da"], "db": so["db"], "ds0": so["ds0"], "dg": eo["dg"]}
    _check(got, ref, 2e-4, "scan + epilogue", tuple(ref))
    assert np.isfinite(H.to64(z)).all()
