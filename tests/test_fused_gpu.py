"""Fused time-mix inputs (WKV7_FUSED_INPUTS): the library forms w, a, b from
omega, kk and the gate, and returns d omega, d kk, d gate, against the fp64
oracle of the same formulas (oracle.fused), through the C ABI (MI355X only)."""
import numpy as np
import pytest
import torch

import oracle.fused as OF
from linear_attention_rnn_wkv7_amd import api
from linear_attention_rnn_wkv7_amd.synthetic import WORKLOADS, custom, make_inputs
from linear_attention_rnn_wkv7_amd.synthetic import state_slice, vec_slice

import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _run(inp, ckpt_handoff=True):
    y, sT, ck = api.wkv7_forward(*(inp[n] for n in H.IN), inp["s0"], want_ckpt=ckpt_handoff,
                                 fused=True)
    g = api.wkv7_backward(*(inp[n] for n in H.IN), inp["dy"], inp["s0"], inp["dsT"],
                          ck if ckpt_handoff else None, fused=True)
    out = dict(g)
    out["y"], out["sT"] = y, sT
    return out


def _oracle(inp, pairs=None):
    if pairs is None:
        sl = {n: H.to64(inp[n]) for n in H.IN + ("dy",)}
        s0, dsT = H.to64(inp["s0"]), H.to64(inp["dsT"])
    else:
        sl = {n: np.concatenate([H.to64(vec_slice(inp[n], b, h)) for b, h in pairs], axis=2)
              for n in H.IN + ("dy",)}
        s0 = None if inp["s0"] is None else np.concatenate(
            [H.to64(state_slice(inp["s0"], b, h)) for b, h in pairs], axis=1)
        dsT = None if inp["dsT"] is None else np.concatenate(
            [H.to64(state_slice(inp["dsT"], b, h)) for b, h in pairs], axis=1)
    y, sT = OF.forward(*(sl[n] for n in H.IN), s0=s0)
    g = OF.backward(*(sl[n] for n in H.IN), sl["dy"], s0=s0, dsT=dsT)
    g["y"], g["sT"] = y, sT
    return g


def _check(out, ref, tau, label):
    errs, bad = H.compare(out, ref, tau)
    _say(f"{label}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    assert not bad, f"{label}: over {tau:g}*RMS: {bad} {errs}"


CASES = [
    # (B, T, H, dtype, s0, dsT)
    (2, 130, 3, "f32", True, True),
    (1, 64, 2, "f32", False, False),
    (3, 33, 2, "f32", True, False),
    (2, 1, 4, "f32", True, True),
    (1, 200, 2, "bf16", True, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}_t{}_h{}_{}_s0{}_dsT{}".format(*c))
def test_fused_parity(case):
    B, T, Hh, dt, s0, dsT = case
    _say(f"case fused {case}")
    inp = make_inputs(custom(B, T, Hh, 64, dt, s0, dsT, seed=500 + T), device="cuda", fused=True)
    out = _run(inp)
    torch.cuda.synchronize()
    _check(out, _oracle(inp), H.TAU[inp["r"].dtype], f"fused{case}")


@pytest.mark.timeout(1200)
def test_fused_full_size():
    """The benchmark workload in fused form, in the benchmark's launch
    configuration; every element of every (b, h) against the fused oracle,
    streamed over batch rows."""
    wl = WORKLOADS["b8_t4096_h32_n64"]
    _say(f"case fused {wl.name} (all (b,h))")
    inp = make_inputs(wl, device="cuda", fused=True)
    out = _run(inp)
    torch.cuda.synchronize()
    for n, x in out.items():
        assert torch.isfinite(x).all(), n
    errs, bad = H.full_compare(inp, out, 2e-4, f"fused {wl.name}", oracle_fn=_oracle, say=_say)
    assert not bad, f"fused {wl.name}: {bad} {errs}"


def test_fused_recompute_matches_handoff():
    inp = make_inputs(custom(2, 150, 3, 64, "f32", True, True, seed=61), device="cuda", fused=True)
    a, b = _run(inp, True), _run(inp, False)
    for n in H.GRADS + ("ds0",):
        assert torch.equal(a[n], b[n]), n


def test_fused_matches_unfused_path():
    """The fused kernels against the plain kernels run on inputs formed by
    torch in fp32, both compared with the oracle, and with each other."""
    inp = make_inputs(custom(2, 96, 3, 64, "f32", True, True, seed=62), device="cuda", fused=True)
    fused = _run(inp)
    c = float(np.exp(-0.5))
    om, kk, ag = inp["w"], inp["a"], inp["b"]
    plain = dict(inp)
    plain["w"] = torch.exp(-c * torch.sigmoid(om))
    plain["a"] = -kk
    plain["b"] = kk * ag
    p = H.gpu_run(plain)
    sg = torch.sigmoid(om)
    chained = {"dw": p["dw"] * plain["w"] * (-c) * sg * (1 - sg), "da": -p["da"] + ag * p["db"],
               "db": kk * p["db"]}
    for n in ("y", "sT", "dr", "dk", "dv", "ds0"):
        chained[n] = p[n]
    ref = _oracle(inp)
    _check(chained, ref, 2e-4, "unfused+torch chain")
    errs, bad = H.compare({n: H.to64(x) for n, x in fused.items()},
                          {n: H.to64(x) for n, x in chained.items()}, 2e-4)
    _say("fused vs unfused: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    assert not bad, bad


def test_fused_slow_decay_whole_sequences():
    """Decay pre-activations near -6 (w ~ 0.9985) on a shape that runs one
    workgroup per (b, h) (80 heads, no split): d omega is formed from omega,
    not from the ratio of cumulative decays, and meets the bar."""
    wl = custom(2, 300, 40, 64, has_s0=True, has_dsT=True, seed=71)
    _say(f"case fused slow decay {wl.name}")
    inp = make_inputs(wl, device="cuda", fused=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(72)
    inp["w"] = -6.0 + 0.5 * torch.randn(inp["w"].shape, generator=gen, device="cuda")
    out = _run(inp)
    torch.cuda.synchronize()
    _check(out, _oracle(inp), 2e-4, "fused slow decay")
