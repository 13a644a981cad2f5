"""The RWKV-8 rho / rho_norm recurrence on the device (rwkv8_forward,
rwkv8_backward through the C ABI) against the fp64 oracle (oracle.rwkv8),
MI355X only.  Every element of every output.

Bar, per element x of each output tensor X:
    |x_gpu - x_ref| <= 2e-4 * (RMS(X_ref) + |x_ref|)
the fp32 bar of the WKV7 path (2e-4 of the RMS) widened by the element's own
size.  The readout divides by rho_norm + 1e-6, and dL/dq picks up
1 / (n + 1e-6)^2 where a latent's norm has decayed over a run of zero
queries: such elements reach 10^3 - 10^4 times the tensor's RMS, and fp32
rounding of them is relative to their own magnitude.  The plain
max|err| / RMS figure is printed beside it."""
import ctypes

import numpy as np
import pytest
import torch

import oracle.rwkv8 as R8
from linear_attention_rnn_wkv7_amd import _lib, api
from linear_attention_rnn_wkv7_amd.synthetic import (RWKV8_WORKLOADS, make_rwkv8_inputs,
                                                     rwkv8_custom)

pytestmark = pytest.mark.gpu
TAU = 2e-4
OUTS = ("y", "rhoT", "normT", "dq", "dv", "ddecay", "drho0", "dnorm0")


def _say(msg):
    print(msg, flush=True)


def _gpu(inp, handoff=True):
    y, rT, nT, ck = api.rwkv8_forward(inp["q"], inp["v"], inp["decay"], inp["rho0"], inp["norm0"],
                                      want_ckpt=handoff)
    g = api.rwkv8_backward(inp["q"], inp["v"], inp["decay"], inp["dy"], inp["rho0"], inp["norm0"],
                           inp["drhoT"], inp["dnormT"], ck)
    out = dict(g)
    out.update(y=y, rhoT=rT, normT=nT)
    return out


def _oracle(inp):
    y, rT, nT = R8.forward(inp["q"], inp["v"], inp["decay"], inp["rho0"], inp["norm0"])
    g = R8.backward(inp["q"], inp["v"], inp["decay"], inp["dy"], inp["rho0"], inp["norm0"],
                    inp["drhoT"], inp["dnormT"])
    g["drho0"], g["dnorm0"] = g.pop("dR0"), g.pop("dn0")
    g.update(y=y, rhoT=rT, normT=nT)
    return g


def _compare(got, ref, label, tau=TAU):
    errs, mixed, bad = {}, {}, []
    for n in OUTS:
        if got.get(n) is None:
            continue
        assert ref.get(n) is not None, f"no reference for {n}"
        g = got[n].detach().cpu().double().numpy()
        r = ref[n]
        if r.size == 0:
            continue
        rms = float(np.sqrt(np.mean(r * r)))
        err = np.abs(g - r)
        errs[n] = float(np.max(err)) / max(rms, 1e-30)
        mixed[n] = float(np.max(err / (rms + np.abs(r) + 1e-30)))
        if not np.isfinite(mixed[n]) or mixed[n] > tau:
            bad.append(n)
    _say(f"{label}: max|err|/RMS " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    _say(f"{label}: max|err|/(RMS+|ref|) " + " ".join(f"{n}={e:.2e}" for n, e in mixed.items()))
    assert not bad, f"{label}: over {tau:g}*(RMS+|ref|): {bad} {mixed}"


CASES = [
    # (B, T, H, Hv, state, final grads)
    (1, 1, 1, 1, True, True),
    (2, 16, 2, 2, True, True),
    (1, 17, 3, 3, False, True),
    (2, 64, 2, 1, True, False),
    (1, 65, 2, 2, True, True),
    (2, 100, 3, 1, True, True),
    (1, 200, 2, 2, False, False),
    (3, 257, 4, 4, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}_t{}_h{}_hv{}_s{}_g{}".format(*c))
def test_rwkv8_parity(case):
    B, T, H, Hv, st, fg = case
    _say(f"case rwkv8 {case}")
    inp = make_rwkv8_inputs(rwkv8_custom(B, T, H, Hv, st, fg, seed=3000 + T), device="cuda")
    out = _gpu(inp)
    torch.cuda.synchronize()
    _compare(out, _oracle(inp), f"rwkv8 {case}")


def test_rwkv8_unit_decay_and_recompute():
    """decay = 1 (the top of the domain) and the backward recomputing the
    checkpoint record itself: bitwise the same as with the record handed
    over, and against the oracle."""
    wl = rwkv8_custom(2, 150, 3, 3, True, True, seed=3101)
    inp = make_rwkv8_inputs(wl, device="cuda")
    inp["decay"] = torch.ones_like(inp["decay"])
    a, b = _gpu(inp, True), _gpu(inp, False)
    torch.cuda.synchronize()
    for n in ("dq", "dv", "ddecay", "drho0", "dnorm0"):
        assert torch.equal(a[n], b[n]), n
    _compare(a, _oracle(inp), "rwkv8 decay 1")


def test_rwkv8_low_decay_edge():
    """Decays at the bottom of the domain (2^-7) and just above."""
    wl = rwkv8_custom(1, 90, 2, 2, True, True, seed=3102)
    inp = make_rwkv8_inputs(wl, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3103)
    inp["decay"] = 2.0 ** -7 + 0.01 * torch.rand(inp["decay"].shape, generator=gen, device="cuda")
    inp["decay"][0, 0] = 2.0 ** -7
    out = _gpu(inp)
    torch.cuda.synchronize()
    _compare(out, _oracle(inp), "rwkv8 low decay")


def test_rwkv8_out_of_domain_decay_is_loud():
    """A head with a decay outside [2^-7, 1] gets NaN outputs and the fault
    bit; the other heads are unaffected and correct."""
    L = _lib.lib()
    f = ctypes.c_uint(0)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.wkv7_fault_status(ctypes.byref(f), 1, s) == 0
    wl = rwkv8_custom(2, 70, 3, 3, True, True, seed=3104)
    inp = make_rwkv8_inputs(wl, device="cuda")
    inp["decay"][1, 5] = 1e-3
    out = _gpu(inp)
    torch.cuda.synchronize()
    assert L.wkv7_fault_status(ctypes.byref(f), 1, s) == 0
    assert f.value & _lib.WKV7_FAULT_RWKV8_DECAY
    for n in ("y", "dq", "dv", "drho0", "dnorm0", "rhoT", "normT"):
        assert torch.isnan(out[n][:, 1]).all(), n
        assert torch.isfinite(out[n][:, 0]).all() and torch.isfinite(out[n][:, 2]).all(), n
    assert torch.isnan(out["ddecay"][1]).all() and torch.isfinite(out["ddecay"][0]).all()
    ref = _oracle(inp)
    keep = [0, 2]
    got = {n: out[n][:, keep] for n in ("y", "dq", "dv", "drho0", "dnorm0", "rhoT", "normT")}
    got["ddecay"] = out["ddecay"][keep]
    refk = {n: ref[n][:, keep] for n in ("y", "dq", "dv", "drho0", "dnorm0", "rhoT", "normT")}
    refk["ddecay"] = ref["ddecay"][keep]
    _compare(got, refk, "rwkv8 other heads")


def test_rwkv8_deterministic_and_empty():
    wl = rwkv8_custom(2, 130, 3, 1, True, True, seed=3105)
    inp = make_rwkv8_inputs(wl, device="cuda")
    a, b = _gpu(inp), _gpu(inp)
    for n in OUTS:
        assert torch.equal(a[n], b[n]), n
    e = make_rwkv8_inputs(rwkv8_custom(2, 0, 3, 3, True, True, seed=3106), device="cuda")
    out = _gpu(e, handoff=False)
    torch.cuda.synchronize()
    assert torch.equal(out["rhoT"], e["rho0"]) and torch.equal(out["normT"], e["norm0"])
    assert torch.equal(out["drho0"], e["drhoT"]) and torch.equal(out["dnorm0"], e["dnormT"])
    assert not out["ddecay"].any()


@pytest.mark.timeout(1200)
def test_rwkv8_full_size():
    """The benchmark workload (8 x 4096 x 32 heads, carry-in state): every
    element of every output against the oracle."""
    wl = RWKV8_WORKLOADS["rwkv8_b8_t4096_h32"]
    _say(f"case {wl.name}")
    inp = make_rwkv8_inputs(wl, device="cuda")
    out = _gpu(inp)
    torch.cuda.synchronize()
    for n, x in out.items():
        if x is not None:
            assert torch.isfinite(x).all(), n
    _compare(out, _oracle(inp), wl.name)
