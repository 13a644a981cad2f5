"""Few, long sequences run in segments (the library splits a shape with at
most 64 (b, h) pairs into up to 8 segments of at least 2 chunks, carrying
states and state gradients between them): against the oracle, through the
C ABI (MI355X only)."""
import numpy as np
import pytest
import torch

import oracle.fused as OF
from linear_attention_rnn_wkv7_amd import api
from linear_attention_rnn_wkv7_amd.synthetic import custom, make_inputs

import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _check(out, ref, tau, label):
    errs, bad = H.compare(out, ref, tau)
    _say(f"{label}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    assert not bad, f"{label}: over {tau:g}*RMS: {bad} {errs}"


# (B, T, H, dtype, s0, dsT): 8 segments of 2 chunks; 8 of 8 chunks; 8 of 4
# with a ragged last chunk; bf16 (8 of 3); 7 segments, the last one chunk of
# 15 steps (a partial 32-step block; the forward without a record runs whole)
CASES = [
    (1, 1024, 2, "f32", True, True),
    (1, 4096, 4, "f32", False, True),
    (2, 2000, 3, "f32", True, True),
    (1, 1536, 2, "bf16", True, True),
    (1, 1551, 1, "f32", True, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}_t{}_h{}_{}_s0{}_dsT{}".format(*c))
def test_split_parity(case):
    B, T, Hh, dt, s0, dsT = case
    wl = custom(B, T, Hh, 64, dtype=dt, has_s0=s0, has_dsT=dsT, seed=700 + T)
    _say(f"case split {wl.name}")
    inp = make_inputs(wl, device="cuda")
    out = H.gpu_run(inp)
    torch.cuda.synchronize()
    _check(out, H.oracle_run(inp), H.TAU[inp["r"].dtype], wl.name)


def test_split_recompute_and_scan():
    """The backward recomputing the (split) forward into its workspace gives
    the same bits as the handed-over record; the step scan (no split in the
    backward) reads the same record."""
    wl = custom(1, 2048, 3, 64, has_s0=True, has_dsT=True, seed=31)
    inp = make_inputs(wl, device="cuda")
    a = H.gpu_run(inp, ckpt_handoff=True)
    b = H.gpu_run(inp, ckpt_handoff=False)
    for n in H.GRADS + ("ds0",):
        assert torch.equal(a[n], b[n]), n
    s = H.gpu_run(inp, algo="scan")
    ref = H.oracle_run(inp)
    _check(s, ref, 2e-4, "scan on the split record")


def test_split_fused():
    wl = custom(1, 2048, 2, 64, has_s0=True, has_dsT=True, seed=41)
    _say(f"case split fused {wl.name}")
    inp = make_inputs(wl, device="cuda", fused=True)
    y, sT, ck = api.wkv7_forward(*(inp[n] for n in H.IN), inp["s0"], want_ckpt=True, fused=True)
    g = api.wkv7_backward(*(inp[n] for n in H.IN), inp["dy"], inp["s0"], inp["dsT"], ck, fused=True)
    torch.cuda.synchronize()
    out = dict(g)
    out["y"], out["sT"] = y, sT
    sl = {n: H.to64(inp[n]) for n in H.IN + ("dy",)}
    ry, rs = OF.forward(*(sl[n] for n in H.IN), s0=H.to64(inp["s0"]))
    ref = OF.backward(*(sl[n] for n in H.IN), sl["dy"], s0=H.to64(inp["s0"]), dsT=H.to64(inp["dsT"]))
    ref["y"], ref["sT"] = ry, rs
    _check(out, ref, 2e-4, "split fused")


def test_split_falls_back_per_head():
    """A head with a decay out of the chunk form's range in any segment is
    redone whole by the step scan (bitwise equal to it); the others are not."""
    wl = custom(2, 1280, 3, 64, has_s0=True, has_dsT=True, seed=23)
    _say(f"case split fallback {wl.name}")
    inp = make_inputs(wl, device="cuda")
    w = inp["w"]
    w[1, 1000, 2, 7] = 0.0         # a decay of 0 in the sixth of 7 segments
    w[0, 100:120, 1, :] = 0.02     # decays below 1/16 in the first segment
    flagged = [(1, 2), (0, 1)]
    a = H.gpu_run(inp)
    s = H.gpu_run(inp, algo="scan")
    torch.cuda.synchronize()
    _check(a, H.oracle_run(inp), 2e-4, "split fallback")
    for b in range(wl.B):
        for h in range(wl.H):
            same = all(torch.equal(a[n][b, :, h], s[n][b, :, h]) for n in H.GRADS) and \
                torch.equal(a["ds0"][b, h], s["ds0"][b, h])
            assert same == ((b, h) in flagged), (b, h, same)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}_t{}_h{}_{}_s0{}_dsT{}".format(*c))
def test_split_inference(case):
    """The forward without a checkpoint record runs split with its carries in
    y's rows: the same bits as the forward with a record, y prefilled with
    NaN (every row is overwritten), against the oracle."""
    B, T, Hh, dt, s0, _ = case
    wl = custom(B, T, Hh, 64, dtype=dt, has_s0=s0, has_dsT=False, seed=800 + T)
    _say(f"case split inference {wl.name}")
    inp = make_inputs(wl, device="cuda")
    y0 = torch.full((B, T, Hh, 64), float("nan"), device="cuda")
    y, sT, _ = api.wkv7_forward(*(inp[n] for n in H.IN), inp["s0"], out=(y0, None, None))
    yc, sTc, _ = api.wkv7_forward(*(inp[n] for n in H.IN), inp["s0"], want_ckpt=True)
    torch.cuda.synchronize()
    assert torch.equal(y, yc) and torch.equal(sT, sTc)
    sl = {n: H.to64(inp[n]) for n in H.IN}
    import oracle
    ry, rs = oracle.forward(*(sl[n] for n in H.IN), s0=H.to64(inp["s0"]))
    _check({"y": y, "sT": sT}, {"y": ry, "sT": rs}, H.TAU[inp["r"].dtype], wl.name)


def test_split_inference_fused_and_state_only():
    """Fused inputs without a record (split, carries in y); and sT alone
    (no y to hold the carries: one pass per (b, h))."""
    wl = custom(1, 2048, 2, 64, has_s0=True, has_dsT=False, seed=43)
    _say(f"case split inference fused {wl.name}")
    inp = make_inputs(wl, device="cuda", fused=True)
    y, sT, _ = api.wkv7_forward(*(inp[n] for n in H.IN), inp["s0"], fused=True)
    _, sT2, _ = api.wkv7_forward(*(inp[n] for n in H.IN), inp["s0"], want_y=False, fused=True)
    torch.cuda.synchronize()
    sl = {n: H.to64(inp[n]) for n in H.IN}
    ry, rs = OF.forward(*(sl[n] for n in H.IN), s0=H.to64(inp["s0"]))
    _check({"y": y, "sT": sT}, {"y": ry, "sT": rs}, 2e-4, "split inference fused")
    _check({"sT": sT2}, {"sT": rs}, 2e-4, "state only, fused")


SLOW = [(1, 1024, 2, True), (2, 2000, 3, True), (1, 4096, 4, False)]


@pytest.mark.parametrize("case", SLOW, ids=lambda c: "b{}_t{}_h{}_s0{}".format(*c))
def test_split_slow_decay(case):
    """Decays in [0.99, 1): a segment's carry-in state survives its 128 or
    more steps (0.995^128 ~ 0.5), so the transition products P and the
    compose kernels decide the later segments' results, forward (with and
    without a record) and backward.  With the workloads' decays (median
    0.74) the carry-in fades below an ulp within a segment."""
    B, T, Hh, s0 = case
    wl = custom(B, T, Hh, 64, has_s0=s0, has_dsT=True, seed=900 + T)
    _say(f"case split slow decay {wl.name}")
    inp = make_inputs(wl, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(17 + T)
    inp["w"] = 1.0 - 0.01 * torch.rand(inp["w"].shape, generator=gen, device="cuda")
    out = H.gpu_run(inp)
    y0 = torch.full((B, T, Hh, 64), float("nan"), device="cuda")
    yi, sTi, _ = api.wkv7_forward(*(inp[n] for n in H.IN), inp["s0"], out=(y0, None, None))
    torch.cuda.synchronize()
    ref = H.oracle_run(inp)
    _check(out, ref, 2e-4, f"slow decay {wl.name}")
    _check({"y": yi, "sT": sTi}, ref, 2e-4, f"slow decay inference {wl.name}")
    # these inputs make the carry matter: the second half's y from a zero
    # state is far from the true one
    import oracle
    half = {n: H.to64(inp[n])[:, T // 2:] for n in H.IN}
    yz, _ = oracle.forward(*(half[n] for n in H.IN))
    yt = ref["y"][:, T // 2:]
    assert np.abs(yz - yt).max() > 0.1 * np.sqrt(np.mean(yt * yt))


def test_split_slow_decay_fused():
    """Fused inputs with decay pre-activations near -6 (w = exp(-e^-0.5
    sigmoid(omega)) ~ 0.9985): the carries matter, through the fused forms of
    both passes of the split, against the fused oracle."""
    wl = custom(1, 2048, 3, 64, has_s0=True, has_dsT=True, seed=61)
    _say(f"case split slow decay fused {wl.name}")
    inp = make_inputs(wl, device="cuda", fused=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(62)
    inp["w"] = -6.0 + 0.5 * torch.randn(inp["w"].shape, generator=gen, device="cuda")
    y, sT, ck = api.wkv7_forward(*(inp[n] for n in H.IN), inp["s0"], want_ckpt=True, fused=True)
    g = api.wkv7_backward(*(inp[n] for n in H.IN), inp["dy"], inp["s0"], inp["dsT"], ck, fused=True)
    yi, sTi, _ = api.wkv7_forward(*(inp[n] for n in H.IN), inp["s0"], fused=True)
    torch.cuda.synchronize()
    out = dict(g)
    out["y"], out["sT"] = y, sT
    sl = {n: H.to64(inp[n]) for n in H.IN + ("dy",)}
    ry, rs = OF.forward(*(sl[n] for n in H.IN), s0=H.to64(inp["s0"]))
    ref = OF.backward(*(sl[n] for n in H.IN), sl["dy"], s0=H.to64(inp["s0"]), dsT=H.to64(inp["dsT"]))
    ref["y"], ref["sT"] = ry, rs
    _check(out, ref, 2e-4, "split slow decay fused")
    _check({"y": yi, "sT": sTi}, {"y": ry, "sT": rs}, 2e-4, "split slow decay fused, no record")
    # the carry matters: the second half's y from a zero state is far off
    half = {n: sl[n][:, 1024:] for n in H.IN}
    yz, _ = OF.forward(*(half[n] for n in H.IN))
    yt = ry[:, 1024:]
    assert np.abs(yz - yt).max() > 0.1 * np.sqrt(np.mean(yt * yt))
