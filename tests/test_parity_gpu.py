"""HIP path vs the fp64 oracle, through the C ABI (MI355X only)."""
import numpy as np
import pytest
import torch

from linear_attention_rnn_wkv7_amd import api
from linear_attention_rnn_wkv7_amd.synthetic import WORKLOADS, custom, make_inputs

import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _check(out, ref, tau, label):
    errs, bad = H.compare(out, ref, tau)
    _say(f"{label}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    assert not bad, f"{label}: over {tau:g}*RMS: {bad} {errs}"


@pytest.mark.parametrize("name", ["tiny_b1_t32_h2_n16", "b4_t512_h8_n64"])
def test_parity_full(name):
    """Every output element of every (b, h) against the oracle."""
    wl = WORKLOADS[name]
    _say(f"case {name}")
    inp = make_inputs(wl, device="cuda")
    out = H.gpu_run(inp, chunk=wl.chunk)
    torch.cuda.synchronize()
    ref = H.oracle_run(inp)
    _check(out, ref, H.TAU[inp["r"].dtype], name)


FULL_SIZE = ["b8_t4096_h32_n64", "b16_t4096_h64_n64_bf16", "long_b1_t65536_h32_n64"]


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", FULL_SIZE)
def test_parity_full_size(name):
    """Full-size workloads in the benchmark's launch configuration (forward
    with checkpoints handed to the backward); every element of every output
    of every (b, h) against the oracle, streamed over batch rows and head
    groups."""
    wl = WORKLOADS[name]
    _say(f"case {name} (all (b,h))")
    inp = make_inputs(wl, device="cuda")
    out = H.gpu_run(inp, chunk=wl.chunk)
    torch.cuda.synchronize()
    for n, x in out.items():
        if x is not None:
            assert torch.isfinite(x).all(), f"{n} has non-finite values"
    tau = H.TAU[inp["r"].dtype]
    errs, bad = H.full_compare(inp, out, tau, name, say=_say)
    assert not bad, f"{name}: over {tau:g}*RMS: {bad} {errs}"


@pytest.mark.parametrize("T,algo", [(131071, "chunked"), (131072, "auto")],
                         ids=["chunk_form_at_offset_limit", "step_scan_past_limit"])
def test_offset_limit(T, algo):
    """One batch row of a vector tensor just below 2^31 bytes (B = 1, H = 64,
    T * H * 64 * 4 = 2^31 - 16 KiB) runs the chunk form with its 32-bit
    buffer offsets (forced: it must apply); at 2^31 bytes the chunk form no
    longer applies and the step scan takes every head.  Tensors of 2 GiB
    each; sampled whole recurrences against the oracle."""
    wl = custom(1, T, 64, 64, "f32", True, True, seed=71)
    _say(f"case offset limit T={T} algo={algo}")
    inp = make_inputs(wl, device="cuda")
    out = H.gpu_run(inp, algo=algo)
    torch.cuda.synchronize()
    pairs = [(0, 0), (0, 63)]
    got = H.gpu_pairs(out, pairs)
    del out
    ref = H.oracle_run(inp, pairs=pairs)
    del inp
    torch.cuda.empty_cache()
    _check(got, ref, 2e-4, f"offset limit T={T}")


EDGE = [
    # (B, T, H, N, dtype, s0, dsT, chunk)
    (1, 1, 1, 64, "f32", True, True, 64),
    (2, 7, 3, 64, "f32", True, False, 64),
    (1, 8, 2, 64, "f32", False, True, 8),
    (1, 9, 2, 64, "f32", True, True, 8),
    (2, 63, 2, 64, "f32", True, True, 16),
    (1, 64, 3, 64, "f32", True, True, 64),
    (1, 65, 2, 64, "f32", True, True, 64),
    (2, 130, 3, 64, "f32", True, True, 64),
    (1, 200, 2, 64, "f32", True, True, 24),
    (3, 77, 2, 16, "f32", True, True, 64),
    (1, 5, 4, 16, "f32", False, False, 8),
    (2, 101, 3, 64, "bf16", True, True, 64),
    (1, 37, 2, 16, "bf16", True, True, 16),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "b{}_t{}_h{}_n{}_{}_s0{}_dsT{}_c{}".format(*c))
def test_parity_edge(case):
    B, T, Hh, N, dt, s0, dsT, chunk = case
    _say(f"case edge {case}")
    wl = custom(B, T, Hh, N, dt, s0, dsT, seed=100 + T, chunk=chunk)
    inp = make_inputs(wl, device="cuda")
    out = H.gpu_run(inp, chunk=chunk)
    torch.cuda.synchronize()
    ref = H.oracle_run(inp)
    _check(out, ref, H.TAU[inp["r"].dtype], f"edge{case}")


def test_backward_recomputes_checkpoints_when_absent():
    """ckpt=NULL (recompute into workspace) gives the same bits as handing
    the forward's checkpoints over."""
    wl = custom(2, 150, 3, 64, "f32", True, True, seed=5)
    inp = make_inputs(wl, device="cuda")
    a = H.gpu_run(inp, ckpt_handoff=True)
    b = H.gpu_run(inp, ckpt_handoff=False)
    for n in H.GRADS + ("ds0",):
        assert torch.equal(a[n], b[n]), n


def test_deterministic_bitwise():
    wl = custom(2, 300, 4, 64, "f32", True, True, seed=6)
    inp = make_inputs(wl, device="cuda")
    a = H.gpu_run(inp)
    b = H.gpu_run(inp)
    for n in a:
        if a[n] is not None:
            assert torch.equal(a[n], b[n]), n


def test_chunk_interval_invariance():
    """Checkpoint interval changes only rounding."""
    wl = custom(1, 257, 4, 64, "f32", True, True, seed=8)
    inp = make_inputs(wl, device="cuda")
    outs = {c: H.gpu_run(inp, chunk=c) for c in (8, 16, 32, 64, 96, 128)}
    ref = H.oracle_run(inp)
    for c, o in outs.items():
        _check(o, ref, 2e-4, f"chunk{c}")


def test_split_sequence_gpu():
    """fwd over [0,T) == fwd over [T1,T) from the state at T1; backward of the
    second half hands ds0 to the first half as dsT."""
    wl = custom(2, 200, 3, 64, "f32", True, True, seed=9)
    inp = make_inputs(wl, device="cuda")
    full = H.gpu_run(inp)
    T1 = 72
    first = {n: (x[:, :T1].contiguous() if n in H.IN + ("dy",) else x) for n, x in inp.items()}
    second = {n: (x[:, T1:].contiguous() if n in H.IN + ("dy",) else x) for n, x in inp.items()}
    _, s_mid, _ = api.wkv7_forward(*(first[n] for n in H.IN), first["s0"], want_y=False)
    second["s0"] = s_mid
    o2 = H.gpu_run(second)
    first["dsT"] = o2["ds0"]
    o1 = H.gpu_run(first)
    ref = H.oracle_run(inp)
    cat = {n: torch.cat([o1[n], o2[n]], 1) for n in ("y",) + H.GRADS}
    cat["sT"], cat["ds0"] = o2["sT"], o1["ds0"]
    _check(cat, ref, 2e-4, "split")


def test_empty_time_axis():
    """T = 0: sT = s0 and ds0 = dsT (zeros when absent)."""
    wl = custom(2, 0, 3, 64, "f32", True, True, seed=10)
    inp = make_inputs(wl, device="cuda")
    y, sT, _ = api.wkv7_forward(*(inp[n] for n in H.IN), inp["s0"])
    g = api.wkv7_backward(*(inp[n] for n in H.IN), inp["dy"], inp["s0"], inp["dsT"])
    assert torch.equal(sT, inp["s0"]) and torch.equal(g["ds0"], inp["dsT"])
    _, sT0, _ = api.wkv7_forward(*(inp[n] for n in H.IN), None)
    g0 = api.wkv7_backward(*(inp[n] for n in H.IN), inp["dy"], None, None)
    assert not sT0.any() and not g0["ds0"].any()
    assert y.shape == (2, 0, 3, 64)
