"""The single-step forward (T = 1, the decode step of batched inference)
against the fp64 oracle, through the C ABI (MI355X only)."""
import pytest
import torch

from linear_attention_rnn_wkv7_amd import api
from linear_attention_rnn_wkv7_amd.synthetic import WORKLOADS, custom, make_inputs

import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _check(out, ref, tau, label, names=("y", "sT")):
    errs, bad = H.compare(out, ref, tau, names=names)
    _say(f"{label}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    assert not bad, f"{label}: over {tau:g}*RMS: {bad} {errs}"


def _oracle_fwd(inp):
    import oracle
    y, sT = oracle.forward(*(H.to64(inp[n]) for n in H.IN), s0=H.to64(inp["s0"]))
    return {"y": y, "sT": sT}


DECODE = [
    # (B, H, N, dtype, s0)
    (3, 5, 16, "f32", True),
    (2, 3, 64, "f32", False),
    (4, 7, 64, "bf16", True),
    (1, 1, 16, "bf16", False),
    (5, 2, 16, "f32", True),
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "b{}_h{}_n{}_{}_s0{}".format(*c))
def test_decode_parity(case):
    B, Hh, N, dt, s0 = case
    _say(f"case decode {case}")
    inp = make_inputs(custom(B, 1, Hh, N, dt, s0, False, seed=300 + B * Hh), device="cuda")
    y, sT, _ = api.wkv7_forward(*(inp[n] for n in H.IN), inp["s0"])
    torch.cuda.synchronize()
    _check({"y": y, "sT": sT}, _oracle_fwd(inp), H.TAU[inp["r"].dtype], f"decode{case}")


def test_decode_batched_workload():
    """The batched decode workload (every (b, h)) against the oracle."""
    wl = WORKLOADS["decode_b256_t1_h32_n64"]
    _say(f"case {wl.name}")
    inp = make_inputs(wl, device="cuda")
    y, sT, _ = api.wkv7_forward(*(inp[n] for n in H.IN), inp["s0"])
    torch.cuda.synchronize()
    _check({"y": y, "sT": sT}, _oracle_fwd(inp), 2e-4, wl.name)


def test_decode_optional_outputs_and_record():
    """Skipped outputs change nothing else; the checkpoint record of a single
    step is the carry-in state and sa = s0 a; the backward consumes it."""
    inp = make_inputs(custom(3, 1, 4, 64, "f32", True, True, seed=77), device="cuda")
    args = [inp[n] for n in H.IN]
    y, sT, ck = api.wkv7_forward(*args, inp["s0"], want_ckpt=True)
    y1, sT1, _ = api.wkv7_forward(*args, inp["s0"], want_sT=False)
    y2, sT2, _ = api.wkv7_forward(*args, inp["s0"], want_y=False)
    assert sT1 is None and y2 is None
    assert torch.equal(y, y1) and torch.equal(sT, sT2)
    B, Hh, N = 3, 4, 64
    slots = B * Hh * N * N
    assert torch.equal(ck[:slots].view(B, Hh, N, N), inp["s0"])
    tape = ck[-B * Hh * N:].view(B, 1, Hh, N).cpu().double()
    sa = torch.einsum("bhij,bhj->bhi", inp["s0"].cpu().double(), inp["a"][:, 0].cpu().double())
    assert torch.allclose(tape[:, 0], sa, rtol=1e-5, atol=1e-6)
    g = api.wkv7_backward(*args, inp["dy"], inp["s0"], inp["dsT"], ck)
    ref = H.oracle_run(inp)
    _check(g, ref, 2e-4, "decode backward", names=H.GRADS + ("ds0",))


def test_decode_in_place_state():
    """T = 1 with sT = s0: the state is updated in place, with the same bits
    as into a separate buffer."""
    inp = make_inputs(custom(4, 1, 6, 64, "f32", True, False, seed=55), device="cuda")
    args = [inp[n] for n in H.IN]
    y, sT, _ = api.wkv7_forward(*args, inp["s0"])
    s = inp["s0"].clone()
    y2, s2, _ = api.wkv7_forward(*args, s, out=(None, s, None))
    torch.cuda.synchronize()
    assert s2.data_ptr() == s.data_ptr()
    assert torch.equal(s, sT) and torch.equal(y, y2)


def test_decode_rollout_matches_sequence():
    """T decode steps, each fed the previous state, give the sequence's y and
    final state (the split-sequence property at every step)."""
    T = 40
    inp = make_inputs(custom(2, T, 3, 64, "f32", True, False, seed=91), device="cuda")
    s = inp["s0"]
    ys = []
    for t in range(T):
        step = [inp[n][:, t:t + 1].contiguous() for n in H.IN]
        y, s, _ = api.wkv7_forward(*step, s)
        ys.append(y)
    torch.cuda.synchronize()
    _check({"y": torch.cat(ys, 1), "sT": s}, _oracle_fwd(inp), 2e-4, "rollout")
