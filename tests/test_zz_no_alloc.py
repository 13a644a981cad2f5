"""wkv7_backward_noalloc (the entry point for callers that cannot allocate:
its workspace is the library's fixed per-GPU device array) against
wkv7_backward with a caller workspace, through the C ABI (MI355X only).
Two calls in a row, the second on a smaller input, each with the forward's
checkpoint record handed over and without it (recomputed inside the
array): the results must be bit for bit those of wkv7_backward."""
import ctypes

import pytest
import torch

from linear_attention_rnn_wkv7_amd import _lib, api
from linear_attention_rnn_wkv7_amd.synthetic import custom, make_inputs

import gpu_helpers as H

pytestmark = pytest.mark.gpu

NAMES = ("dr", "dw", "dk", "dv", "da", "db", "ds0")


def _outs(inp):
    B, T, Hh, N = inp["r"].shape
    o = {n: torch.full((B, T, Hh, N), float("nan"), device="cuda") for n in NAMES[:6]}
    o["ds0"] = torch.full((B, Hh, N, N), float("nan"), device="cuda")
    return o


@pytest.mark.parametrize("handoff", [True, False], ids=["ckpt", "recompute"])
def test_noalloc_matches_backward(handoff):
    # 128 heads of 300 steps (one workgroup per head), then a smaller bf16
    # input of 6 heads of 200 steps (split into segments)
    for wl in (custom(4, 300, 32, 64, "f32", True, True, seed=31),
               custom(2, 200, 3, 64, "bf16", True, True, seed=32)):
        print(f"case noalloc {wl.name} handoff={handoff}", flush=True)
        inp = make_inputs(wl, device="cuda")
        args = [inp[n] for n in H.IN]
        _, _, ck = api.wkv7_forward(*args, inp["s0"], want_y=False, want_sT=False,
                                    want_ckpt=True)
        ck = ck if handoff else None
        ref = api.wkv7_backward(*args, inp["dy"], inp["s0"], inp["dsT"], ck)
        got = api.wkv7_backward_noalloc(*args, inp["dy"], inp["s0"], inp["dsT"], ck,
                                        out=_outs(inp))
        torch.cuda.synchronize()
        for n in NAMES:
            assert torch.equal(got[n], ref[n]), f"{wl.name}: {n} differs"
        errs, bad = H.compare(got, H.oracle_run(inp), H.TAU[inp["r"].dtype])
        print(" ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
        assert not bad, bad


def test_noalloc_rejects_oversized_shape():
    """A shape whose workspace exceeds the array is refused before anything
    is enqueued (the pointers are never touched)."""
    B, T, Hh = 16, 4096, 256      # sub-checkpoints alone: 16*256*7*16 KiB
    sh = api.make_shape(B, T, Hh, 64)
    need = api.wkv7_backward_workspace_bytes(B, T, Hh, 64, ckpt_provided=True)
    assert need > _lib.WKV7_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x10000)
    p = [fake] * 17
    p[6] = p[8] = p[16] = None
    rc = _lib.lib().wkv7_backward_noalloc(ctypes.byref(sh), *p, None)
    assert rc == _lib.WKV7_ERR_WORKSPACE
