"""Failure reporting through the C ABI (MI355X only).  Every condition is
forced from the host with the library's test hooks, so every kernel still
runs and exits normally:
  * a forward helper wait reported as given up: every output the forward
    wrote is NaN and the device's fault bit is set (no finite wrong value);
  * a launch reported as failed: the call returns WKV7_ERR_HIP and the
    binding raises."""
import ctypes

import pytest
import torch

from linear_attention_rnn_wkv7_amd import _lib, api
from linear_attention_rnn_wkv7_amd.synthetic import custom, make_inputs

import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _faults(clear=True):
    f = ctypes.c_uint(0xFFFFFFFF)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert _lib.lib().wkv7_fault_status(ctypes.byref(f), int(clear), s) == _lib.WKV7_OK
    return f.value


def _forward(inp):
    return api.wkv7_forward(*(inp[n] for n in H.IN), inp["s0"], want_ckpt=True)


# (B, T, H): 80 heads run one workgroup per (b, h); 6 heads of 200 steps run
# split into two segments (the transition-product pass and the output pass)
@pytest.mark.parametrize("B,T,Hh", [(2, 200, 40), (2, 200, 3)], ids=["whole", "split"])
def test_given_up_wait_poisons_outputs(B, T, Hh):
    L = _lib.lib()
    inp = make_inputs(custom(B, T, Hh, 64, "f32", True, True, seed=21), device="cuda")
    print(f"case fault inject B={B} T={T} H={Hh}", flush=True)
    _faults()   # start clear
    assert L.wkv7_test_hook(_lib.WKV7_HOOK_FAULT_INJECT, 1) == _lib.WKV7_OK
    try:
        y, sT, ck = _forward(inp)
        torch.cuda.synchronize()
    finally:
        assert L.wkv7_test_hook(_lib.WKV7_HOOK_FAULT_INJECT, 0) == _lib.WKV7_OK
    assert _faults() & _lib.WKV7_FAULT_HELPER_WAIT
    assert torch.isnan(y).all() and torch.isnan(sT).all()
    states = B * Hh * ((T + 63) // 64) * 64 * 64
    tape = B * T * Hh * 64
    assert torch.isnan(ck[:states]).all()
    off = (states * 4 + 255) // 256 * 64   # the tape starts 256-byte aligned
    assert torch.isnan(ck[off:off + tape]).all()
    # the bit stays clear and the results are right once the hook is off
    out = H.gpu_run(inp)
    torch.cuda.synchronize()
    assert _faults() == 0
    errs, bad = H.compare(out, H.oracle_run(inp), 2e-4)
    print(" ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    assert not bad, bad


def test_failed_launch_status():
    L = _lib.lib()
    inp = make_inputs(custom(1, 70, 2, 64, "f32", True, False, seed=22), device="cuda")
    assert L.wkv7_test_hook(_lib.WKV7_HOOK_FAIL_LAUNCHES, 1) == _lib.WKV7_OK
    try:
        with pytest.raises(_lib.Wkv7Error) as e:
            _forward(inp)
        assert e.value.status == _lib.WKV7_ERR_HIP
    finally:
        L.wkv7_test_hook(_lib.WKV7_HOOK_FAIL_LAUNCHES, 0)
    torch.cuda.synchronize()
    y, sT, ck = _forward(inp)   # the next call is not affected
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    # the backward reports its failed launch the same way
    assert L.wkv7_test_hook(_lib.WKV7_HOOK_FAIL_LAUNCHES, 1) == _lib.WKV7_OK
    try:
        with pytest.raises(_lib.Wkv7Error) as e:
            api.wkv7_backward(*(inp[n] for n in H.IN), inp["dy"], inp["s0"], inp["dsT"], ck)
        assert e.value.status == _lib.WKV7_ERR_HIP
    finally:
        L.wkv7_test_hook(_lib.WKV7_HOOK_FAIL_LAUNCHES, 0)
    torch.cuda.synchronize()
    g = api.wkv7_backward(*(inp[n] for n in H.IN), inp["dy"], inp["s0"], inp["dsT"], ck)
    torch.cuda.synchronize()
    assert all(torch.isfinite(x).all() for x in g.values() if x is not None)
