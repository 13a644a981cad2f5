"""fp64 CPU oracle of the RWKV-8 rho / rho_norm recurrence (normalised
pre-update readout) and its exact gradient.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the test suite, the
smoke check and the benchmark's CPU-baseline leg may use it; the product
library never does.

The arithmetic lives in ``rwkv8_oracle.c`` (plain fp64 loops; the recurrence
and its gradient as the burn_dragon_kernel page src/sequence/rwkv8/backward.rs
states them in compute_chunk_traces and backward_chunk_impl); this module
marshals numpy arrays and sums the per-(b,h) value and decay gradients in a
fixed order (over heads when the value is shared, Hv = 1; over the batch for
the decay, which is one [H][L] parameter).

Shapes as on the page: query q [B, H, T, L]; value v [B, Hv, T, E] with Hv
1 or H; output y [B, H, T, E]; rho [B, H, L, E]; rho_norm [B, H, L]; decay
[H, L].
"""
import ctypes
import os

import numpy as np

from . import build as _build
from . import default_threads

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None
_LIB_PATH = None
_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64
EPS = 1e-6


def load(path=None):
    global _LIB, _LIB_PATH
    path = path or os.path.join(_HERE, "librwkv8_oracle.so")
    if _LIB is not None and _LIB_PATH == path:
        return _LIB
    if not os.path.exists(path):
        _build.build(src=os.path.join(_HERE, "rwkv8_oracle.c"), out=path)
    lib = ctypes.CDLL(path)
    lib.rwkv8_oracle_forward.restype = ctypes.c_int
    lib.rwkv8_oracle_forward.argtypes = [_dp] * 8 + [_i64] * 6 + [ctypes.c_int]
    lib.rwkv8_oracle_backward.restype = ctypes.c_int
    lib.rwkv8_oracle_backward.argtypes = [_dp] * 13 + [_i64] * 6 + [ctypes.c_int]
    _LIB, _LIB_PATH = lib, path
    return lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(_dp)


def _dims(q, v, decay):
    B, H, T, L = q.shape
    Bv, Hv, Tv, E = v.shape
    if Bv != B or Tv != T or Hv not in (1, H) or decay.shape != (H, L):
        raise ValueError(f"shapes q {q.shape} v {v.shape} decay {decay.shape}")
    return B, H, T, L, Hv, E


def forward(q, v, decay, R0=None, n0=None, want_y=True, threads=None, lib=None):
    """Return (y, RT, nT) in fp64 (y None when not wanted)."""
    q, v, decay, R0, n0 = map(_f64, (q, v, decay, R0, n0))
    B, H, T, L, Hv, E = _dims(q, v, decay)
    y = np.empty((B, H, T, E)) if want_y else None
    RT, nT = np.empty((B, H, L, E)), np.empty((B, H, L))
    lib = lib or load()
    rc = lib.rwkv8_oracle_forward(*map(_ptr, (q, v, decay, R0, n0, y, RT, nT)),
                                  B, T, H, Hv, L, E, threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"rwkv8 oracle forward failed ({rc})")
    return y, RT, nT


def backward(q, v, decay, dy, R0=None, n0=None, dRT=None, dnT=None, threads=None, lib=None):
    """Return dict dq [B,H,T,L], dv [B,Hv,T,E], ddecay [H,L], dR0 [B,H,L,E],
    dn0 [B,H,L], all fp64."""
    q, v, decay, dy, R0, n0, dRT, dnT = map(_f64, (q, v, decay, dy, R0, n0, dRT, dnT))
    B, H, T, L, Hv, E = _dims(q, v, decay)
    dq = np.empty((B, H, T, L))
    dv = np.empty((B, H, T, E))
    dd = np.empty((B, H, L))
    dR0, dn0 = np.empty((B, H, L, E)), np.empty((B, H, L))
    lib = lib or load()
    rc = lib.rwkv8_oracle_backward(*map(_ptr, (q, v, decay, R0, n0, dy, dRT, dnT, dq, dv, dd,
                                               dR0, dn0)),
                                   B, T, H, Hv, L, E, threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"rwkv8 oracle backward failed ({rc})")
    if Hv == 1:
        dv = dv.sum(axis=1, keepdims=True)
    return {"dq": dq, "dv": dv, "ddecay": dd.sum(axis=0), "dR0": dR0, "dn0": dn0}
