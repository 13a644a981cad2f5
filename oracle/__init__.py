"""fp64 CPU oracle of the WKV7 recurrence and its reverse scan.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does.

The arithmetic lives in ``wkv7_oracle.c`` (plain loops, fp64); this module
only marshals numpy arrays.  Shapes: vectors ``[B, T, H, N]``, states
``[B, H, N, N]`` (row i = value index, column j = key index), as on the
Foundry "rwkvx/rx_pretrain.c" page (rx_wkv7_forward_seq, rx_wkv7_backward).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None
_LIB_PATH = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def load(path=None):
    """Load (building first if absent) the oracle shared library."""
    global _LIB, _LIB_PATH
    path = path or os.path.join(_HERE, "libwkv7_oracle.so")
    if _LIB is not None and _LIB_PATH == path:
        return _LIB
    if not os.path.exists(path):
        _build.build(out=path)
    lib = ctypes.CDLL(path)
    lib.wkv7_oracle_forward.restype = ctypes.c_int
    lib.wkv7_oracle_forward.argtypes = [_dp] * 9 + [_i64] * 4 + [ctypes.c_int]
    lib.wkv7_oracle_backward.restype = ctypes.c_int
    lib.wkv7_oracle_backward.argtypes = [_dp] * 16 + [_i64] * 4 + [ctypes.c_int]
    _LIB, _LIB_PATH = lib, path
    return lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(_dp)


def default_threads():
    """Host cores available to this process, capped by OMP_NUM_THREADS when
    that is set (a machine shared by several jobs sets it to each job's
    share)."""
    try:
        n = max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return n


def _check(shape_v, *arrs):
    for x in arrs:
        if x is not None and x.shape != shape_v:
            raise ValueError(f"shape {x.shape} != {shape_v}")


def forward(r, w, k, v, a, b, s0=None, want_y=True, want_sT=True, threads=None,
            lib=None):
    """Return ``(y, sT)`` in fp64 (either is None when not wanted)."""
    r, w, k, v, a, b, s0 = map(_f64, (r, w, k, v, a, b, s0))
    B, T, H, N = r.shape
    _check(r.shape, w, k, v, a, b)
    if s0 is not None and s0.shape != (B, H, N, N):
        raise ValueError("s0 shape")
    y = np.empty((B, T, H, N)) if want_y else None
    sT = np.empty((B, H, N, N)) if want_sT else None
    lib = lib or load()
    rc = lib.wkv7_oracle_forward(*map(_ptr, (r, w, k, v, a, b, s0, y, sT)),
                                 B, T, H, N, threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle forward failed ({rc})")
    return y, sT


def backward(r, w, k, v, a, b, dy, s0=None, dsT=None, want_ds0=True,
             threads=None, lib=None):
    """Return a dict of fp64 gradients: dr, dw, dk, dv, da, db, ds0."""
    r, w, k, v, a, b, dy, s0, dsT = map(_f64, (r, w, k, v, a, b, dy, s0, dsT))
    B, T, H, N = r.shape
    _check(r.shape, w, k, v, a, b, dy)
    for s in (s0, dsT):
        if s is not None and s.shape != (B, H, N, N):
            raise ValueError("state shape")
    out = {n: np.empty((B, T, H, N)) for n in ("dr", "dw", "dk", "dv", "da", "db")}
    out["ds0"] = np.empty((B, H, N, N)) if want_ds0 else None
    lib = lib or load()
    rc = lib.wkv7_oracle_backward(
        *map(_ptr, (r, w, k, v, a, b, dy, s0, dsT,
                    out["dr"], out["dw"], out["dk"], out["dv"], out["da"], out["db"],
                    out["ds0"])),
        B, T, H, N, threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle backward failed ({rc})")
    return out
