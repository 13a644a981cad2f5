"""Thin torch-facing binding of the libwkv7 C ABI.

Argument marshalling only: torch allocates device memory and supplies the
stream; every step of the recurrence runs in the library's HIP kernels.
Names mirror the C entry points (include/wkv7.h).
"""
import ctypes

import torch

from . import _lib

_VEC_DTYPES = {torch.float32: _lib.WKV7_F32, torch.bfloat16: _lib.WKV7_BF16}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocate the buffers a call creates on the stream its kernels run on,
    so that the caching allocator does not hand their memory to other work
    before those kernels are done with it."""
    return torch.cuda.stream(stream) if stream is not None else _Nothing()


class _Nothing:
    def __enter__(self):
        return None

    def __exit__(self, *exc):
        return False


_ALGOS = {"auto": _lib.WKV7_ALGO_AUTO, "scan": _lib.WKV7_ALGO_SCAN,
          "chunked": _lib.WKV7_ALGO_CHUNKED}


def make_shape(B, T, H, N, dtype=torch.float32, chunk=64, algo="auto", fused=False):
    return _lib.Shape(B, T, H, N, _VEC_DTYPES[dtype], chunk, _ALGOS[algo],
                      _lib.WKV7_FUSED_INPUTS if fused else 0)


def _check_vecs(names, tensors):
    ref = tensors[0]
    if ref.dim() != 4:
        raise ValueError(f"{names[0]} must be [B, T, H, N]")
    if ref.dtype not in _VEC_DTYPES:
        raise ValueError(f"{names[0]}: dtype {ref.dtype} not supported")
    for n, t in zip(names, tensors):
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError(f"{n}: shape/dtype must match {names[0]}")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous device tensor")
    return tuple(ref.shape), ref.dtype


def _check_state(name, t, B, H, N):
    if t is None:
        return
    if t.shape != (B, H, N, N) or t.dtype != torch.float32 or not t.is_cuda \
            or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous fp32 device tensor [B, H, N, N]")


def wkv7_checkpoint_bytes(B, T, H, N, dtype=torch.float32, chunk=64):
    sh = make_shape(B, T, H, N, dtype, chunk)
    return _lib.lib().wkv7_checkpoint_bytes(ctypes.byref(sh))


def wkv7_backward_workspace_bytes(B, T, H, N, dtype=torch.float32, chunk=64, ckpt_provided=True):
    sh = make_shape(B, T, H, N, dtype, chunk)
    return _lib.lib().wkv7_backward_workspace_bytes(ctypes.byref(sh), int(bool(ckpt_provided)))


def wkv7_forward(r, w, k, v, a, b, s0=None, *, chunk=64, want_y=True, want_sT=True,
                 want_ckpt=False, stream=None, out=None, fused=False):
    """Run the forward scan.  Returns (y, sT, ckpt); unwanted outputs are None.

    fused=True (WKV7_FUSED_INPUTS): w, a, b carry omega, kk and the gate, and
    the library forms w = exp(-exp(-0.5) sigmoid(omega)), a = -kk, b = kk gate.

    ckpt is the flat fp32 checkpoint record (states every `chunk` steps, then
    the per-step sa) that wkv7_backward consumes.

    ``out`` may supply preallocated (y, sT, ckpt) tensors (None entries are
    allocated when wanted)."""
    (B, T, H, N), dt = _check_vecs("rwkvab", (r, w, k, v, a, b))
    _check_state("s0", s0, B, H, N)
    dev = r.device
    y, sT, ckpt = out if out is not None else (None, None, None)
    with _on(stream):
        if want_y and y is None:
            y = torch.empty((B, T, H, N), device=dev, dtype=torch.float32)
        if want_sT and sT is None:
            sT = torch.empty((B, H, N, N), device=dev, dtype=torch.float32)
        if want_ckpt and ckpt is None:
            ckpt = torch.empty(wkv7_checkpoint_bytes(B, T, H, N, dt, chunk) // 4, device=dev,
                               dtype=torch.float32)
    sh = make_shape(B, T, H, N, dt, chunk, fused=fused)
    rc = _lib.lib().wkv7_forward(ctypes.byref(sh), *map(_ptr, (r, w, k, v, a, b, s0)),
                                 _ptr(y if want_y else None), _ptr(sT if want_sT else None),
                                 _ptr(ckpt if want_ckpt else None), _stream(stream))
    _lib.check("wkv7_forward", rc)
    return (y if want_y else None), (sT if want_sT else None), (ckpt if want_ckpt else None)


def wkv7_backward(r, w, k, v, a, b, dy, s0=None, dsT=None, ckpt=None, *, chunk=64,
                  want_ds0=True, workspace=None, stream=None, out=None, algo="auto",
                  fused=False):
    """Run the reverse scan.  Returns dict(dr, dw, dk, dv, da, db, ds0).

    algo: "auto", "scan" or "chunked" (wkv7_algo).  fused=True: the inputs
    as for wkv7_forward(fused=True), and dw, da, db hold d omega, d kk and
    d gate."""
    (B, T, H, N), dt = _check_vecs("rwkvab dy", (r, w, k, v, a, b, dy))
    _check_state("s0", s0, B, H, N)
    _check_state("dsT", dsT, B, H, N)
    dev = r.device
    names = ("dr", "dw", "dk", "dv", "da", "db")
    grads = dict(out) if out is not None else {}
    need = wkv7_backward_workspace_bytes(B, T, H, N, dt, chunk, ckpt is not None)
    with _on(stream):
        for n in names:
            if grads.get(n) is None:
                grads[n] = torch.empty((B, T, H, N), device=dev, dtype=torch.float32)
        if want_ds0 and grads.get("ds0") is None:
            grads["ds0"] = torch.empty((B, H, N, N), device=dev, dtype=torch.float32)
        if workspace is None and need > 0:
            workspace = torch.empty(need, device=dev, dtype=torch.uint8)
    if not want_ds0:
        grads["ds0"] = None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sh = make_shape(B, T, H, N, dt, chunk, algo, fused=fused)
    rc = _lib.lib().wkv7_backward(
        ctypes.byref(sh), *map(_ptr, (r, w, k, v, a, b, s0, dy, dsT, ckpt)),
        *map(_ptr, (grads[n] for n in names)), _ptr(grads["ds0"]),
        _ptr(workspace), ws_bytes, _stream(stream))
    _lib.check("wkv7_backward", rc)
    return grads


def wkv7_backward_noalloc(r, w, k, v, a, b, dy, s0=None, dsT=None, ckpt=None, *, out,
                          chunk=64, stream=None, algo="auto", fused=False):
    """wkv7_backward with the library's own fixed device workspace
    (WKV7_NOALLOC_SCRATCH_BYTES per GPU) instead of a caller workspace; the
    caller supplies every output in `out` (dict dr, dw, dk, dv, da, db and
    optionally ds0), so nothing is allocated.  Returns `out`."""
    (B, T, H, N), dt = _check_vecs("rwkvab dy", (r, w, k, v, a, b, dy))
    _check_state("s0", s0, B, H, N)
    _check_state("dsT", dsT, B, H, N)
    names = ("dr", "dw", "dk", "dv", "da", "db")
    for n in names:
        _check_f32(n, out[n], (B, T, H, N))
    if out.get("ds0") is not None:
        _check_f32("ds0", out["ds0"], (B, H, N, N))
    sh = make_shape(B, T, H, N, dt, chunk, algo, fused=fused)
    rc = _lib.lib().wkv7_backward_noalloc(
        ctypes.byref(sh), *map(_ptr, (r, w, k, v, a, b, s0, dy, dsT, ckpt)),
        *map(_ptr, (out[n] for n in names)), _ptr(out.get("ds0")), _stream(stream))
    _lib.check("wkv7_backward_noalloc", rc)
    return out


def _check_f32(name, t, shape):
    if t.shape != shape or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous fp32 device tensor {list(shape)}")


def wkv7_epilogue_forward(y, r, k, v, g, ln_w, ln_b, r_k, *, stream=None, out=None):
    """Group norm, bonus and gate after the scan (wkv7_epilogue_forward):
    z = ((y - mean) rstd ln_w + ln_b + (sum r k r_k) v) g per (b, t, h)."""
    (B, T, H, N), dt = _check_vecs("rkvg", (r, k, v, g))
    _check_f32("y", y, (B, T, H, N))
    for n, p in (("ln_w", ln_w), ("ln_b", ln_b), ("r_k", r_k)):
        _check_f32(n, p, (H, N))
    with _on(stream):
        z = out if out is not None else torch.empty((B, T, H, N), device=y.device,
                                                    dtype=torch.float32)
    sh = make_shape(B, T, H, N, dt)
    rc = _lib.lib().wkv7_epilogue_forward(ctypes.byref(sh), *map(_ptr, (y, r, k, v, g, ln_w, ln_b, r_k, z)),
                                          _stream(stream))
    _lib.check("wkv7_epilogue_forward", rc)
    return z


def wkv7_epilogue_backward(dz, y, r, k, v, g, ln_w, ln_b, r_k, *, workspace=None, stream=None):
    """The epilogue's backward: dict(dy, dg, dr, dk, dv, dln_w, dln_b, dr_k);
    dr, dk, dv are the bonus term's shares (added to the scan's by the caller)."""
    (B, T, H, N), dt = _check_vecs("rkvg", (r, k, v, g))
    _check_f32("y", y, (B, T, H, N))
    _check_f32("dz", dz, (B, T, H, N))
    for n, p in (("ln_w", ln_w), ("ln_b", ln_b), ("r_k", r_k)):
        _check_f32(n, p, (H, N))
    dev = y.device
    sh = make_shape(B, T, H, N, dt)
    need = _lib.lib().wkv7_epilogue_workspace_bytes(ctypes.byref(sh))
    with _on(stream):
        out = {n: torch.empty((B, T, H, N), device=dev, dtype=torch.float32)
               for n in ("dy", "dg", "dr", "dk", "dv")}
        for n in ("dln_w", "dln_b", "dr_k"):
            out[n] = torch.empty((H, N), device=dev, dtype=torch.float32)
        if workspace is None and need > 0:
            workspace = torch.empty(need, device=dev, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _lib.lib().wkv7_epilogue_backward(
        ctypes.byref(sh), *map(_ptr, (dz, y, r, k, v, g, ln_w, ln_b, r_k)),
        *map(_ptr, (out[n] for n in ("dy", "dg", "dr", "dk", "dv", "dln_w", "dln_b", "dr_k"))),
        _ptr(workspace), ws_bytes, _stream(stream))
    _lib.check("wkv7_epilogue_backward", rc)
    return out


# ---------------------------------------------------------------- RWKV-8 rho

def _rwkv8_dims(q, v, decay):
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [B, H, T, L] and v [B, Hv, T, E]")
    B, H, T, L = q.shape
    Bv, Hv, Tv, E = v.shape
    if Bv != B or Tv != T or Hv not in (1, H) or tuple(decay.shape) != (H, L):
        raise ValueError(f"shapes q {tuple(q.shape)} v {tuple(v.shape)} decay {tuple(decay.shape)}")
    for n, t in (("q", q), ("v", v), ("decay", decay)):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous fp32 device tensor")
    return B, H, T, L, Hv, E


def rwkv8_shape(B, T, H, Hv, L=64, E=64):
    return _lib.Rwkv8Shape(B, T, H, Hv, L, E)


def rwkv8_checkpoint_bytes(B, T, H, Hv, L=64, E=64):
    return _lib.lib().rwkv8_checkpoint_bytes(ctypes.byref(rwkv8_shape(B, T, H, Hv, L, E)))


def rwkv8_backward_workspace_bytes(B, T, H, Hv, L=64, E=64, ckpt_provided=True):
    return _lib.lib().rwkv8_backward_workspace_bytes(ctypes.byref(rwkv8_shape(B, T, H, Hv, L, E)),
                                                      int(bool(ckpt_provided)))


def rwkv8_forward(q, v, decay, rho0=None, norm0=None, *, want_y=True, want_state=True,
                  want_ckpt=False, stream=None, out=None):
    """The RWKV-8 rho / rho_norm forward (rwkv8_forward).  q [B, H, T, 64],
    v [B, Hv, T, 64], decay [H, 64], rho0 [B, H, 64, 64], norm0 [B, H, 64].
    Returns (y, rhoT, normT, ckpt); unwanted outputs are None."""
    B, H, T, L, Hv, E = _rwkv8_dims(q, v, decay)
    dev = q.device
    y, rT, nT, ck = out if out is not None else (None, None, None, None)
    with _on(stream):
        if want_y and y is None:
            y = torch.empty((B, H, T, E), device=dev, dtype=torch.float32)
        if want_state and rT is None:
            rT = torch.empty((B, H, L, E), device=dev, dtype=torch.float32)
            nT = torch.empty((B, H, L), device=dev, dtype=torch.float32)
        if want_ckpt and ck is None:
            ck = torch.empty(rwkv8_checkpoint_bytes(B, T, H, Hv, L, E) // 4, device=dev,
                             dtype=torch.float32)
    sh = rwkv8_shape(B, T, H, Hv, L, E)
    rc = _lib.lib().rwkv8_forward(ctypes.byref(sh), *map(_ptr, (q, v, decay, rho0, norm0)),
                                  _ptr(y if want_y else None), _ptr(rT if want_state else None),
                                  _ptr(nT if want_state else None), _ptr(ck if want_ckpt else None),
                                  _stream(stream))
    _lib.check("rwkv8_forward", rc)
    return ((y if want_y else None), (rT if want_state else None), (nT if want_state else None),
            (ck if want_ckpt else None))


def rwkv8_backward(q, v, decay, dy, rho0=None, norm0=None, drhoT=None, dnormT=None, ckpt=None, *,
                   want_state_grads=True, workspace=None, stream=None, out=None):
    """The RWKV-8 rho / rho_norm backward (rwkv8_backward).  Returns dict dq,
    dv, ddecay, drho0, dnorm0 (the last two None when not wanted)."""
    B, H, T, L, Hv, E = _rwkv8_dims(q, v, decay)
    dev = q.device
    g = dict(out) if out is not None else {}
    need = rwkv8_backward_workspace_bytes(B, T, H, Hv, L, E, ckpt is not None)
    with _on(stream):
        shapes = {"dq": (B, H, T, L), "dv": (B, Hv, T, E), "ddecay": (H, L)}
        if want_state_grads:
            shapes.update(drho0=(B, H, L, E), dnorm0=(B, H, L))
        for n, shp in shapes.items():
            if g.get(n) is None:
                g[n] = torch.empty(shp, device=dev, dtype=torch.float32)
        if workspace is None and need > 0:
            workspace = torch.empty(need, device=dev, dtype=torch.uint8)
    if not want_state_grads:
        g["drho0"] = g["dnorm0"] = None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sh = rwkv8_shape(B, T, H, Hv, L, E)
    rc = _lib.lib().rwkv8_backward(
        ctypes.byref(sh), *map(_ptr, (q, v, decay, rho0, norm0, dy, drhoT, dnormT, ckpt)),
        *map(_ptr, (g["dq"], g["dv"], g["ddecay"], g["drho0"], g["dnorm0"])),
        _ptr(workspace), ws_bytes, _stream(stream))
    _lib.check("rwkv8_backward", rc)
    return g
