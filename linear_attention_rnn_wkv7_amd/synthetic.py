"""Seeded synthetic inputs for the WKV7 recurrence (shared by tests, bench
and the oracle checks; holds none of the recurrence's arithmetic).

Distributions follow how the Foundry "rwkvx/rx_pretrain.c" page forms the
recurrence inputs in its time-mix pre-forward (tm_pre_forward):
  * r, k, v, dy ~ N(0, 1)
  * w = exp(-c * sigmoid(x)), x ~ N(0, 1), c = exp(-0.5)   (RX_WDECAY_COEFF)
  * kk = L2-normalised N(0, 1) over the N entries of each (b, t, h) with the
    page's 1e-12 guard (l2norm_head); a = -kk; b = kk * sigmoid(z), z ~ N(0, 1)
  * s0 ~ N(0, 0.1^2) per element where the workload has a carry-in state
  * dsT ~ N(0, 1) where the workload has a final-state gradient
Draw order from one generator: r, k, v, x, kk_raw, z, dy, s0, dsT.  For the
bf16 workload r, w, k, v, a, b, dy are rounded to bf16 (round to nearest
even) once, after w, a and b are formed; s0, dsT stay fp32.
"""
import math
from dataclasses import dataclass
from typing import Optional

import torch

DECAY_COEFF = math.exp(-0.5)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    N: int
    dtype: str           # "f32" or "bf16": dtype of r, w, k, v, a, b, dy
    has_s0: bool
    has_dsT: bool
    seed: int
    chunk: int = 64      # checkpoint interval of the forward

    @property
    def tokens(self):
        return self.B * self.T

    @property
    def token_heads(self):
        return self.B * self.T * self.H


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_b1_t32_h2_n16", 1, 32, 2, 16, "f32", False, False, 1001),
        Workload("b4_t512_h8_n64", 4, 512, 8, 64, "f32", True, False, 1002),
        Workload("b8_t4096_h32_n64", 8, 4096, 32, 64, "f32", False, False, 1003),
        Workload("b16_t4096_h64_n64_bf16", 16, 4096, 64, 64, "bf16", True, False, 1004),
        Workload("long_b1_t65536_h32_n64", 1, 65536, 32, 64, "f32", True, True, 1005),
        # one decode step of batched inference: 256 sequences of a width-2048
        # model (32 heads of 64), each with its carry-in state
        Workload("decode_b256_t1_h32_n64", 256, 1, 32, 64, "f32", True, False, 1006),
    )
}
WORKLOAD_ORDER = list(WORKLOADS)


def custom(B, T, H, N, dtype="f32", has_s0=True, has_dsT=True, seed=7, chunk=64):
    return Workload(f"custom_b{B}_t{T}_h{H}_n{N}_{dtype}", B, T, H, N, dtype,
                    has_s0, has_dsT, seed, chunk)


def make_inputs(wl: Workload, device="cpu", seed: Optional[int] = None, fused=False):
    """Return a dict of tensors r, w, k, v, a, b, dy, s0 (or None), dsT (or None).

    fused=True returns the same draws before w, a and b are formed, in their
    places: w holds the decay pre-activation x, a the normalised key kk and
    b the gate sigmoid(z) (the inputs of the fused form of the library)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed if seed is None else seed)
    shp = (wl.B, wl.T, wl.H, wl.N)
    f32 = torch.float32

    def randn(shape):
        return torch.randn(shape, generator=g, device=dev, dtype=f32)

    r = randn(shp)
    k = randn(shp)
    v = randn(shp)
    x = randn(shp)
    kk = randn(shp)
    kk = kk / (torch.linalg.vector_norm(kk, dim=-1, keepdim=True) + 1e-12)
    gate = torch.sigmoid(randn(shp))
    if fused:
        w, a, b = x, kk, gate
    else:
        w = torch.exp(-DECAY_COEFF * torch.sigmoid(x))
        a = -kk
        b = kk * gate
    del x, kk, gate
    dy = randn(shp)
    s0 = 0.1 * randn((wl.B, wl.H, wl.N, wl.N)) if wl.has_s0 else None
    dsT = randn((wl.B, wl.H, wl.N, wl.N)) if wl.has_dsT else None
    out = dict(r=r, w=w, k=k, v=v, a=a, b=b, dy=dy, s0=s0, dsT=dsT)
    if wl.dtype == "bf16":
        for n in ("r", "w", "k", "v", "a", "b", "dy"):
            out[n] = out[n].to(torch.bfloat16)
    elif wl.dtype != "f32":
        raise ValueError(wl.dtype)
    return out


def vec_slice(x, b, h):
    """The [1, T, 1, N] slice of (b, h) from a [B, T, H, N] vector tensor."""
    return None if x is None else x[b:b + 1, :, h:h + 1, :]


def state_slice(x, b, h):
    """The [1, 1, N, N] slice of (b, h) from a [B, H, N, N] state tensor."""
    return None if x is None else x[b:b + 1, h:h + 1]


# ------------------------------------------------ RWKV-8 rho / rho_norm inputs
#   q = relu(N(0, 1))         non-negative latent features, half of them zero
#   v, dy ~ N(0, 1)
#   decay = exp(-c sigmoid(x)), x ~ N(0, 1), per (head, latent)   (in (0.545, 1))
#   carry-in: norm0 ~ U(0.5, 2.5), rho0 = norm0 * N(0, 1) per element (a
#             state whose rows are norm-weighted averages of values)
#   final-state gradients (when the workload has them): N(0, 1)
# Draw order from one generator: q, v, x, dy, norm0, rho0, drhoT, dnormT.

@dataclass(frozen=True)
class Rwkv8Workload:
    name: str
    B: int
    T: int
    H: int
    Hv: int
    has_state: bool
    has_final_grads: bool
    seed: int
    L: int = 64
    E: int = 64

    @property
    def tokens(self):
        return self.B * self.T


RWKV8_WORKLOADS = {
    w.name: w
    for w in (
        Rwkv8Workload("rwkv8_b2_t300_h4", 2, 300, 4, 4, True, True, 2001),
        # the WKV7 benchmark's shape (width 2048 as 32 heads of 64) with a
        # carry-in state
        Rwkv8Workload("rwkv8_b8_t4096_h32", 8, 4096, 32, 32, True, False, 2002),
    )
}


def rwkv8_custom(B, T, H, Hv=None, has_state=True, has_final_grads=True, seed=7):
    Hv = H if Hv is None else Hv
    return Rwkv8Workload(f"rwkv8_custom_b{B}_t{T}_h{H}_hv{Hv}", B, T, H, Hv, has_state,
                         has_final_grads, seed)


def make_rwkv8_inputs(wl: Rwkv8Workload, device="cpu", seed: Optional[int] = None):
    """Dict of fp32 tensors q, v, decay, dy, rho0, norm0, drhoT, dnormT (the
    last four None when the workload has no carry-in state / final-state
    gradients)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed if seed is None else seed)
    f32 = torch.float32

    def randn(shape):
        return torch.randn(shape, generator=g, device=dev, dtype=f32)

    q = torch.relu(randn((wl.B, wl.H, wl.T, wl.L)))
    v = randn((wl.B, wl.Hv, wl.T, wl.E))
    decay = torch.exp(-DECAY_COEFF * torch.sigmoid(randn((wl.H, wl.L))))
    dy = randn((wl.B, wl.H, wl.T, wl.E))
    out = dict(q=q, v=v, decay=decay, dy=dy, rho0=None, norm0=None, drhoT=None, dnormT=None)
    if wl.has_state:
        norm0 = 0.5 + 2.0 * torch.rand((wl.B, wl.H, wl.L), generator=g, device=dev, dtype=f32)
        out["norm0"] = norm0
        out["rho0"] = norm0[..., None] * randn((wl.B, wl.H, wl.L, wl.E))
    if wl.has_final_grads:
        out["drhoT"] = randn((wl.B, wl.H, wl.L, wl.E))
        out["dnormT"] = randn((wl.B, wl.H, wl.L))
    return out
