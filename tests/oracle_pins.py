"""Checks that pin the fp64 oracle to facts other than itself.

Each function runs the oracle (optionally a given build of it, so that the
mutation test can point the same checks at deliberately broken copies) and
returns the worst relative error against an independent statement of the
result: a hand-worked fixture, a closed form, exact rational arithmetic,
central finite differences, torch autograd, or an exact identity.
"""
import os
from fractions import Fraction

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NAMES_IN = ("r", "w", "k", "v", "a", "b")
NAMES_GRAD = ("dr", "dw", "dk", "dv", "da", "db")


def rel(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = max(1e-300, float(np.sqrt(np.mean(ref * ref))) if ref.size else 1.0)
    return float(np.max(np.abs(x - ref))) / scale if ref.size else 0.0


def rand_inputs(rng, B, T, H, N, s0=True, dsT=True, decay=True, incontext=True):
    """Recurrence-shaped random inputs (|a| = 1, |b| <= 1, w in (0.5, 1))."""
    shp = (B, T, H, N)
    d = {n: rng.standard_normal(shp) for n in ("r", "k", "v", "dy")}
    d["w"] = np.exp(-np.exp(-0.5) / (1 + np.exp(-rng.standard_normal(shp)))) if decay \
        else np.ones(shp)
    kk = rng.standard_normal(shp)
    kk /= np.linalg.norm(kk, axis=-1, keepdims=True)
    if incontext:
        d["a"] = -kk
        d["b"] = kk / (1 + np.exp(-rng.standard_normal(shp)))
    else:
        d["a"] = np.zeros(shp)
        d["b"] = np.zeros(shp)
    d["s0"] = 0.3 * rng.standard_normal((B, H, N, N)) if s0 else None
    d["dsT"] = rng.standard_normal((B, H, N, N)) if dsT else None
    return d


def run_fwd(d, lib=None):
    return oracle.forward(*(d[n] for n in NAMES_IN), s0=d["s0"], lib=lib)


def run_bwd(d, lib=None):
    return oracle.backward(*(d[n] for n in NAMES_IN), d["dy"], s0=d["s0"], dsT=d["dsT"],
                           lib=lib)


def loss(d, lib=None):
    y, sT = run_fwd(d, lib)
    L = float(np.sum(d["dy"] * y))
    if d["dsT"] is not None:
        L += float(np.sum(d["dsT"] * sT))
    return L


# ---------------------------------------------------------------- fixtures
def load_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rhs = (s.strip() for s in line.split("=", 1))
            vals[key] = [float(t) for t in rhs.split()]
    B, T, H, N = (int(x) for x in vals.pop("B T H N"))
    out = {}
    for key, xs in vals.items():
        if key in ("s0", "dsT", "sT", "ds0"):
            out[key] = np.array(xs).reshape(B, H, N, N)
        else:
            out[key] = np.array(xs).reshape(B, T, H, N)
    return out


def pin_golden(name, lib=None):
    g = load_golden(name)
    d = {n: g[n] for n in NAMES_IN + ("dy", "s0", "dsT")}
    y, sT = run_fwd(d, lib)
    grads = run_bwd(d, lib)
    errs = [rel(y, g["y"]), rel(sT, g["sT"])]
    errs += [rel(grads[n], g[n]) for n in NAMES_GRAD + ("ds0",)]
    return max(errs)


# ----------------------------------------------------------- closed forms
def pin_no_decay_closed_form(rng, lib=None, B=2, T=9, H=2, N=5):
    """w = 1, a = b = 0:  S_t = s0 + sum_{tau<=t} v_tau k_tau^T,  y_t = S_t r_t."""
    d = rand_inputs(rng, B, T, H, N, decay=False, incontext=False)
    y, sT = run_fwd(d, lib)
    outer = np.einsum("bthi,bthj->bthij", d["v"], d["k"])
    S = d["s0"][:, None] + np.cumsum(outer, axis=1)             # [B,T,H,N,N]
    y_ref = np.einsum("bthij,bthj->bthi", S, d["r"])
    return max(rel(y, y_ref), rel(sT, S[:, -1]))


def pin_diagonal_closed_form(rng, lib=None, B=1, T=7, H=2, N=4):
    """a = b = 0: each entry is a decayed sum, evaluated by brute force."""
    d = rand_inputs(rng, B, T, H, N, incontext=False)
    y, sT = run_fwd(d, lib)
    y_ref = np.zeros_like(y)
    S_last = np.zeros_like(sT)
    for bb in range(B):
        for h in range(H):
            w, k, v, r = (d[n][bb, :, h] for n in ("w", "k", "v", "r"))
            for t in range(T):
                S = d["s0"][bb, h] * np.prod(w[: t + 1], axis=0)[None, :]
                for tau in range(t + 1):
                    S = S + np.outer(v[tau], k[tau] * np.prod(w[tau + 1: t + 1], axis=0))
                y_ref[bb, t, h] = S @ r[t]
                if t == T - 1:
                    S_last[bb, h] = S
    return max(rel(y, y_ref), rel(sT, S_last))


def pin_scalar_n1(rng, lib=None, T=40):
    """N = 1: the scalar linear recurrence s_t = s_{t-1}(w_t + a_t b_t) + v_t k_t."""
    d = rand_inputs(rng, 1, T, 1, 1)
    y, sT = run_fwd(d, lib)
    s = d["s0"][0, 0, 0, 0]
    ys = []
    for t in range(T):
        w, k, v, a, b, r = (d[n][0, t, 0, 0] for n in ("w", "k", "v", "a", "b", "r"))
        s = s * (w + a * b) + v * k
        ys.append(s * r)
    return max(rel(y[0, :, 0, 0], ys), rel(sT[0, 0, 0, 0], s))


def pin_matrix_form(rng, lib=None, B=2, T=11, H=3, N=6):
    """S_t = S_{t-1} (diag(w_t) + a_t b_t^T) + v_t k_t^T, with dense products."""
    d = rand_inputs(rng, B, T, H, N)
    y, sT = run_fwd(d, lib)
    y_ref = np.zeros_like(y)
    S_ref = np.zeros_like(sT)
    for bb in range(B):
        for h in range(H):
            S = d["s0"][bb, h].copy()
            for t in range(T):
                w, k, v, a, b, r = (d[n][bb, t, h] for n in ("w", "k", "v", "a", "b", "r"))
                M = np.diag(w) + np.outer(a, b)
                S = S @ M + np.outer(v, k)
                y_ref[bb, t, h] = S @ r
            S_ref[bb, h] = S
    return max(rel(y, y_ref), rel(sT, S_ref))


# ------------------------------------------------------------ split sequence
def pin_split_sequence(rng, lib=None, B=2, T=13, H=2, N=5, T1=6):
    d = rand_inputs(rng, B, T, H, N)
    y, sT = run_fwd(d, lib)
    g = run_bwd(d, lib)
    first = {n: (d[n][:, :T1] if n in NAMES_IN + ("dy",) else d[n]) for n in d}
    second = {n: (d[n][:, T1:] if n in NAMES_IN + ("dy",) else d[n]) for n in d}
    y1, s_mid = run_fwd(first, lib)
    second["s0"] = s_mid
    y2, sT2 = run_fwd(second, lib)
    g2 = run_bwd(second, lib)
    first["dsT"] = g2["ds0"]
    g1 = run_bwd(first, lib)
    errs = [rel(np.concatenate([y1, y2], 1), y), rel(sT2, sT), rel(g1["ds0"], g["ds0"])]
    for n in NAMES_GRAD:
        errs.append(rel(np.concatenate([g1[n], g2[n]], 1), g[n]))
    return max(errs)


# ------------------------------------------------------ finite differences
def pin_finite_differences(rng, lib=None, B=1, T=5, H=2, N=3, h=1e-6):
    """Central differences of L = sum dy.y + <dsT, sT> for every input element."""
    d = rand_inputs(rng, B, T, H, N)
    g = run_bwd(d, lib)
    worst = 0.0
    for n, gn in list(zip(NAMES_IN, NAMES_GRAD)) + [("s0", "ds0")]:
        fd = np.zeros_like(d[n])
        for idx in np.ndindex(d[n].shape):
            keep = d[n][idx]
            d[n][idx] = keep + h
            lp = loss(d, lib)
            d[n][idx] = keep - h
            lm = loss(d, lib)
            d[n][idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        worst = max(worst, rel(g[gn], fd))
    return worst


# ------------------------------------------------------- exact identities
def pin_identities(rng, lib=None, B=2, T=17, H=2, N=8):
    d = rand_inputs(rng, B, T, H, N)
    y, sT = run_fwd(d, lib)
    g = run_bwd(d, lib)
    errs = []
    # y_t is linear in r_t:  <dr_t, r_t> = <dy_t, y_t>  per (b, t, h)
    errs.append(rel(np.sum(g["dr"] * d["r"], -1), np.sum(d["dy"] * y, -1)))
    # L depends on a_t, b_t only through a_t b_t^T:  <da_t, a_t> = <db_t, b_t>
    errs.append(rel(np.sum(g["da"] * d["a"], -1), np.sum(g["db"] * d["b"], -1)))
    # (y, sT) is linear in (v, s0) jointly and in (k, s0) jointly (per (b, h))
    L_bh = np.sum(d["dy"] * y, axis=(1, 3)) + np.sum(d["dsT"] * sT, axis=(2, 3))
    s0_term = np.sum(g["ds0"] * d["s0"], axis=(2, 3))
    errs.append(rel(np.sum(g["dv"] * d["v"], axis=(1, 3)) + s0_term, L_bh))
    errs.append(rel(np.sum(g["dk"] * d["k"], axis=(1, 3)) + s0_term, L_bh))
    # gradients are linear in (dy, dsT)
    d2 = dict(d)
    d2["dy"] = rng.standard_normal(d["dy"].shape)
    d2["dsT"] = rng.standard_normal(d["dsT"].shape)
    d3 = dict(d)
    d3["dy"] = 2.0 * d["dy"] - 3.0 * d2["dy"]
    d3["dsT"] = 2.0 * d["dsT"] - 3.0 * d2["dsT"]
    g2, g3 = run_bwd(d2, lib), run_bwd(d3, lib)
    for n in NAMES_GRAD + ("ds0",):
        errs.append(rel(g3[n], 2.0 * g[n] - 3.0 * g2[n]))
    return max(errs)


# ------------------------------------------------------ torch autograd
def pin_torch_autograd(rng, lib=None, B=1, T=6, H=2, N=4):
    import torch
    d = rand_inputs(rng, B, T, H, N)
    g = run_bwd(d, lib)
    y, sT = run_fwd(d, lib)
    tv = {n: torch.tensor(d[n], dtype=torch.float64, requires_grad=True)
          for n in NAMES_IN + ("s0",)}
    ys = []
    S_all = []
    for bb in range(B):
        for h in range(H):
            S = tv["s0"][bb, h]
            yt = []
            for t in range(T):
                w, k, v, a, b, r = (tv[n][bb, t, h] for n in NAMES_IN[1:2] + ("k", "v", "a", "b", "r"))
                S = S * w[None, :] + torch.outer(v, k) + torch.outer(S @ a, b)
                yt.append(S @ r)
            ys.append(torch.stack(yt))
            S_all.append(S)
    Y = torch.stack(ys).reshape(B, H, T, N).permute(0, 2, 1, 3)
    ST = torch.stack(S_all).reshape(B, H, N, N)
    L = (torch.tensor(d["dy"]) * Y).sum() + (torch.tensor(d["dsT"]) * ST).sum()
    L.backward()
    errs = [rel(y, Y.detach().numpy()), rel(sT, ST.detach().numpy())]
    for n, gn in list(zip(NAMES_IN, NAMES_GRAD)) + [("s0", "ds0")]:
        errs.append(rel(g[gn], tv[n].grad.numpy()))
    return max(errs)


def pin_torch_autograd_long(rng, lib=None):
    """The same check over 150 steps: the oracle's backward replays the
    forward in stretches of 64 steps from kept states, so a sequence of two
    whole stretches and a ragged third pins the replay bookkeeping."""
    return pin_torch_autograd(rng, lib, B=1, T=150, H=2, N=3)


# ------------------------------------------- exact rational forward mode
class Dual:
    """a + b*eps with eps^2 = 0, over exact rationals."""
    __slots__ = ("a", "b")

    def __init__(self, a, b=Fraction(0)):
        self.a, self.b = a, b

    def __add__(self, o):
        return Dual(self.a + o.a, self.b + o.b)

    def __mul__(self, o):
        return Dual(self.a * o.a, self.a * o.b + self.b * o.a)


def _exact_loss(d, seed_name, seed_idx, N, T):
    """Exact L and dL/d(seed) for a single (b, h) via dual rationals."""
    def val(n, idx):
        x = Fraction(float(d[n][idx]))
        return Dual(x, Fraction(1) if (n == seed_name and idx == seed_idx) else Fraction(0))
    S = [[val("s0", (0, 0, i, j)) for j in range(N)] for i in range(N)]
    L = Dual(Fraction(0))
    for t in range(T):
        g = {n: [val(n, (0, t, 0, j)) for j in range(N)] for n in NAMES_IN}
        sa = []
        for i in range(N):
            acc = Dual(Fraction(0))
            for j in range(N):
                acc = acc + S[i][j] * g["a"][j]
            sa.append(acc)
        for i in range(N):
            yi = Dual(Fraction(0))
            for j in range(N):
                S[i][j] = S[i][j] * g["w"][j] + g["v"][i] * g["k"][j] + sa[i] * g["b"][j]
                yi = yi + S[i][j] * g["r"][j]
            L = L + yi * Dual(Fraction(float(d["dy"][0, t, 0, i])))
    for i in range(N):
        for j in range(N):
            L = L + S[i][j] * Dual(Fraction(float(d["dsT"][0, 0, i, j])))
    return L


def pin_exact_rational(rng, lib=None, T=3, N=2):
    """Exact forward-mode derivatives (rational arithmetic) of every input."""
    d = rand_inputs(rng, 1, T, 1, N)
    g = run_bwd(d, lib)
    errs = []
    for n, gn in list(zip(NAMES_IN, NAMES_GRAD)) + [("s0", "ds0")]:
        exact = np.zeros_like(d[n])
        for idx in np.ndindex(d[n].shape):
            exact[idx] = float(_exact_loss(d, n, idx, N, T).b)
        errs.append(rel(g[gn], exact))
    L_exact = float(_exact_loss(d, None, None, N, T).a)
    errs.append(abs(loss(d, lib) - L_exact) / max(1.0, abs(L_exact)))
    return max(errs)


# --------------------------------------- fused time-mix inputs (oracle.fused)
def rand_fused(rng, B, T, H, N):
    """omega ~ N(0,1), kk unit per (b,t,h), ag = sigmoid(N(0,1)), in the
    recurrence's positional slots of w, a, b."""
    shp = (B, T, H, N)
    d = {n: rng.standard_normal(shp) for n in ("r", "k", "v", "dy")}
    d["w"] = rng.standard_normal(shp)
    kk = rng.standard_normal(shp)
    d["a"] = kk / np.linalg.norm(kk, axis=-1, keepdims=True)
    d["b"] = 1.0 / (1.0 + np.exp(-rng.standard_normal(shp)))
    d["s0"] = 0.3 * rng.standard_normal((B, H, N, N))
    d["dsT"] = rng.standard_normal((B, H, N, N))
    return d


def _fused_loss(d, lib=None):
    import oracle.fused as F
    y, sT = F.forward(*(d[n] for n in NAMES_IN), s0=d["s0"], lib=lib)
    return float(np.sum(d["dy"] * y)) + float(np.sum(d["dsT"] * sT))


def pin_fused_finite_differences(rng, lib=None, B=1, T=4, H=2, N=3, h=1e-6):
    """Central differences of the loss through the formed inputs, for every
    element of r, omega, k, v, kk, ag and s0."""
    import oracle.fused as F
    d = rand_fused(rng, B, T, H, N)
    g = F.backward(*(d[n] for n in NAMES_IN), d["dy"], s0=d["s0"], dsT=d["dsT"], lib=lib)
    worst = 0.0
    for n, gn in list(zip(NAMES_IN, NAMES_GRAD)) + [("s0", "ds0")]:
        fd = np.zeros_like(d[n])
        for idx in np.ndindex(d[n].shape):
            keep = d[n][idx]
            d[n][idx] = keep + h
            lp = _fused_loss(d, lib)
            d[n][idx] = keep - h
            lm = _fused_loss(d, lib)
            d[n][idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        worst = max(worst, rel(g[gn], fd))
    return worst


def pin_fused_torch_autograd(rng, lib=None, B=1, T=5, H=2, N=4):
    """torch autograd of a plain loop that forms w, a, b from omega, kk, ag."""
    import torch

    import oracle.fused as F
    d = rand_fused(rng, B, T, H, N)
    g = F.backward(*(d[n] for n in NAMES_IN), d["dy"], s0=d["s0"], dsT=d["dsT"], lib=lib)
    tv = {n: torch.tensor(d[n], dtype=torch.float64, requires_grad=True)
          for n in NAMES_IN + ("s0",)}
    c = float(np.exp(-0.5))
    L = torch.zeros((), dtype=torch.float64)
    for bb in range(B):
        for h in range(H):
            S = tv["s0"][bb, h]
            for t in range(T):
                om, kk, ag = tv["w"][bb, t, h], tv["a"][bb, t, h], tv["b"][bb, t, h]
                w = torch.exp(-c * torch.sigmoid(om))
                a, b = -kk, kk * ag
                k, v, r = tv["k"][bb, t, h], tv["v"][bb, t, h], tv["r"][bb, t, h]
                S = S * w[None, :] + torch.outer(v, k) + torch.outer(S @ a, b)
                L = L + torch.dot(torch.tensor(d["dy"][bb, t, h]), S @ r)
            L = L + (torch.tensor(d["dsT"][bb, h]) * S).sum()
    L.backward()
    return max(rel(g[gn], tv[n].grad.numpy())
               for n, gn in list(zip(NAMES_IN, NAMES_GRAD)) + [("s0", "ds0")])


# ------------------------------------------- epilogue (oracle.epilogue)
def rand_epilogue(rng, B, T, H, N):
    shp = (B, T, H, N)
    d = {n: rng.standard_normal(shp) for n in ("y", "r", "k", "v", "dz")}
    d["y"] = 3.0 * d["y"] + 0.5
    d["g"] = 1.0 / (1.0 + np.exp(-rng.standard_normal(shp)))
    for n in ("ln_w", "ln_b", "r_k"):
        d[n] = rng.standard_normal((H, N))
    return d


EPI_IN = ("y", "r", "k", "v", "g", "ln_w", "ln_b", "r_k")
EPI_GRAD = {"y": "dy", "r": "dr", "k": "dk", "v": "dv", "g": "dg", "ln_w": "dln_w",
            "ln_b": "dln_b", "r_k": "dr_k"}


def pin_epilogue_finite_differences(rng, lib=None, B=1, T=3, H=2, N=5, h=1e-6):
    """Central differences of L = sum dz . z for every input element and
    parameter of the group norm + bonus + gate epilogue."""
    import oracle.epilogue as E
    d = rand_epilogue(rng, B, T, H, N)
    g = E.backward(d["dz"], *(d[n] for n in EPI_IN))

    def L():
        return float(np.sum(d["dz"] * E.forward(*(d[n] for n in EPI_IN))))
    worst = 0.0
    for n in EPI_IN:
        fd = np.zeros_like(d[n])
        for idx in np.ndindex(d[n].shape):
            keep = d[n][idx]
            d[n][idx] = keep + h
            lp = L()
            d[n][idx] = keep - h
            lm = L()
            d[n][idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        worst = max(worst, rel(g[EPI_GRAD[n]], fd))
    return worst


def pin_epilogue_torch(rng, lib=None, B=2, T=3, H=2, N=8):
    """torch's own group norm (F.group_norm, one group per head) and autograd
    against the forward and every gradient."""
    import torch
    import torch.nn.functional as F

    import oracle.epilogue as E
    d = rand_epilogue(rng, B, T, H, N)
    z = E.forward(*(d[n] for n in EPI_IN))
    g = E.backward(d["dz"], *(d[n] for n in EPI_IN))
    tv = {n: torch.tensor(d[n], dtype=torch.float64, requires_grad=True) for n in EPI_IN}
    yy = tv["y"].reshape(B * T, H * N)
    yn = F.group_norm(yy, H, tv["ln_w"].reshape(-1), tv["ln_b"].reshape(-1), eps=E.EPS)
    yn = yn.reshape(B, T, H, N)
    s = (tv["r"] * tv["k"] * tv["r_k"]).sum(-1, keepdim=True)
    zt = (yn + s * tv["v"]) * tv["g"]
    (torch.tensor(d["dz"]) * zt).sum().backward()
    errs = [rel(z, zt.detach().numpy())]
    for n in EPI_IN:
        errs.append(rel(g[EPI_GRAD[n]], tv[n].grad.numpy()))
    return max(errs)


ALL_PINS = {
    "golden_n1": (lambda rng, lib: pin_golden("hand_n1_t2.txt", lib), 1e-15),
    "golden_n2": (lambda rng, lib: pin_golden("hand_n2_t1.txt", lib), 1e-15),
    "no_decay_closed_form": (pin_no_decay_closed_form, 1e-12),
    "diagonal_closed_form": (pin_diagonal_closed_form, 1e-12),
    "scalar_n1": (pin_scalar_n1, 1e-12),
    "matrix_form": (pin_matrix_form, 1e-12),
    "split_sequence": (pin_split_sequence, 1e-12),
    "finite_differences": (pin_finite_differences, 1e-7),
    "identities": (pin_identities, 1e-11),
    "torch_autograd": (pin_torch_autograd, 1e-12),
    "torch_autograd_long": (pin_torch_autograd_long, 1e-11),
    "exact_rational": (pin_exact_rational, 1e-13),
    "fused_finite_differences": (pin_fused_finite_differences, 1e-7),
    "fused_torch_autograd": (pin_fused_torch_autograd, 1e-12),
    "epilogue_finite_differences": (pin_epilogue_finite_differences, 1e-7),
    "epilogue_torch_group_norm": (pin_epilogue_torch, 1e-12),
}
