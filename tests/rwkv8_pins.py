"""Checks that pin the RWKV-8 rho oracle (oracle.rwkv8) to facts other than
itself: closed forms, brute force, exact rational arithmetic, central finite
differences, torch autograd and exact identities.  Each returns the worst
relative error (max|err| / RMS of the independent reference), and takes an
optional library build so that planted mistakes can be pointed at them."""
from fractions import Fraction

import numpy as np

import oracle.rwkv8 as R8


def rel(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    scale = max(1e-300, float(np.sqrt(np.mean(ref * ref))))
    return float(np.max(np.abs(x - ref))) / scale


def rand_inputs(rng, B, H, T, L, E, Hv=None, states=True, final_grads=True, unit_decay=False):
    """Non-negative queries (half of them zero, like rectified features),
    decays in (0.5, 1), a positive carry-in norm and a state consistent with
    it, and final-state gradients."""
    Hv = H if Hv is None else Hv
    q = np.maximum(rng.standard_normal((B, H, T, L)), 0.0) + 0.05 * rng.random((B, H, T, L))
    d = {
        "q": q,
        "v": rng.standard_normal((B, Hv, T, E)),
        "decay": np.ones((H, L)) if unit_decay else 0.5 + 0.5 * rng.random((H, L)),
        "dy": rng.standard_normal((B, H, T, E)),
    }
    if states:
        d["n0"] = 0.2 + rng.random((B, H, L))
        d["R0"] = d["n0"][..., None] * rng.standard_normal((B, H, L, E))
    else:
        d["n0"] = d["R0"] = None
    if final_grads:
        d["dRT"] = rng.standard_normal((B, H, L, E))
        d["dnT"] = rng.standard_normal((B, H, L))
    else:
        d["dRT"] = d["dnT"] = None
    return d


def run_fwd(d, lib=None):
    return R8.forward(d["q"], d["v"], d["decay"], d["R0"], d["n0"], lib=lib)


def run_bwd(d, lib=None):
    return R8.backward(d["q"], d["v"], d["decay"], d["dy"], d["R0"], d["n0"], d["dRT"], d["dnT"],
                       lib=lib)


def loss(d, lib=None):
    y, RT, nT = run_fwd(d, lib)
    L = float(np.sum(d["dy"] * y))
    if d["dRT"] is not None:
        L += float(np.sum(d["dRT"] * RT)) + float(np.sum(d["dnT"] * nT))
    return L


# ----------------------------------------------------------- closed forms
def _expand_v(v, H):
    return np.broadcast_to(v, (v.shape[0], H) + v.shape[2:]) if v.shape[1] == 1 else v


def _readout_ref(q, n, R):
    """y = sum_l (q[l] / (sum q + EPS)) R[l, :] / (n[l] + EPS), vectorised."""
    w = q / (q.sum(-1, keepdims=True) + R8.EPS) / (n + R8.EPS)
    return np.einsum("...l,...le->...e", w, R)


def pin_unit_decay_closed_form(rng, lib=None, B=2, H=2, T=9, L=4, E=5):
    """decay = 1: R_t = R_0 + sum_{u<t} q_u v_u^T, n_t = n_0 + sum_{u<t} q_u."""
    d = rand_inputs(rng, B, H, T, L, E, unit_decay=True)
    y, RT, nT = run_fwd(d, lib)
    v = _expand_v(d["v"], H)
    outer = np.einsum("bhtl,bhte->bhtle", d["q"], v)
    incl = np.cumsum(outer, axis=2)
    R_before = d["R0"][:, :, None] + np.concatenate([np.zeros_like(incl[:, :, :1]), incl[:, :, :-1]], 2)
    n_incl = np.cumsum(d["q"], axis=2)
    n_before = d["n0"][:, :, None] + np.concatenate([np.zeros_like(n_incl[:, :, :1]), n_incl[:, :, :-1]], 2)
    y_ref = _readout_ref(d["q"], n_before, R_before)
    return max(rel(y, y_ref), rel(RT, d["R0"] + incl[:, :, -1]), rel(nT, d["n0"] + n_incl[:, :, -1]))


def pin_decay_brute_force(rng, lib=None, B=1, H=2, T=7, L=3, E=4, Hv=1):
    """General decay: R_t[l] = d^t R_0[l] + sum_{u<t} d^(t-1-u) q_u[l] v_u,
    summed term by term (shared value, Hv = 1)."""
    d = rand_inputs(rng, B, H, T, L, E, Hv=Hv)
    y, RT, nT = run_fwd(d, lib)
    v = _expand_v(d["v"], H)
    y_ref = np.zeros_like(y)
    errs = []
    for b in range(B):
        for h in range(H):
            dec = d["decay"][h]
            for t in range(T + 1):
                R = d["R0"][b, h] * (dec ** t)[:, None]
                n = d["n0"][b, h] * dec ** t
                for u in range(t):
                    R = R + np.outer(d["q"][b, h, u] * dec ** (t - 1 - u), v[b, h, u])
                    n = n + d["q"][b, h, u] * dec ** (t - 1 - u)
                if t < T:
                    y_ref[b, h, t] = _readout_ref(d["q"][b, h, t], n, R)
                else:
                    errs += [rel(RT[b, h], R), rel(nT[b, h], n)]
    return max([rel(y, y_ref)] + errs)


# ------------------------------------------------------------ split sequence
def pin_split_sequence(rng, lib=None, B=2, H=2, T=13, L=3, E=4, T1=5):
    d = rand_inputs(rng, B, H, T, L, E)
    y, RT, nT = run_fwd(d, lib)
    g = run_bwd(d, lib)
    first = dict(d, q=d["q"][:, :, :T1], v=d["v"][:, :, :T1], dy=d["dy"][:, :, :T1])
    second = dict(d, q=d["q"][:, :, T1:], v=d["v"][:, :, T1:], dy=d["dy"][:, :, T1:])
    y1, Rm, nm = run_fwd(first, lib)
    second["R0"], second["n0"] = Rm, nm
    y2, RT2, nT2 = run_fwd(second, lib)
    g2 = run_bwd(second, lib)
    first["dRT"], first["dnT"] = g2["dR0"], g2["dn0"]
    g1 = run_bwd(first, lib)
    return max(rel(np.concatenate([y1, y2], 2), y), rel(RT2, RT), rel(nT2, nT),
               rel(np.concatenate([g1["dq"], g2["dq"]], 2), g["dq"]),
               rel(np.concatenate([g1["dv"], g2["dv"]], 2), g["dv"]),
               rel(g1["ddecay"] + g2["ddecay"], g["ddecay"]),
               rel(g1["dR0"], g["dR0"]), rel(g1["dn0"], g["dn0"]))


# ------------------------------------------------------ finite differences
def _fd_pin(rng, lib, B, H, T, L, E, Hv, h=1e-6):
    d = rand_inputs(rng, B, H, T, L, E, Hv=Hv)
    g = run_bwd(d, lib)
    worst = 0.0
    for n, gn in (("q", "dq"), ("v", "dv"), ("decay", "ddecay"), ("R0", "dR0"), ("n0", "dn0")):
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


def pin_finite_differences(rng, lib=None):
    """Central differences of L = sum dy.y + <dR_T, R_T> + <dn_T, n_T> for
    every element of q, v, decay, R_0 and n_0 (value per head)."""
    return _fd_pin(rng, lib, 2, 2, 5, 3, 4, Hv=2)


def pin_finite_differences_shared_value(rng, lib=None):
    """The same with one value shared by the heads (Hv = 1)."""
    return _fd_pin(rng, lib, 1, 3, 4, 3, 2, Hv=1)


# ------------------------------------------------------- exact identities
def pin_identities(rng, lib=None, B=2, H=2, T=11, L=4, E=5):
    d = rand_inputs(rng, B, H, T, L, E)
    y, RT, nT = run_fwd(d, lib)
    g = run_bwd(d, lib)
    errs = []
    # (y, R_T) are linear in (v, R_0) jointly and n does not depend on them:
    # sum_t <dv_t, v_t> + <dR_0, R_0> = sum_t <dy_t, y_t> + <dR_T, R_T>  per (b, h)
    lhs = np.sum(g["dv"] * d["v"], axis=(2, 3)) + np.sum(g["dR0"] * d["R0"], axis=(2, 3))
    rhs = np.sum(d["dy"] * y, axis=(2, 3)) + np.sum(d["dRT"] * RT, axis=(2, 3))
    errs.append(rel(lhs, rhs))
    # gradients are linear in (dy, dR_T, dn_T)
    d2 = dict(d, dy=rng.standard_normal(d["dy"].shape), dRT=rng.standard_normal(d["dRT"].shape),
              dnT=rng.standard_normal(d["dnT"].shape))
    d3 = dict(d, dy=2 * d["dy"] - 3 * d2["dy"], dRT=2 * d["dRT"] - 3 * d2["dRT"],
              dnT=2 * d["dnT"] - 3 * d2["dnT"])
    g2, g3 = run_bwd(d2, lib), run_bwd(d3, lib)
    for n in g:
        errs.append(rel(g3[n], 2 * g[n] - 3 * g2[n]))
    return max(errs)


# ------------------------------------------------------ torch autograd
def _torch_pin(rng, lib, B, H, T, L, E, Hv):
    import torch
    d = rand_inputs(rng, B, H, T, L, E, Hv=Hv)
    y, RT, nT = run_fwd(d, lib)
    g = run_bwd(d, lib)
    tv = {n: torch.tensor(d[n], dtype=torch.float64, requires_grad=True)
          for n in ("q", "v", "decay", "R0", "n0")}
    ys, Rs, ns = [], [], []
    for b in range(B):
        for h in range(H):
            R, n, dec = tv["R0"][b, h], tv["n0"][b, h], tv["decay"][h]
            yt = []
            for t in range(T):
                q = tv["q"][b, h, t]
                v = tv["v"][b, 0 if Hv == 1 else h, t]
                w = q / (q.sum() + R8.EPS) / (n + R8.EPS)
                yt.append(R.T @ w)
                R = dec[:, None] * R + torch.outer(q, v)
                n = dec * n + q
            ys.append(torch.stack(yt))
            Rs.append(R)
            ns.append(n)
    Y = torch.stack(ys).reshape(B, H, T, E)
    RTt = torch.stack(Rs).reshape(B, H, L, E)
    nTt = torch.stack(ns).reshape(B, H, L)
    Lt = (torch.tensor(d["dy"]) * Y).sum() + (torch.tensor(d["dRT"]) * RTt).sum() + \
        (torch.tensor(d["dnT"]) * nTt).sum()
    Lt.backward()
    errs = [rel(y, Y.detach().numpy()), rel(RT, RTt.detach().numpy()), rel(nT, nTt.detach().numpy())]
    for n, gn in (("q", "dq"), ("v", "dv"), ("decay", "ddecay"), ("R0", "dR0"), ("n0", "dn0")):
        errs.append(rel(g[gn], tv[n].grad.numpy()))
    return max(errs)


def pin_torch_autograd(rng, lib=None):
    """fp64 torch autograd of a plain loop, value per head and shared."""
    return max(_torch_pin(rng, lib, 2, 2, 6, 3, 4, Hv=2), _torch_pin(rng, lib, 1, 2, 5, 4, 3, Hv=1))


def pin_torch_autograd_long(rng, lib=None):
    """150 steps: two whole replay stretches of the oracle's backward and a
    ragged third."""
    return _torch_pin(rng, lib, 1, 2, 150, 3, 2, Hv=2)


# ------------------------------------------- exact rational forward mode
class Dual:
    """a + b*eps with eps^2 = 0, over exact rationals."""
    __slots__ = ("a", "b")

    def __init__(self, a, b=Fraction(0)):
        self.a, self.b = a, b

    def __add__(self, o):
        return Dual(self.a + o.a, self.b + o.b)

    def __sub__(self, o):
        return Dual(self.a - o.a, self.b - o.b)

    def __mul__(self, o):
        return Dual(self.a * o.a, self.a * o.b + self.b * o.a)

    def __truediv__(self, o):
        return Dual(self.a / o.a, (self.b * o.a - self.a * o.b) / (o.a * o.a))


def _exact(d, seed, T, L, E):
    """Exact L and dL/d(seed) for one (b, h) (B = H = Hv = 1) with the
    readout's EPS = 1e-6 as an exact rational."""
    eps = Dual(Fraction(1, 10 ** 6))

    def val(n, idx):
        return Dual(Fraction(float(d[n][idx])), Fraction(1) if seed == (n, idx) else Fraction(0))
    R = [[val("R0", (0, 0, l, e)) for e in range(E)] for l in range(L)]
    n = [val("n0", (0, 0, l)) for l in range(L)]
    dec = [val("decay", (0, l)) for l in range(L)]
    loss_ = Dual(Fraction(0))
    for t in range(T):
        q = [val("q", (0, 0, t, l)) for l in range(L)]
        v = [val("v", (0, 0, t, e)) for e in range(E)]
        sigma = eps
        for x in q:
            sigma = sigma + x
        for e in range(E):
            ye = Dual(Fraction(0))
            for l in range(L):
                ye = ye + q[l] / sigma / (n[l] + eps) * R[l][e]
            loss_ = loss_ + ye * Dual(Fraction(float(d["dy"][0, 0, t, e])))
        R = [[dec[l] * R[l][e] + q[l] * v[e] for e in range(E)] for l in range(L)]
        n = [dec[l] * n[l] + q[l] for l in range(L)]
    for l in range(L):
        loss_ = loss_ + n[l] * Dual(Fraction(float(d["dnT"][0, 0, l])))
        for e in range(E):
            loss_ = loss_ + R[l][e] * Dual(Fraction(float(d["dRT"][0, 0, l, e])))
    return loss_


def pin_exact_rational(rng, lib=None, T=3, L=2, E=2):
    """Exact forward-mode derivatives (rational arithmetic) for every input
    element, and the exact loss."""
    d = rand_inputs(rng, 1, 1, T, L, E)
    g = run_bwd(d, lib)
    errs = []
    for n, gn in (("q", "dq"), ("v", "dv"), ("decay", "ddecay"), ("R0", "dR0"), ("n0", "dn0")):
        exact = np.zeros_like(d[n])
        for idx in np.ndindex(d[n].shape):
            exact[idx] = float(_exact(d, (n, idx), T, L, E).b)
        errs.append(rel(g[gn], exact))
    L_exact = float(_exact(d, None, T, L, E).a)
    errs.append(abs(loss(d, lib) - L_exact) / max(1.0, abs(L_exact)))
    return max(errs)


ALL_PINS = {
    "unit_decay_closed_form": (pin_unit_decay_closed_form, 1e-12),
    "decay_brute_force": (pin_decay_brute_force, 1e-12),
    "split_sequence": (pin_split_sequence, 1e-11),
    "finite_differences": (pin_finite_differences, 1e-6),
    "finite_differences_shared_value": (pin_finite_differences_shared_value, 1e-6),
    "identities": (pin_identities, 1e-11),
    "torch_autograd": (pin_torch_autograd, 1e-12),
    "torch_autograd_long": (pin_torch_autograd_long, 1e-11),
    "exact_rational": (pin_exact_rational, 1e-13),
}
