"""fp64 oracle of the time-mix epilogue that follows the WKV7 scan.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the test suite, the
smoke check and the benchmark's CPU-baseline leg may use it; the product
library never does.

On the Foundry "rwkvx/rx_pretrain.c" page the scan's output y goes, per
(b, t, h) over the N entries of the head, through gn_forward (group norm:
mean, variance, epsilon 64e-5, per-channel scale ln_x_w and shift ln_x_b),
plus the bonus term (s = sum_j r_j k_j r_k[j] per head, added as s v), and
then the gate g element-wise (tg = yb * g, before the output projection,
which stays outside):

  z = ((y - mean) * rstd * ln_w + ln_b + s v) * g.

``backward`` follows the page's "post-processing backward per token" block
in its order: the gate, the bonus, the group norm, returning dy (the scan's
output gradient), dg, the bonus terms of dr, dk, dv, and the per-channel
parameter gradients summed over (b, t).  Shapes: vectors [B, T, H, N];
parameters [H, N].
"""
import numpy as np

EPS = 64e-5


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _norm(y):
    mean = y.mean(-1, keepdims=True)
    var = ((y - mean) ** 2).mean(-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + EPS)
    return (y - mean) * rstd, rstd


def forward(y, r, k, v, g, ln_w, ln_b, r_k):
    y, r, k, v, g, ln_w, ln_b, r_k = map(_f64, (y, r, k, v, g, ln_w, ln_b, r_k))
    yn, _ = _norm(y)
    s = np.sum(r * k * r_k, -1, keepdims=True)        # bonus per (b, t, h)
    return (yn * ln_w + ln_b + s * v) * g


def backward(dz, y, r, k, v, g, ln_w, ln_b, r_k):
    dz, y, r, k, v, g, ln_w, ln_b, r_k = map(_f64, (dz, y, r, k, v, g, ln_w, ln_b, r_k))
    yn, rstd = _norm(y)
    s = np.sum(r * k * r_k, -1, keepdims=True)
    yb = yn * ln_w + ln_b + s * v
    # gate
    dyb = dz * g
    dg = dz * yb
    # bonus: yb += s v, s = sum_j r k r_k
    ds = np.sum(dyb * v, -1, keepdims=True)
    dv = dyb * s
    dr = ds * k * r_k
    dk = ds * r * r_k
    dr_k = np.sum(ds * r * k, axis=(0, 1))
    # group norm
    dln_w = np.sum(dyb * yn, axis=(0, 1))
    dln_b = np.sum(dyb, axis=(0, 1))
    dnorm = dyb * ln_w
    mdn = dnorm.mean(-1, keepdims=True)
    mdnn = (dnorm * yn).mean(-1, keepdims=True)
    dy = rstd * (dnorm - mdn - yn * mdnn)
    return {"dy": dy, "dg": dg, "dr": dr, "dk": dk, "dv": dv,
            "dln_w": dln_w, "dln_b": dln_b, "dr_k": dr_k}
