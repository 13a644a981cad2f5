"""fp64 oracle of the WKV7 scan with its time-mix inputs formed in place.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the test suite, the
smoke check and the benchmark's CPU-baseline leg may use it; the product
library never does.

The Foundry "rwkvx/rx_pretrain.c" page forms three of the recurrence's
inputs element-wise just before the scan (tm_pre_forward) and takes their
gradients apart just after the reverse scan (the time-mix backward):

  * the decay:    w = exp(-c * sigmoid(omega)),  c = RX_WDECAY_COEFF = exp(-0.5),
                  with omega the decay pre-activation (w0 plus its LoRA);
  * the in-context pair:  a = -kk,  b = kk * ag,
                  with kk the L2-normalised key and ag the sigmoid gate.

Here ``forward`` forms w, a, b that way and runs the fp64 recurrence of
``oracle.forward``; ``backward`` runs ``oracle.backward`` and applies the
chain rule of those three formulas:

  d omega = dw * w * (-c) * sigmoid(omega) * (1 - sigmoid(omega))
  d kk    = -da + ag * db
  d ag    = kk * db

(the page's "w_vec" and "recombine nkk/kka" steps of the time-mix backward).
Arguments keep the recurrence's positional order with omega, kk, ag in the
places of w, a, b; results keep the keys dw, da, db for d omega, d kk, d ag.
"""
import math

import numpy as np

from . import backward as _backward
from . import forward as _forward

DECAY_COEFF = math.exp(-0.5)


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def unfuse(omega, kk, ag):
    """(w, a, b) from the decay pre-activation, the normalised key and the gate."""
    omega, kk, ag = map(_f64, (omega, kk, ag))
    return np.exp(-DECAY_COEFF * sigmoid(omega)), -kk, kk * ag


def forward(r, omega, k, v, kk, ag, s0=None, **kw):
    w, a, b = unfuse(omega, kk, ag)
    return _forward(r, w, k, v, a, b, s0=s0, **kw)


def backward(r, omega, k, v, kk, ag, dy, s0=None, dsT=None, **kw):
    omega, kk, ag = map(_f64, (omega, kk, ag))
    w, a, b = unfuse(omega, kk, ag)
    g = _backward(r, w, k, v, a, b, dy, s0=s0, dsT=dsT, **kw)
    sg = sigmoid(omega)
    out = dict(g)
    out["dw"] = g["dw"] * w * (-DECAY_COEFF) * sg * (1.0 - sg)
    out["da"] = -g["da"] + ag * g["db"]
    out["db"] = kk * g["db"]
    return out
