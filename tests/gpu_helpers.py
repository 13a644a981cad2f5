"""Shared helpers for the GPU parity tests: run the HIP path through the C
ABI binding, run the oracle on the same inputs (copied back from the
device), compare per tensor against max|err| <= tau * RMS(reference)."""
import numpy as np
import torch

import oracle
from linear_attention_rnn_wkv7_amd import api
from linear_attention_rnn_wkv7_amd.synthetic import state_slice, vec_slice

IN = ("r", "w", "k", "v", "a", "b")
GRADS = ("dr", "dw", "dk", "dv", "da", "db")
# Parity bar: fp32 inputs 2e-4, bf16 inputs 2e-2 (relative to the RMS of the
# fp64 reference, per output tensor).
TAU = {torch.float32: 2e-4, torch.bfloat16: 2e-2}


def gpu_run(inp, chunk=64, ckpt_handoff=True, algo="auto"):
    """Forward (with checkpoints) + backward on the device.  Returns dict of
    fp32 device tensors y, sT, dr..db, ds0."""
    y, sT, ck = api.wkv7_forward(*(inp[n] for n in IN), inp["s0"], chunk=chunk,
                                 want_ckpt=ckpt_handoff)
    g = api.wkv7_backward(*(inp[n] for n in IN), inp["dy"], inp["s0"], inp["dsT"],
                          ck if ckpt_handoff else None, chunk=chunk, algo=algo)
    out = dict(g)
    out["y"], out["sT"] = y, sT
    return out


def to64(x):
    return None if x is None else x.detach().to("cpu").double().numpy()


def oracle_run(inp, pairs=None, threads=None):
    """fp64 oracle on all (b, h), or on the listed (b, h) pairs stacked along
    the head axis (the pairs are independent recurrences)."""
    if pairs is None:
        sl = {n: to64(inp[n]) for n in IN + ("dy",)}
        s0, dsT = to64(inp["s0"]), to64(inp["dsT"])
    else:
        sl = {n: np.concatenate([to64(vec_slice(inp[n], b, h)) for b, h in pairs], axis=2)
              for n in IN + ("dy",)}
        s0 = None if inp["s0"] is None else np.concatenate(
            [to64(state_slice(inp["s0"], b, h)) for b, h in pairs], axis=1)
        dsT = None if inp["dsT"] is None else np.concatenate(
            [to64(state_slice(inp["dsT"], b, h)) for b, h in pairs], axis=1)
    y, sT = oracle.forward(*(sl[n] for n in IN), s0=s0, threads=threads)
    g = oracle.backward(*(sl[n] for n in IN), sl["dy"], s0=s0, dsT=dsT, threads=threads)
    g["y"], g["sT"] = y, sT
    return g


def gpu_pairs(out, pairs):
    """Gather the listed (b, h) pairs from full device outputs, stacked like
    oracle_run(pairs=...)."""
    res = {}
    for n, x in out.items():
        if x is None:
            continue
        if n in ("sT", "ds0"):
            res[n] = np.concatenate([to64(state_slice(x, b, h)) for b, h in pairs], axis=1)
        else:
            res[n] = np.concatenate([to64(vec_slice(x, b, h)) for b, h in pairs], axis=2)
    return res


def full_compare(inp, out, tau, label, oracle_fn=None, elem_budget=64 << 20, say=print):
    """Every element of every output against the oracle, streamed over
    blocks of one batch row and a group of heads (each block's oracle inputs
    stay within ~elem_budget elements per tensor).  Returns {name: max|err| /
    RMS(ref)} with max and RMS taken over the whole tensor, and the names over
    tau.  oracle_fn(block_inputs) -> dict of fp64 outputs (oracle_run by
    default)."""
    oracle_fn = oracle_fn or oracle_run
    B, T, Hh, N = inp["r"].shape
    hg = max(1, min(Hh, elem_budget // max(1, T * N)))
    stats = {}
    for b in range(B):
        for h0 in range(0, Hh, hg):
            h1 = min(Hh, h0 + hg)
            blk = {n: (None if x is None else
                       (x[b:b + 1, :, h0:h1] if n in IN + ("dy",) else x[b:b + 1, h0:h1]))
                   for n, x in inp.items()}
            ref = oracle_fn(blk)
            for n, r in ref.items():
                if r is None or out.get(n) is None:
                    continue
                g = out[n][b:b + 1, h0:h1] if n in ("sT", "ds0") else out[n][b:b + 1, :, h0:h1]
                g = to64(g)
                st = stats.setdefault(n, [0.0, 0.0, 0])
                if r.size:
                    st[0] = max(st[0], float(np.max(np.abs(g - r))))
                    st[1] += float(np.sum(r * r))
                    st[2] += r.size
            del ref
    errs, bad = {}, []
    for n, (mx, ss, cnt) in stats.items():
        rms = float(np.sqrt(ss / cnt)) if cnt else 0.0
        e = mx / max(rms, 1e-30) if cnt else 0.0
        errs[n] = e
        if not np.isfinite(e) or e > tau:
            bad.append(n)
    say(f"{label} (all {B * Hh} (b,h), blocks of {hg} heads): "
        + " ".join(f"{n}={errs[n]:.2e}" for n in sorted(errs)))
    return errs, bad


def compare(got, ref, tau, names=("y", "sT") + GRADS + ("ds0",)):
    """Return {name: max|err| / RMS(ref)} and the list of names over tau."""
    errs, bad = {}, []
    for n in names:
        if ref.get(n) is None or got.get(n) is None:
            continue
        g = got[n] if isinstance(got[n], np.ndarray) else to64(got[n])
        r = ref[n]
        if r.size == 0:
            errs[n] = 0.0
            continue
        rms = float(np.sqrt(np.mean(r * r)))
        e = float(np.max(np.abs(g - r))) / max(rms, 1e-30)
        errs[n] = e
        if not np.isfinite(e) or e > tau:
            bad.append(n)
    return errs, bad
