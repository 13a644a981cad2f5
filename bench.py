#!/usr/bin/env python3
"""WKV7 forward + backward throughput on one MI355X.

One step = the whole hot path over one batch of synthetic inputs already
resident in HBM: the forward scan (writing y, the final state and the
checkpoints every `chunk` steps) followed by the reverse scan that consumes
those checkpoints and writes dr, dw, dk, dv, da, db and ds0.

Prints ONE JSON line.  `value` is tokens (B*T) per second of fwd+bwd.
`roofline` is for the dominant kernel (the reverse scan; at N = 64 and
C = 64 its chunk form, whose contractions run on fp32 MFMA): its algorithmic
fp32 flops per launch (26*N^2 per token-head) over its mean launch time,
timed with HIP events on the stream it runs on, against the MI355X fp32
peak (157.3 TFLOP/s, the same for dense fp32 MFMA and packed fp32 VALU).
`fwd_only_tokens_per_s` times the forward alone without checkpoints
(inference).  `cpu_baseline` times the fp64 oracle on a bounded sample of
whole (b, h) recurrences of the same workload on the host's cores.

``--fused`` runs the same step on the fused time-mix inputs (omega, kk and
the gate in the places of w, a, b; the library forms w, a, b and returns
d omega, d kk, d gate) and adds ``unfused_pipeline_ms``: the same result
from the plain kernels with torch forming w, a, b before and chaining the
gradients after, the element-wise HBM passes the fused form saves.

``--epilogue`` times the time-mix epilogue after the scan (group norm,
bonus, gate; wkv7_epilogue_forward and _backward) on the workload's shape,
an HBM-bound pass each way, against the 8 TB/s roofline.

A workload with T = 1 (``--workload decode_b256_t1_h32_n64``) times the
decode step of batched inference instead: one forward step of every (b, h)
from its carry-in state, bound by HBM bandwidth (each (b, h) reads and
writes its N x N fp32 state).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "WKV7 fwd+bwd tokens/sec at 1 GPU; % of HBM/VALU roofline (rocprof)"
PEAK_FP32_VALU = 157.3e12   # MI355X published fp32 vector peak (FLOP/s)
PEAK_HBM = 8.0e12           # MI355X HBM3E (B/s)
DEFAULT_WORKLOAD = "b8_t4096_h32_n64"
PROFILES = os.path.join(ROOT, "profiles")


def algorithmic(wl):
    """Algorithmic work per launch (fp32 flops with FMA = 2, HBM bytes)."""
    th = wl.B * wl.T * wl.H
    N = wl.N
    eb = 4 if wl.dtype == "f32" else 2
    ck = 4 * N * N / wl.chunk                     # checkpoint bytes per token-head
    fwd_flops = 9 * N * N * th
    bwd_flops = 26 * N * N * th
    fwd_bytes = (6 * N * eb + 4 * N + ck) * th    # r,w,k,v,a,b in; y out; ckpt out
    bwd_bytes = (7 * N * eb + 6 * N * 4 + ck) * th  # 7 vectors in; 6 grads out; ckpt in
    # (the sa tape, 2*4*N more bytes per token-head, is this build's choice
    # and is not counted as algorithmic)
    return fwd_flops, bwd_flops, fwd_bytes, bwd_bytes


DECODE_METRIC = "WKV7 decode step tokens/sec at 1 GPU; % of HBM roofline (rocprof)"


def decode_bytes(wl):
    """Algorithmic HBM bytes of one decode step: the state in and out, six
    input vectors in, y out."""
    eb = 4 if wl.dtype == "f32" else 2
    N = wl.N
    return wl.B * wl.H * (2 * 4 * N * N + 6 * eb * N + 4 * N)


def decode_bench(args, wl):
    import torch

    import oracle
    from linear_attention_rnn_wkv7_amd import api
    from linear_attention_rnn_wkv7_amd.synthetic import make_inputs

    names = ("r", "w", "k", "v", "a", "b")
    inp = make_inputs(wl, device="cuda")
    B, H, N = wl.B, wl.H, wl.N
    y = torch.empty((B, 1, H, N), device="cuda", dtype=torch.float32)
    sT = torch.empty((B, H, N, N), device="cuda", dtype=torch.float32)
    stream = torch.cuda.current_stream()

    def step():
        api.wkv7_forward(*(inp[n] for n in names), inp["s0"], out=(y, sT, None), stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    for n, x in (("y", y), ("sT", sT)):
        if not torch.isfinite(x).all():
            raise RuntimeError(f"non-finite values in {n}")
    nbytes = decode_bytes(wl)
    achieved = nbytes / (ms * 1e-3)
    rec = {
        "metric": DECODE_METRIC,
        "value": B / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "T": 1, "H": H, "N": N,
                   "input_dtype": wl.dtype, "s0": wl.has_s0},
        "roofline": {
            "kernel": "wkv7_decode_kernel",
            "bound": "hbm",
            "achieved": achieved / 1e9,
            "peak": PEAK_HBM / 1e9,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM,
            "traffic": measured_traffic("wkv7_decode_kernel", wl.name),
            "achieved_gbps": counter_fields("wkv7_decode_kernel", wl.name, ms)["achieved_gbps"],
        },
    }
    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes, device="cuda", dtype=torch.uint8)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_bytes"] = args.copy_bytes
    if not args.no_cpu_baseline:
        host = {n: inp[n].cpu().double().numpy() for n in names}
        s0 = inp["s0"].cpu().double().numpy()
        cores = oracle.default_threads()
        reps, t0 = 0, time.perf_counter()
        while True:   # whole decode steps of every (b, h), up to the budget
            oracle.forward(*(host[n] for n in names), s0=s0, threads=cores)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_budget:
                break
        rec["cpu_baseline"] = {"value": reps * B / el, "unit": "tokens/s", "cores": cores,
                               "kind": "oracle",
                               "sample": f"{reps} whole decode steps of all {B * H} (b,h), fp64, "
                                         f"in {el:.2f} s"}
    print(json.dumps(rec), flush=True)


def unfused_pipeline_ms(api, inp, names, C, ck, ws, y, sT, grads, stream, args):
    """The fused step's result without fusion: torch forms w, a, b from
    omega, kk and the gate, the plain kernels run, torch chains dw, da, db
    into d omega, d kk, d gate.  Mean ms per step over the same step count."""
    import math

    import torch

    c = math.exp(-0.5)
    om, kk, ag = inp["w"], inp["a"], inp["b"]

    def step():
        sg = torch.sigmoid(om)
        w = torch.exp(-c * sg)
        a = -kk
        b = kk * ag
        plain = (inp["r"], w, inp["k"], inp["v"], a, b)
        api.wkv7_forward(*plain, inp["s0"], chunk=C, want_ckpt=True, out=(y, sT, ck),
                         stream=stream)
        g = api.wkv7_backward(*plain, inp["dy"], inp["s0"], inp["dsT"], ck, chunk=C, workspace=ws,
                              out=grads, stream=stream)
        return (g["dw"] * w * (-c) * sg * (1 - sg), -g["da"] + ag * g["db"], kk * g["db"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / args.steps


EPILOGUE_METRIC = "WKV7 epilogue (group norm, bonus, gate) fwd+bwd tokens/sec at 1 GPU; % of HBM roofline"


def epilogue_bench(args, wl):
    import ctypes

    import torch

    import oracle.epilogue as OE
    from linear_attention_rnn_wkv7_amd import api
    from linear_attention_rnn_wkv7_amd.synthetic import make_inputs

    inp = make_inputs(wl, device="cuda")
    B, T, H, N = wl.B, wl.T, wl.H, wl.N
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed + 1)
    shp = (B, T, H, N)
    y = 4.0 * torch.randn(shp, generator=gen, device="cuda")
    g = torch.sigmoid(torch.randn(shp, generator=gen, device="cuda")).to(inp["r"].dtype)
    dz = torch.randn(shp, generator=gen, device="cuda")
    par = [1.0 + 0.1 * torch.randn((H, N), generator=gen, device="cuda"),
           0.1 * torch.randn((H, N), generator=gen, device="cuda"),
           0.5 * torch.randn((H, N), generator=gen, device="cuda")]
    args_ = (y, inp["r"], inp["k"], inp["v"], g, *par)
    z = torch.empty(shp, device="cuda", dtype=torch.float32)
    stream = torch.cuda.current_stream()
    sh = api.make_shape(B, T, H, N, inp["r"].dtype)
    ws = torch.empty(max(1, api._lib.lib().wkv7_epilogue_workspace_bytes(ctypes.byref(sh))),
                     device="cuda", dtype=torch.uint8)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    f_ms = timed(lambda: api.wkv7_epilogue_forward(*args_, out=z, stream=stream))
    b_ms = timed(lambda: api.wkv7_epilogue_backward(dz, *args_, workspace=ws, stream=stream))
    eb = 4 if wl.dtype == "f32" else 2
    rows_el = B * T * H * N
    f_bytes = rows_el * (4 + 4 * eb + 4)          # y, r, k, v, g in; z out
    b_bytes = rows_el * (8 + 4 * eb + 20)         # dz, y, r, k, v, g in; dy, dg, dr, dk, dv out
    ms = f_ms + b_ms
    achieved = (f_bytes + b_bytes) / (ms * 1e-3)
    rec = {
        "metric": EPILOGUE_METRIC, "value": B * T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "T": T, "H": H, "N": N, "input_dtype": wl.dtype,
                   "epilogue": True},
        "roofline": {"kernel": "epi_fwd_kernel + epi_bwd_kernel", "bound": "hbm",
                     "achieved": achieved / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM, "traffic": None},
        "fwd_ms": f_ms, "bwd_ms": b_ms,
        "fwd_gbps": f_bytes / (f_ms * 1e-3) / 1e9, "bwd_gbps": b_bytes / (b_ms * 1e-3) / 1e9,
    }
    if not args.no_cpu_baseline:
        # the oracle on a bounded sample of (b, t) rows (all heads)
        nb = max(1, min(B, 1))
        nt = min(T, 512)
        h = {n: x[:nb, :nt].detach().cpu().double().numpy() for n, x in
             (("y", y), ("r", inp["r"]), ("k", inp["k"]), ("v", inp["v"]), ("g", g), ("dz", dz))}
        hp = [p.cpu().double().numpy() for p in par]
        t0, reps = time.perf_counter(), 0
        while True:
            OE.forward(h["y"], h["r"], h["k"], h["v"], h["g"], *hp)
            OE.backward(h["dz"], h["y"], h["r"], h["k"], h["v"], h["g"], *hp)
            reps += 1
            el = time.perf_counter() - t0
            if el >= min(args.cpu_budget, 10.0):
                break
        rec["cpu_baseline"] = {"value": reps * nb * nt / el, "unit": "tokens/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{reps} x ({nb} x {nt} tokens, all {H} heads), fp64 numpy "
                                         f"fwd+bwd in {el:.1f} s"}
    print(json.dumps(rec), flush=True)


RWKV8_METRIC = "RWKV-8 rho fwd+bwd tokens/sec at 1 GPU; % of fp32 roofline (rocprof)"


def rwkv8_algorithmic(wl):
    """Algorithmic work per launch of the RWKV-8 rho recurrence (fp32 flops
    with FMA = 2, HBM bytes), L = E = 64, per token-head:
      forward : readout R^T c 2LE, state update diag(d) R + q v^T 3LE        = 5LE
      backward: dv, dq, the decay's row sums, the carry's decay 1LE, R dy,
                c dy^T (2LE each), the state replayed from a checkpoint 3LE  = 14LE
      bytes   : forward q, v in, y out, a checkpoint of R and n every 64
                steps out; backward q, v, dy and the checkpoint in, dq, dv out."""
    th = wl.B * wl.T * wl.H
    L, E = wl.L, wl.E
    ck = 4.0 * (L * E + L) / 64
    fwd_flops, bwd_flops = 5 * L * E * th, 14 * L * E * th
    vb = 4 * E * (wl.Hv / wl.H)
    fwd_bytes = (4 * L + vb + 4 * E + ck) * th
    bwd_bytes = (4 * L + vb + 4 * E + ck + 4 * L + vb) * th
    return fwd_flops, bwd_flops, fwd_bytes, bwd_bytes


def rwkv8_bench(args, wl):
    import numpy as np
    import torch

    import oracle.rwkv8 as R8
    from linear_attention_rnn_wkv7_amd import api
    from linear_attention_rnn_wkv7_amd.synthetic import make_rwkv8_inputs

    inp = make_rwkv8_inputs(wl, device="cuda")
    B, T, H, Hv, L, E = wl.B, wl.T, wl.H, wl.Hv, wl.L, wl.E
    f32 = torch.float32
    y = torch.empty((B, H, T, E), device="cuda", dtype=f32)
    rT = torch.empty((B, H, L, E), device="cuda", dtype=f32)
    nT = torch.empty((B, H, L), device="cuda", dtype=f32)
    ck = torch.empty(api.rwkv8_checkpoint_bytes(B, T, H, Hv, L, E) // 4, device="cuda", dtype=f32)
    grads = {"dq": torch.empty((B, H, T, L), device="cuda", dtype=f32),
             "dv": torch.empty((B, Hv, T, E), device="cuda", dtype=f32),
             "ddecay": torch.empty((H, L), device="cuda", dtype=f32),
             "drho0": torch.empty((B, H, L, E), device="cuda", dtype=f32),
             "dnorm0": torch.empty((B, H, L), device="cuda", dtype=f32)}
    ws = torch.empty(max(1, api.rwkv8_backward_workspace_bytes(B, T, H, Hv, L, E, True)),
                     device="cuda", dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    a = (inp["q"], inp["v"], inp["decay"])

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        api.rwkv8_forward(*a, inp["rho0"], inp["norm0"], want_ckpt=True, out=(y, rT, nT, ck),
                          stream=stream)
        if ev:
            ev[1].record(stream)
        api.rwkv8_backward(*a, inp["dy"], inp["rho0"], inp["norm0"], inp["drhoT"], inp["dnormT"],
                           ck, workspace=ws, out=grads, stream=stream)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(evs[i])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    for n, x in list(grads.items()) + [("y", y), ("rhoT", rT)]:
        if not torch.isfinite(x).all():
            raise RuntimeError(f"non-finite values in {n}")
    ff, bf, fb, bb = rwkv8_algorithmic(wl)
    t_roof = max((ff + bf) / PEAK_FP32_VALU, (fb + bb) / PEAK_HBM)
    achieved = bf / (bwd_ms * 1e-3)
    rec = {
        "metric": RWKV8_METRIC, "value": B * T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "T": T, "H": H, "Hv": Hv, "L": L, "E": E,
                   "carry_in_state": wl.has_state},
        "roofline": {"kernel": "rwkv8_bwd_kernel", "bound": "mfma", "achieved": achieved / 1e12,
                     "peak": PEAK_FP32_VALU / 1e12, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP32_VALU,
                     "traffic": measured_traffic("rwkv8_bwd_kernel", wl.name),
                     "mfma_type": "v_mfma_f32_16x16x4f32",
                     **counter_fields("rwkv8_bwd_kernel", wl.name, bwd_ms)},
        "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
        "fwd_bwd_roofline_frac": t_roof / (ms * 1e-3),
    }
    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes, device="cuda", dtype=torch.uint8)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_bytes"] = args.copy_bytes
    if not args.no_cpu_baseline:
        cores = oracle_threads()
        host = {n: (None if x is None else x.detach().cpu().double().numpy())
                for n, x in inp.items()}
        # whole (b, h) recurrences of the first batch rows, as many heads as
        # fit the budget (a probe of one head sets the count)
        def run(nb, nh):
            sl = {n: (None if x is None else x[:nb, :nh]) for n, x in host.items()
                  if n not in ("decay",)}
            t0 = time.perf_counter()
            R8.forward(sl["q"], sl["v"], host["decay"][:nh], sl["rho0"], sl["norm0"], threads=cores)
            R8.backward(sl["q"], sl["v"], host["decay"][:nh], sl["dy"], sl["rho0"], sl["norm0"],
                        sl["drhoT"], sl["dnormT"], threads=cores)
            return time.perf_counter() - t0
        probe = run(1, 1)
        nh = int(max(1, min(H, cores * max(1, int(args.cpu_budget / max(probe, 1e-3) / 2)))))
        el = run(1, nh)
        rec["cpu_baseline"] = {"value": nh * T / el / H, "unit": "tokens/s", "cores": min(cores, nh),
                               "kind": "oracle",
                               "sample": f"{nh} of {B * H} whole (b,h) recurrences (T={T}), fp64 "
                                         f"fwd+bwd in {el:.1f} s; tokens/s = token-heads/s / H"}
    print(json.dumps(rec), flush=True)


def oracle_threads():
    import oracle
    return oracle.default_threads()


def _profile_record(kernel, workload, kind):
    """A committed rocprofv3 counter record of `kernel` on `workload`, or None
    when absent or taken on a different kernel source."""
    path = os.path.join(PROFILES, f"{kernel.replace('_kernel', '')}_{workload}_{kind}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from linear_attention_rnn_wkv7_amd.profiling import kernel_sha

    if rec.get("kernel_sha") != kernel_sha(kernel):
        return None
    return rec


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from committed FETCH_SIZE / WRITE_SIZE
    counter runs, or None (absent, or taken on other sources)."""
    rec = _profile_record(kernel, workload, "traffic")
    return None if rec is None else rec.get("bytes_per_launch")


def counter_fields(kernel, workload, kernel_ms):
    """Counter-based figures for the roofline record: achieved HBM GB/s (the
    traffic counters' bytes per launch over the kernel's time in this run)
    and the matrix cores' busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over
    active cycles x SIMDs); None where no current record exists."""
    traffic = measured_traffic(kernel, workload)
    sq = _profile_record(kernel, workload, "sq")
    return {
        "achieved_gbps": None if traffic is None else traffic / (kernel_ms * 1e-3) / 1e9,
        "mfma_busy": None if sq is None else sq.get("mfma_busy"),
    }


def cpu_baseline(inp, wl, budget_s, fused=False):
    """Time the fp64 oracle (fwd + bwd) on whole (b, h) recurrences (its
    fused-input form with fused=True)."""
    import numpy as np

    import oracle
    import oracle.fused
    from linear_attention_rnn_wkv7_amd.synthetic import state_slice, vec_slice

    cores = oracle.default_threads()
    names = ("r", "w", "k", "v", "a", "b", "dy")

    def sample(pairs):
        def c64(x):
            return x.detach().to("cpu").double().numpy()
        sl = {n: np.concatenate([c64(vec_slice(inp[n], b, h)) for b, h in pairs], 2)
              for n in names}
        s0 = None if inp["s0"] is None else np.concatenate(
            [c64(state_slice(inp["s0"], b, h)) for b, h in pairs], 1)
        dsT = None if inp["dsT"] is None else np.concatenate(
            [c64(state_slice(inp["dsT"], b, h)) for b, h in pairs], 1)
        return sl, s0, dsT

    def run(pairs, data=None):
        sl, s0, dsT = data if data is not None else sample(pairs)
        threads = min(cores, len(pairs))
        t = time.perf_counter()
        orc = oracle.fused if fused else oracle
        orc.forward(*(sl[n] for n in names[:6]), s0=s0, want_sT=True, threads=threads)
        orc.backward(*(sl[n] for n in names[:6]), sl["dy"], s0=s0, dsT=dsT, threads=threads)
        return time.perf_counter() - t, threads

    all_pairs = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    probe_t, _ = run(all_pairs[:1])
    # one pair per core per round; as many pairs as fit the time budget
    n = int(max(1, min(len(all_pairs), cores * max(1, int(budget_s / max(probe_t, 1e-3))))))
    pairs = all_pairs[:n]
    # whole passes over the sample until the budget is spent (at least one)
    data = sample(pairs)
    dt, passes = 0.0, 0
    while passes == 0 or dt < 0.6 * budget_s:
        t, threads = run(pairs, data)
        dt += t
        passes += 1
    token_heads = passes * len(pairs) * wl.T
    return {
        "value": token_heads / dt / wl.H,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(pairs)} of {wl.B * wl.H} whole (b,h) recurrences (T={wl.T}) x {passes} "
                  f"passes, fp64 fwd+bwd in {dt:.1f} s; tokens/s = token-heads/s / H",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fused", action="store_true",
                    help="fused time-mix inputs (WKV7_FUSED_INPUTS)")
    ap.add_argument("--epilogue", action="store_true",
                    help="time the epilogue (group norm, bonus, gate) instead of the scan")
    ap.add_argument("--algo", default="auto", choices=("auto", "scan", "chunked"),
                    help="backward form (wkv7_algo): scan times the step-by-step reverse scan")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, run a plain device copy of this many bytes (the "
                         "reference point for the HBM traffic counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} (world {world}) is not "
              "supported; each (b, h) recurrence is independent, so N GPUs would each run "
              "1/N of the heads with no communication.", file=sys.stderr)
        sys.exit(2)

    import torch

    from linear_attention_rnn_wkv7_amd import api
    from linear_attention_rnn_wkv7_amd.synthetic import WORKLOADS, make_inputs

    from linear_attention_rnn_wkv7_amd.synthetic import RWKV8_WORKLOADS
    if args.workload in RWKV8_WORKLOADS:
        return rwkv8_bench(args, RWKV8_WORKLOADS[args.workload])
    wl = WORKLOADS[args.workload]
    if args.epilogue:
        return epilogue_bench(args, wl)
    if wl.T == 1:
        return decode_bench(args, wl)
    names = ("r", "w", "k", "v", "a", "b")
    fused = args.fused
    inp = make_inputs(wl, device="cuda", fused=fused)
    B, T, H, N, C = wl.B, wl.T, wl.H, wl.N, wl.chunk
    dev = inp["r"].device
    f32 = torch.float32
    y = torch.empty((B, T, H, N), device=dev, dtype=f32)
    sT = torch.empty((B, H, N, N), device=dev, dtype=f32)
    ck = torch.empty(api.wkv7_checkpoint_bytes(B, T, H, N, inp["r"].dtype, C) // 4, device=dev,
                     dtype=f32)
    grads = {n: torch.empty((B, T, H, N), device=dev, dtype=f32)
             for n in ("dr", "dw", "dk", "dv", "da", "db")}
    grads["ds0"] = torch.empty((B, H, N, N), device=dev, dtype=f32)
    need = api.wkv7_backward_workspace_bytes(B, T, H, N, inp["r"].dtype, C, True)
    ws = torch.empty(max(need, 1), device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        api.wkv7_forward(*(inp[n] for n in names), inp["s0"], chunk=C, want_ckpt=True,
                         out=(y, sT, ck), stream=stream, fused=fused)
        if ev:
            ev[1].record(stream)
        api.wkv7_backward(*(inp[n] for n in names), inp["dy"], inp["s0"], inp["dsT"], ck,
                          chunk=C, workspace=ws, out=grads, stream=stream, fused=fused,
                          algo=args.algo)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    # forward alone, no checkpoints (inference), after the timed region
    f0 = torch.cuda.Event(enable_timing=True)
    f1 = torch.cuda.Event(enable_timing=True)
    f0.record(stream)
    for _ in range(args.steps):
        api.wkv7_forward(*(inp[n] for n in names), inp["s0"], chunk=C, want_ckpt=False,
                         out=(y, sT, None), stream=stream, fused=fused)
    f1.record(stream)
    torch.cuda.synchronize()
    fwd_only_ms = f0.elapsed_time(f1) / args.steps
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    for n, x in list(grads.items()) + [("y", y), ("sT", sT)]:
        if not torch.isfinite(x).all():
            raise RuntimeError(f"non-finite values in {n}")

    fwd_flops, bwd_flops, fwd_bytes, bwd_bytes = algorithmic(wl)
    chunked = N == 64 and C == 64 and args.algo != "scan"   # the chunk form runs
    achieved = bwd_flops / (bwd_ms * 1e-3)
    kernel = "wkv7_bwdc_kernel" if chunked else "wkv7_bwd_kernel"
    traffic = measured_traffic(kernel, wl.name)
    t_roof = max((fwd_flops + bwd_flops) / PEAK_FP32_VALU, (fwd_bytes + bwd_bytes) / PEAK_HBM)
    tokens = B * T
    rec = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "T": T, "H": H, "N": N, "chunk": C,
                   "input_dtype": wl.dtype, "s0": wl.has_s0, "dsT": wl.has_dsT,
                   **({"fused_inputs": True} if fused else {}),
                   **({"backward": args.algo} if args.algo != "auto" else {})},
        "roofline": {
            "kernel": kernel,
            "bound": "mfma" if chunked else "alu",
            "achieved": achieved / 1e12,
            "peak": PEAK_FP32_VALU / 1e12,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP32_VALU,
            "traffic": traffic,
            "mfma_type": "v_mfma_f32_16x16x4f32" if chunked else None,
            **counter_fields(kernel, wl.name, bwd_ms),
        },
        "fwd_ms": fwd_ms,
        "bwd_ms": bwd_ms,
        "fwd_only_tokens_per_s": tokens / (fwd_only_ms * 1e-3),
        "fwd_bwd_roofline_frac": t_roof / (ms * 1e-3),
    }
    if fused:
        rec["unfused_pipeline_ms"] = unfused_pipeline_ms(api, inp, names, C, ck, ws, y, sT,
                                                         grads, stream, args)
    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes, device=dev, dtype=torch.uint8)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_bytes"] = args.copy_bytes
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(inp, wl, args.cpu_budget, fused=fused)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
