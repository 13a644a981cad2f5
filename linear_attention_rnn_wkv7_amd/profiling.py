"""Summaries of rocprofv3 output for the profiles/ directory.

    python -m linear_attention_rnn_wkv7_amd.profiling stats  --csv K.csv --cmd "..." --out F.md
    python -m linear_attention_rnn_wkv7_amd.profiling traffic --fetch F.csv --write W.csv \
        --kernel wkv7_bwd_kernel --copy-bytes N --workload NAME --cmd "..." --out F.json

`stats` condenses a --kernel-trace --stats kernel_stats.csv.  `sq` sums SQ
and GRBM counters per dispatch of each wkv7 kernel (MFMA busy fraction, LDS
bank-conflict cycles per CU).  `traffic`
turns per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of a kernel into bytes per
launch, scaling each counter by what it reads for the plain device copy of
`copy-bytes` bytes that bench.py --copy-bytes runs in the same process.
"""
import argparse
import csv
import hashlib
import json
import os
import re
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_CSRC = "linear_attention_rnn_wkv7_amd/csrc/"
KERNEL_SOURCES = tuple(_CSRC + f for f in ("wkv7_bwd.hip", "wkv7_bwdc.hip", "wkv7_fwd.hip",
                                           "wkv7_fwdc.hip", "wkv7_decode.hip", "wkv7_split.hip",
                                           "wkv7_epilogue.hip", "wkv7_device.h", "rwkv8.hip"))
# the sources each kernel is built from (its traffic record is stale once
# one of them changes)
_KERNEL_FILES = {
    "wkv7_bwdc_kernel": ("wkv7_bwdc.hip", "wkv7_device.h"),
    "wkv7_fwdc_kernel": ("wkv7_fwdc.hip", "wkv7_device.h"),
    "wkv7_bwd_kernel": ("wkv7_bwd.hip", "wkv7_device.h"),
    "wkv7_fwd_kernel": ("wkv7_fwd.hip", "wkv7_device.h"),
    "wkv7_decode_kernel": ("wkv7_decode.hip", "wkv7_device.h"),
    "epi_fwd_kernel": ("wkv7_epilogue.hip", "wkv7_device.h"),
    "epi_bwd_kernel": ("wkv7_epilogue.hip", "wkv7_device.h"),
    "rwkv8_fwd_kernel": ("rwkv8.hip",),
    "rwkv8_bwd_kernel": ("rwkv8.hip",),
}


def kernel_sha(kernel=None):
    """Hash of the sources of `kernel` (all kernel sources when None)."""
    files = KERNEL_SOURCES if kernel is None else tuple(_CSRC + f for f in _KERNEL_FILES[kernel])
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name):
    m = re.search(r"(wkv7_\w+_kernel|rwkv8_\w+_kernel|epi_\w+_kernel|compose_\w+_kernel|sum_\w+_kernel|"
                  r"flag_reduce_kernel|fill_kernel)", name)
    if m:
        return m.group(1)
    return name[:60]


def stats(csv_path, cmd, out):
    rows = list(csv.DictReader(open(csv_path)))
    lines = ["# rocprofv3 kernel statistics", "", "Command:", "", "```", cmd, "```", "",
             "| kernel | calls | total ms | average us | min us | max us | % | sources sha |",
             "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        if "wkv7" not in name and "rwkv8" not in name and float(r.get("Percentage", 0)) < 1.0:
            continue
        k = _short(name)
        sha = kernel_sha(k) if k in _KERNEL_FILES else "-"
        lines.append(f"| `{k}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} | `{sha}` |")
    lines.append("")
    lines.append("The sha of a kernel is that of the sources it is built from; a row is current "
                 "while it matches.")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out


def sq(csv_path, cmd, out, n_simd=1024, n_cu=256, n_xcd=8, workload=None):
    sums, disp = {}, {}
    for r in csv.DictReader(open(csv_path)):
        m = re.search(r"((?:wkv7|rwkv8)_\w+_kernel)", r["Kernel_Name"])
        if not m:
            continue
        k = m.group(1)
        key = (k, r["Counter_Name"])
        sums[key] = sums.get(key, 0.0) + float(r["Counter_Value"])
        disp.setdefault(k, set()).add(r["Dispatch_Id"])
    lines = ["# rocprofv3 SQ counters per dispatch", "", "Command:", "", "```", cmd, "```", "",
             "| kernel | counter | per dispatch |", "|---|---|---|"]
    for (k, c), v in sorted(sums.items()):
        lines.append(f"| `{k}` | {c} | {v / len(disp[k]):.4e} |")
    lines += ["", "| kernel | MFMA busy / (active cycles x SIMDs) | LDS bank-conflict cycles per CU / active cycles |",
              "|---|---|---|"]
    recs = {}
    for k in sorted(disp):
        n = len(disp[k])
        act = sums.get((k, "GRBM_GUI_ACTIVE"), 0.0) / n / n_xcd
        mf = sums.get((k, "SQ_VALU_MFMA_BUSY_CYCLES"), 0.0) / n
        bc = sums.get((k, "SQ_LDS_BANK_CONFLICT"), 0.0) / n
        if act > 0:
            lines.append(f"| `{k}` | {mf / (act * n_simd):.3f} | {bc / n_cu / act:.3f} |")
            recs[k] = {"mfma_busy": mf / (act * n_simd), "lds_conflict_frac": bc / n_cu / act,
                       "kernel_sha": kernel_sha(k) if k in _KERNEL_FILES else None}
    lines += ["", "Sources sha per kernel: " + ", ".join(
        f"`{k}` `{r['kernel_sha']}`" for k, r in recs.items())]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    # one machine-readable record per kernel, read by bench.py
    if workload:
        for k, r in recs.items():
            path = os.path.join(os.path.dirname(os.path.abspath(out)),
                                f"{k.replace('_kernel', '')}_{workload}_sq.json")
            with open(path, "w") as fh:
                json.dump(dict(r, workload=workload, kernel=k, command=cmd), fh, indent=1)
    return out


def _per_dispatch(csv_path, counter):
    vals = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def _pick(vals, substr):
    hits = [v for k, v in vals.items() if substr in k]
    if not hits:
        raise SystemExit(f"no dispatches of {substr}")
    return statistics.median([x for h in hits for x in h])


def traffic(fetch_csv, write_csv, kernel, copy_bytes, workload, cmd, out):
    f = _per_dispatch(fetch_csv, "FETCH_SIZE")
    w = _per_dispatch(write_csv, "WRITE_SIZE")
    copy_key = "copy"                    # torch's elementwise copy kernel
    f_k, w_k = _pick(f, kernel), _pick(w, kernel)
    # the copy of known size is the largest copy dispatch (torch also issues
    # small host<->device copies)
    f_c = max(x for k, v in f.items() if copy_key in k.lower() for x in v)
    w_c = max(x for k, v in w.items() if copy_key in k.lower() for x in v)
    fetch_scale = copy_bytes / (f_c * 1024.0)
    write_scale = copy_bytes / (w_c * 1024.0)
    rec = {
        "workload": workload,
        "kernel": kernel,
        "kernel_sha": kernel_sha(kernel),
        "command": cmd,
        "fetch_kib_per_dispatch": f_k,
        "write_kib_per_dispatch": w_k,
        "copy_bytes": copy_bytes,
        "copy_fetch_kib": f_c,
        "copy_write_kib": w_c,
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "bytes_per_launch": f_k * 1024.0 * fetch_scale + w_k * 1024.0 * write_scale,
    }
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    return rec


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("--csv", required=True)
    a.add_argument("--cmd", required=True)
    a.add_argument("--out", required=True)
    q = sub.add_parser("sq")
    q.add_argument("--csv", required=True)
    q.add_argument("--cmd", required=True)
    q.add_argument("--out", required=True)
    q.add_argument("--workload")
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernel", default="wkv7_bwd_kernel")
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--workload", required=True)
    b.add_argument("--cmd", required=True)
    b.add_argument("--out", required=True)
    args = ap.parse_args()
    if args.what == "stats":
        print(stats(args.csv, args.cmd, args.out))
    elif args.what == "sq":
        print(sq(args.csv, args.cmd, args.out, workload=args.workload))
    else:
        print(json.dumps(traffic(args.fetch, args.write, args.kernel, args.copy_bytes,
                                 args.workload, args.cmd, args.out)))
