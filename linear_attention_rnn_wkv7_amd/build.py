"""Build libwkv7.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Each source compiles to its own object in parallel (under _build/ beside
the package), then one link makes the shared library.

Usage: python -m linear_attention_rnn_wkv7_amd.build [--verbose]
"""
import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libwkv7.so")
OBJDIR = os.path.join(ROOT, "_build")
SOURCES = ["wkv7_abi.cpp", "wkv7_fwd.hip", "wkv7_bwd.hip", "wkv7_bwdc.hip", "wkv7_fwdc.hip",
           "wkv7_decode.hip", "wkv7_split.hip",
           "wkv7_epilogue.hip", "wkv7_noalloc.hip", "rwkv8.hip"]
ARCH = "gfx950"

# Packed-FP32 VALU forms are switched off for the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
NOISE = "is not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if NOISE not in ln]
    return res.returncode, msgs


def build(out=LIB, verbose=False, extra=(), jobs=None):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tag = os.path.splitext(os.path.basename(out))[0]
    objdir = os.path.join(OBJDIR, tag)
    os.makedirs(objdir, exist_ok=True)
    common = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
              "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS, *extra]
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [common + ["-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1), 16)
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), cmds))
    failed = False
    for (rc, msgs), src in zip(results, SOURCES):
        if rc != 0:
            failed = True
            sys.stderr.write(f"--- {src}\n" + "\n".join(msgs) + "\n")
        elif verbose and msgs:
            print("\n".join(msgs))
    if failed:
        raise RuntimeError("hipcc failed")
    rc, msgs = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
                     "-o", out + ".tmp"], verbose)
    if rc != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc link failed")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--out", default=LIB)
    args = ap.parse_args()
    print(build(args.out, args.verbose))
