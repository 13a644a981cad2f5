"""Build libwkv7.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m linear_attention_rnn_wkv7_amd.build [--verbose]
"""
import argparse
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libwkv7.so")
SOURCES = ["wkv7_abi.cpp", "wkv7_fwd.hip", "wkv7_bwd.hip", "wkv7_bwdc.hip", "wkv7_fwdc.hip",
           "wkv7_decode.hip", "wkv7_split.hip",
           "wkv7_epilogue.hip"]
ARCH = "gfx950"

# Packed-FP32 VALU forms are switched off for the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(out=LIB, verbose=False, extra=()):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS, *extra,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--out", default=LIB)
    args = ap.parse_args()
    print(build(args.out, args.verbose))
