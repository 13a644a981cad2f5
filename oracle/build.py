"""Compile the fp64 CPU oracle (test infrastructure only) with gcc.

Usage: python oracle/build.py [--src FILE] [--out FILE]   (no arguments: both oracles)
"""
import argparse
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "wkv7_oracle.c")
OUT = os.path.join(HERE, "libwkv7_oracle.so")
RWKV8_SRC = os.path.join(HERE, "rwkv8_oracle.c")
RWKV8_OUT = os.path.join(HERE, "librwkv8_oracle.so")


def build(src=SRC, out=OUT):
    # -ffp-contract=off: every product and sum is rounded separately, in the
    # order the loops state.
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
           "-std=c11", "-Wall", "-Wextra", "-o", out, src]
    subprocess.run(cmd, check=True)
    return out


def build_all():
    """Both oracles: WKV7 and the RWKV-8 rho recurrence."""
    return [build(SRC, OUT), build(RWKV8_SRC, RWKV8_OUT)]


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--src")
    ap.add_argument("--out")
    args = ap.parse_args()
    if args.src:
        print(build(args.src, args.out or OUT))
    else:
        print(build_all())
