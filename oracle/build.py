"""Compile the fp64 CPU oracle (test infrastructure only) with gcc.

Usage: python oracle/build.py [--src FILE] [--out FILE]
"""
import argparse
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "wkv7_oracle.c")
OUT = os.path.join(HERE, "libwkv7_oracle.so")


def build(src=SRC, out=OUT):
    # -ffp-contract=off: every product and sum is rounded separately, in the
    # order the loops state.
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
           "-std=c11", "-Wall", "-Wextra", "-o", out, src]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--src", default=SRC)
    ap.add_argument("--out", default=OUT)
    args = ap.parse_args()
    print(build(args.src, args.out))
