"""Build libtwl.so in-tree with hipcc for gfx950.

    python -m top_sparse_attention_int4_amd.build            # build (always recompiles)
    python -m top_sparse_attention_int4_amd.build --asm DIR  # also write gfx950 assembly per source

The library is a single shared object holding every kernel (single-source HIP, no runtime code
loading).  Floating-point contraction is off (the committed float32 roundings of the page scores and
the estimate rely on it; fused multiply-adds are written explicitly where wanted) and packed fp32
instructions are disabled.
"""

from __future__ import annotations

import argparse
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libtwl.so")

SOURCES = ["api.cpp", "quantize.hip", "select.hip", "estimate.hip", "topp.hip", "topp_wide.hip", "attention.hip",
           "cluster.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def sources() -> list[str]:
    return [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-shared", "-I", INCLUDE, "-I", CSRC, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libtwl.so")
    noise = [ln for ln in res.stderr.splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, LIB)
    return LIB


def write_asm(outdir: str) -> None:
    os.makedirs(outdir, exist_ok=True)
    for src in sources():
        if not src.endswith(".hip"):
            continue
        out = os.path.join(outdir, os.path.basename(src).replace(".hip", ".s"))
        cmd = [hipcc(), *FLAGS, "-I", INCLUDE, "-I", CSRC, "--cuda-device-only", "-S", src, "-o", out]
        subprocess.run(cmd, check=True)


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(verbose=a.verbose))
    if a.asm:
        write_asm(a.asm)


if __name__ == "__main__":
    main()
