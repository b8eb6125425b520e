"""Build libtwl.so in-tree with hipcc for gfx950.

    python -m top_sparse_attention_int4_amd.build            # build (always recompiles)
    python -m top_sparse_attention_int4_amd.build --asm DIR  # also write gfx950 assembly per source

The library is a single shared object holding every kernel (single-source HIP, no runtime code
loading).  Floating-point contraction is off (the committed float32 roundings of the page scores and
the estimate rely on it; fused multiply-adds are written explicitly where wanted), packed fp32
instructions are disabled, and matrix-core instructions write their results to ordinary VGPRs.
"""

from __future__ import annotations

import argparse
import hashlib
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
           "cluster.hip", "noalloc.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results straight into VGPRs (no accumulator-register reads after every MFMA)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def source_hash() -> str:
    """sha256 (first 16 hex digits) of every file under csrc/ and of include/twl.h, the sources the
    library is built from; embedded in the library's version string and checked when it is loaded."""
    h = hashlib.sha256()
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))] + [os.path.join(INCLUDE, "twl.h")]
    for f in files:
        if os.path.isfile(f):
            with open(f, "rb") as fh:
                h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def sources() -> list[str]:
    return [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel, under _build/), then link libtwl.so."""
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    define = f'-DTWL_SOURCE_HASH="{source_hash()}"'
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [hipcc(), *FLAGS, define, "-c", "-I", INCLUDE, "-I", CSRC, src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    failed = False
    for src, pr in procs:
        out, err = pr.communicate()
        if pr.returncode != 0:
            sys.stderr.write(out + err)
            failed = True
        elif verbose:
            noise = [ln for ln in err.splitlines()
                     if ln.strip() and "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
            if noise:
                sys.stderr.write("\n".join(noise) + "\n")
    if failed:
        raise RuntimeError("hipcc failed building libtwl.so")
    tmp = LIB + ".tmp"
    res = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                         capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed linking libtwl.so")
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
