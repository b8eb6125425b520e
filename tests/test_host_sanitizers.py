"""The host library under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C-ABI layer (``csrc/api.cpp``: argument validation, workspace planning, kernel orchestration) is
compiled with both sanitizers for the host and linked, with the kernels as built, into a small C
driver (``tests/host_abi_check.c``) that drives every entry point through its rejection paths and the
pure host queries, including shapes at and past the documented size limits.  Nothing reaches a GPU:
each call returns before its first HIP call (or fails it, on a machine without one).  The oracle is
numpy only and has no native code to sanitise."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm/bin"
KERNEL_SOURCES = ["quantize.hip", "select.hip", "estimate.hip", "topp.hip", "topp_wide.hip", "attention.hip",
                  "cluster.hip", "noalloc.hip"]


def _tools():
    from top_sparse_attention_int4_amd import build
    cc, cxx = os.path.join(LLVM, "clang"), os.path.join(LLVM, "clang++")
    have_hipcc = os.path.exists(build.hipcc()) or shutil.which(build.hipcc()) is not None
    if not (os.path.exists(cc) and os.path.exists(cxx) and have_hipcc):
        pytest.skip("ROCm clang/hipcc not available")
    return build, cc, cxx


def test_abi_validation_under_asan_and_ubsan(tmp_path):
    build, cc, cxx = _tools()
    import top_sparse_attention_int4_amd as twl
    try:
        twl.lib()  # the kernel objects under _build/ belong to the library built from this tree
    except ImportError:
        build.build()
    objs = [os.path.join(ROOT, "_build", s + ".o") for s in KERNEL_SOURCES]
    assert all(os.path.exists(o) for o in objs)
    api_o, drv_o, exe = str(tmp_path / "api.o"), str(tmp_path / "drv.o"), str(tmp_path / "abi_check")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    define = f'-DTWL_SOURCE_HASH="{build.source_hash()}"'
    subprocess.run([build.hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
                    *host_san, define, "-I", os.path.join(ROOT, "include"), "-I", build.CSRC, "-c",
                    os.path.join(build.CSRC, "api.cpp"), "-o", api_o], check=True, capture_output=True)
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    subprocess.run([cc, "-O1", "-g", *san, "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(ROOT, "tests", "host_abi_check.c"), "-o", drv_o], check=True, capture_output=True)
    subprocess.run([cxx, *san, drv_o, api_o, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                    "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("TWL_TRACE", None)
    # plain, and with the optional roctx ranges switched on (the tracer loads roctx at run time)
    for trace in (None, "1"):
        if trace:
            env["TWL_TRACE"] = trace
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "host ABI checks passed" in r.stdout
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
