"""Compile libfa.so for gfx950 with hipcc (runs on a machine without a GPU).

    python -m exact_attention_25_amd.build_lib [--resource-usage]

All HIP code is compiled with packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_mask.hip", "fa_noalloc.hip", "fa_fwd_d128.hip", "fa_fwd_short.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def hipcc_flags(resource_usage=False):
    flags = [
        "--offload-arch=" + ARCH,
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I" + INCLUDE,
        "-I" + CSRC,
        "-Wall",
        "-Wno-unused-function",
    ]
    if resource_usage:
        flags += ["-Rpass-analysis=kernel-resource-usage"]
    return flags


def _run(cmd, verbose, show_stderr, what):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed: " + what)
    if show_stderr:
        sys.stderr.write(res.stderr)


def build(verbose=False, resource_usage=False, out=LIB_PATH):
    """Compile every source to an object in parallel (one hipcc each), then
    link libfa.so; the library is replaced only when everything succeeded."""
    from concurrent.futures import ThreadPoolExecutor
    import tempfile

    compile_flags = [f for f in hipcc_flags(resource_usage) if f != "-shared"]
    tmp = out + ".tmp%d" % os.getpid()
    with tempfile.TemporaryDirectory(prefix="fa_build_") as d:
        objs = [os.path.join(d, s + ".o") for s in SOURCES]
        jobs = [([HIPCC] + compile_flags + ["-c", os.path.join(CSRC, s), "-o", o], s) for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as pool:
            for f in [pool.submit(_run, cmd, verbose, resource_usage or verbose, s) for cmd, s in jobs]:
                f.result()
        _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp], verbose, verbose,
             "linking libfa.so")
    os.replace(tmp, out)
    return out


def build_c_client(verbose=False):
    """Compile tests/c_abi_client.cpp (a torch-free client of the C ABI) into
    tests/c_abi_client, linked against libfa.so by its in-tree path."""
    src = os.path.join(ROOT, "tests", "c_abi_client.cpp")
    out = os.path.join(ROOT, "tests", "c_abi_client")
    cmd = [HIPCC, "-O2", "-std=c++17", "-I" + INCLUDE, src, "-o", out + ".tmp",
           "-L" + PKG_DIR, "-lfa", "-Wl,-rpath," + PKG_DIR]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building the C ABI client")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True, resource_usage="--resource-usage" in sys.argv)
