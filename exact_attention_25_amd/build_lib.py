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

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_mask.hip"]
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


def build(verbose=False, resource_usage=False, out=LIB_PATH):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + hipcc_flags(resource_usage) + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libfa.so")
    if resource_usage or verbose:
        sys.stderr.write(res.stderr)
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
