"""Builds libsparse_mla.so (gfx950) in-tree with hipcc.

Usage: python -m sparse_mla_attention_fp8_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsparse_mla.so")
# device code (hipcc, gfx950) and host-only code (the C ABI's validation and
# the launch plan, plain C++ built by the host compiler)
SOURCES = ["kv_write.hip", "attn.hip", "merge.hip", "gather.hip", "split_pages.hip",
           "noalloc.hip", "measure.hip", "api.cpp", "plan.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-fvisibility=hidden",
    # keep the compiler from forming packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc",
]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-fvisibility=hidden", "-D__HIP_PLATFORM_AMD__",
              "-I/opt/rocm/include"]


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        if src.endswith(".hip"):
            cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        else:
            cmd = [CXX, *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    errors = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the packed-fp32 feature; that note is harmless
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            errors.append(f"{src}:\n{text}")
        elif verbose and text.strip():
            print(text, flush=True)
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
