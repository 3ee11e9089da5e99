"""Compile the HIP sources under csrc/ into ``libgpt2mi.so`` for gfx950.

Run as ``python -m transformer_lm_step_flat_amd.build``.  hipcc cross-compiles,
so no GPU is needed.  Packed fp32 instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgpt2mi.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["gpt2.hip", "gemm.hip", "kernels.hip", "attention.hip", "probe.hip", "noalloc.hip", "decode.hip", "checkpoint.cpp", "audit.cpp"]
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, obj: str) -> None:
    if src.endswith(".cpp"):  # host-only C++ (no device code)
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-c", os.path.join(CSRC, src), "-o", obj]
    else:
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; anything else is shown
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if msgs:
        print("\n".join(msgs), file=sys.stderr)


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda a: _compile(*a), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
