"""Build libsv.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python verify_pass_amd/csrc/build.py [-v]

Runs as a plain script (it does not import the package, whose import loads
the library being rebuilt).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

CSRC = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(CSRC)
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsv.so")
SOURCES = ["sv_prep.hip", "sv_gemm.hip", "sv_gemm_bf16.hip", "sv_gemm_int4.hip", "sv_gemm_f32.hip",
           "sv_attn.hip", "sv_head.hip", "sv_accept.hip", "sv_accept_noalloc.hip", "sv_tree.hip", "sv_abi.cpp",
           "sv_plan.cpp", "sv_sched.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall", "-Wno-unused-function",
         # keep the compiler from emitting packed-fp32 VALU instructions
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg, flush=True)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    # -z defs: a symbol left undefined (e.g. a kernel whose host stub was not
    # emitted) fails the link instead of the first dlopen
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
