"""Builds the HIP attention library in-tree for gfx950.

``python -m scaled_dot_product_attn_amd._build`` compiles every ``csrc/*.hip``
source with hipcc (offload arch gfx950) and links
``scaled_dot_product_attn_amd/libattn_mi355x.so``.  It always recompiles.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libattn_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["attn_api.hip", "attn_fwd_bf16.hip", "attn_fwd_f32.hip", "attn_decode.hip",
           "attn_bwd.hip", "attn_sparse.hip"]

# Packed fp32 VALU forms are switched off for all device code.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n"
                           f"{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for cmd, _ in zip(cmds, ex.map(_run, cmds)):
            if verbose:
                print(" ".join(cmd), flush=True)
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
          "-Wl,-rpath,/opt/rocm/lib", "-Wno-unused-command-line-argument"])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH, flush=True)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
