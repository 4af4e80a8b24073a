"""Build libkvq.so (HIP, gfx950) in-tree with hipcc.

Every source is compiled for gfx950 only, with packed-fp32 VALU forms
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops), then linked
into ``libkvq.so`` next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvq.so")
SOURCES = ["kvq_api.cpp", "kvq_quant.hip", "kvq_attn.hip", "kvq_topk.hip",
           "kvq_gather.hip"]
# Sources whose results must match a binary32 definition bit for bit: no
# multiply-add fusion anywhere in the translation unit (headers included).
EXACT = {"kvq_quant.hip", "kvq_topk.hip", "kvq_gather.hip"}
# Sources with no NaN inputs by construction: min/max need no canonicalizing
# of their operands.
NO_NANS = {"kvq_attn.hip"}

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP toolchain is required")
    return exe


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    extra = ["-ffp-contract=off"] if src in EXACT else []
    if src in NO_NANS:
        extra += ["-fno-honor-nans"]
    cmd = [_hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
