"""Build libmsa.so (HIP, gfx950 only) in-tree with hipcc.

    python block_sparse_top_msa_amd/build.py [--verbose]

(run as a script: importing the package needs the library this builds)

Every call recompiles all sources (one hipcc process per translation unit,
in parallel) and links block_sparse_top_msa_amd/libmsa.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmsa.so")

SOURCES = ["api.cpp", "decode.hip", "prefill.hip", "proxy.hip", "qsa.hip", "stage16.hip",
           "tile_union.hip", "topk.hip", "validate.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU ops stay off (plain fp32 code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]

# The attention kernels take row maxima of MFMA results that are never NaN
# for valid inputs (finite bf16 / fp8 / E2M1 operands; masked scores are
# -inf): without NaN semantics the compiler drops the quieting "max x, x"
# it would otherwise put in front of every such maximum.
PER_FILE = {
    "prefill.hip": ["-fno-honor-nans"],
    "decode.hip": ["-fno-honor-nans"],
    "proxy.hip": ["-fno-honor-nans"],
    "qsa.hip": ["-fno-honor-nans"],
}


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *PER_FILE.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass warns about the gfx-only target feature; keep other output
    noise = "unknown target feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l and l.strip())
    if verbose and msg:
        print(msg, flush=True)
    return out


def build(verbose: bool = False) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv)
    print(path)
