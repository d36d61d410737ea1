"""Build libtlg.so in-tree with hipcc for gfx950.

    python -m tiled_dense_gemm_02_amd.build        (or python tiled_dense_gemm_02_amd/build.py)

Every source is compiled on each call (the build is the "does it compile"
check).  Packed fp32 VALU instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtlg.so")

SOURCES = ["gemm_tile_256_f16.hip", "gemm_tile_256_bf16.hip", "gemm_tile_256w8_f16.hip",
           "gemm_tile_256w8_bf16.hip", "gemm_tile_128_f16.hip", "gemm_tile_128_bf16.hip",
           "gemm_lds_f16.hip", "gemm_lds_bf16.hip", "gemm_lds_sk2_f16.hip", "gemm_lds_sk2_bf16.hip", "gemm_lds32.hip", "gemm_mx.hip", "attn_fwd.hip", "gemm_w4.hip", "gemm_sp.hip", "gemm_skinny.hip", "tlg_api.cpp"]
ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtlg.so)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False, save_temps: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    if save_temps:
        DEVICE_FLAGS.extend(["-save-temps=obj"])
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, save_temps="--save-temps" in sys.argv))
