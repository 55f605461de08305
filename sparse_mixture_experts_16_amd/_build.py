"""Builds libmoe.so (the HIP kernels and the C-ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")

SOURCES = ["api.cpp", "route.hip", "permute.hip", "ffn_gemv.hip", "decode.hip", "gemm.hip", "mxgemm.hip",
           "misc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed-fp32 instructions (v_pk_*_f32): keep every fp32 op scalar
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = ["hipcc", *HIPCC_FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


PEAKS_SRC = "peaks.hip"
PEAKS_LIB = os.path.join(HERE, "libmoe_peaks.so")


def _link(objs, lib):
    tmp = lib + ".tmp"
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, lib)
    print(f"built {lib}", flush=True)


def build(extra_flags=()) -> str:
    """libmoe.so (the layer) and libmoe_peaks.so (the benchmark's device peak probes)."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra_flags)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES + [PEAKS_SRC]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    build()
