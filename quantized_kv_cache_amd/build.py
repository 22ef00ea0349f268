"""Build libqkv.so (HIP kernels + C-ABI) for gfx950 with hipcc, in-tree.

Usage: python -m quantized_kv_cache_amd.build   (or build() from Python).
Objects go to quantized_kv_cache_amd/_build/, the library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqkv.so")
ROOT = os.path.dirname(HERE)

SOURCES = ["qkv_api.cpp", "qkv_quantize.hip", "qkv_attn_generic.hip", "qkv_attn_matrix.hip",
           "qkv_attn_narrow.hip", "qkv_prefill_matrix.hip", "qkv_merge.hip", "qkv_measure.hip", "qkv_static.hip",
           "qkv_unfused.hip", "qkv_dequant.hip", "qkv_attn_stream.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-fno-fast-math", "-ffp-contract=on",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # packed fp32 arithmetic is kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


# per-source additions: the quantize kernels take finite inputs (a NaN or an
# infinity in a group gives unspecified codes for it), which lets min/max
# reductions skip NaN quieting and fold their DPP lane moves into the min/max
FILE_FLAGS = {"qkv_quantize.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> str:
    out = os.path.join(OBJ, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *lang, *FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
