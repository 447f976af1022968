"""Builds libhs2.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

Usage: python -m long_context_mqa_amd.build   (or call build()).
Every source is compiled on each call; objects go to long_context_mqa_amd/_build/.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libhs2.so")
ARCH = "gfx950"

SOURCES = ["attn_bf16.hip", "attn_fp8.hip", "attn_chunk.hip", "score_bf16.hip", "attn_f32.hip", "topk.hip", "bridge.hip", "bridge_append.hip", "attn_v1.hip", "noalloc.hip", "sparse_attn.hip",
           "hs2_api.cpp"]
# Kernels whose MFMA results are consumed element by element every tile and that fit in
# the 256 VGPRs: MFMA destinations in VGPRs instead of accumulator registers (AGPRs),
# which saves a v_accvgpr_read per result element.
VGPR_MFMA = {"attn_chunk.hip", "score_bf16.hip", "attn_fp8.hip"}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
        "-I", INCLUDE, "-I", CSRC,
        # no packed fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    extra = ["-mllvm", "-amdgpu-mfma-vgpr-form"] if src in VGPR_MFMA else []
    cmd = [hipcc(), *common_flags(), *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
