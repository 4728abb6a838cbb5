"""Build ``libattn.so`` (the C-ABI library and its gfx950 kernels) in-tree.

Every HIP source is compiled with hipcc for gfx950 only; packed fp32 vector
instructions are disabled for device code.  Objects go to ``_build/`` next to
this file and the library to ``exact_attention_124_amd/libattn.so``.

    python -m exact_attention_124_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libattn.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

ARCH = "gfx950"
SOURCES = ["attn_api.cpp", "attn_fwd_bf16.hip", "attn_fwd_bf16_dense.hip", "attn_fwd_bf16_persistent.hip",
           "attn_fwd_f32.hip", "attn_unfused.hip",
           "attn_bwd_bf16.hip", "attn_fwd_fp8.hip", "attn_fwd_masked.hip", "ew_chain.hip"]
# Per-file extra flags.  The fused bf16 kernel never produces or relies on NaN
# (inputs are required to be finite), which lets max reductions use v_max3
# without canonicalising every operand.
EXTRA = {"attn_fwd_bf16.hip": ["-fno-honor-nans"], "attn_bwd_bf16.hip": ["-fno-honor-nans"],
         "attn_fwd_fp8.hip": ["-fno-honor-nans"],
         # the non-causal 8-wave forward: LLVM's iterative ILP machine scheduler
         "attn_fwd_bf16_dense.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
         # the persistent forward: LLVM's max-memory-clause machine scheduler
         "attn_fwd_bf16_persistent.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]}
# The masked kernel compares against -inf and keeps rows at -inf on purpose,
# so it is built with the default floating-point semantics.


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libattn.so")


def common_flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}",
            "-Wall", "-Wno-unused-function",
            # no packed fp32 (v_pk_*_f32) in device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libattn.so``; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
