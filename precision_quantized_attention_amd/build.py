"""Builds libkq.so in-tree for gfx950 with hipcc (cross-compiles without a GPU)."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkq.so")
ARCH = "gfx950"

SOURCES = ["kq_api.cpp", "quant.hip", "attn_fp8.hip", "gemm.hip", "svdquant_host.cpp"]

# Test-only probe of the matrix instructions' accumulation (tests/probe), built beside libkq.
PROBE_SRC = os.path.join(ROOT, "tests", "probe", "mfma_probe.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "probe", "libmfma_probe.so")

# Packed FP32 VALU ops stay off: every FP32 instruction is a plain single-lane one.
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]
# quant.hip: bit-exact rounding, no fused multiply-add contraction.
# attn_fp8.hip: inputs are finite E4M3 codes, so NaN handling is relaxed and the IEEE mode bit
# is off, which lets fmaxf lower to a bare v_max/v_max3 (no NaN-quieting canonicalize).
PER_FILE = {"quant.hip": ["-ffp-contract=off"],
            "attn_fp8.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    out = os.path.join(OBJ, src + ".o")
    cmd = [hipcc(), *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source and link libkq.so next to this file; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    if os.path.exists(PROBE_SRC):
        tmp = PROBE_LIB + ".tmp"
        cmd = [hipcc(), *COMMON, "-shared", PROBE_SRC, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for the probe:\n{r.stderr}")
        os.replace(tmp, PROBE_LIB)
        if verbose:
            print(f"built {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
