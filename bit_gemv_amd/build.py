"""Build libquant.so (the HIP/gfx950 C-ABI library) in-tree with hipcc.

    python -m bit_gemv_amd.build

compiles every source under ``csrc/`` for gfx950 into ``_build/`` and links
``bit_gemv_amd/libquant.so``. hipcc cross-compiles without a GPU.
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
LIB = os.path.join(HERE, "libquant.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["api.cpp", "quantize.hip", "gemv.hip", "gemv_shared.hip", "gemv8.hip", "gemm.hip", "smooth.hip", "w8a8.hip", "awq.hip", "mx.hip", "gptq.hip", "probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Bit-exact encoding: no FMA contraction, IEEE division/sqrt (HIP default),
    # no fast-math.
    "-ffp-contract=off",
    # Packed fp32 VALU ops off (the compiler would otherwise form them from
    # scalar or float2 code).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-Wall", "-Wno-unused-function",
]
# Per-source extras. The MFMA kernels keep their accumulators in VGPRs: with
# the default heuristic the register allocator places loop-carried MFMA
# accumulators in AGPRs and shuffles them with v_accvgpr moves every
# iteration.
EXTRA = {
    "w8a8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "gemv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "gemv_shared.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "awq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *CXXFLAGS, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile all sources and link libquant.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    build()
    sys.exit(0)
