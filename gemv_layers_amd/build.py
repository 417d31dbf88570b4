"""Build the gfx950 library libgemm_bf16.so in-tree with hipcc (no GPU needed to compile)."""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libgemm_bf16.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["gemm_tile.hip", "gemm_skinny.hip", "gemm_generic.hip", "gemm_mx.hip", "gemm_packed.hip",
           "peak.hip", "plan.cpp", "abi.cpp"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions in device code (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int | None = None) -> str:
    """Compile every source and link libgemm_bf16.so next to this file. Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(16, len(os.sched_getaffinity(0)))))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else None))
