"""Builds libawq.so (the library's HIP sources, gfx950 only) and libawq_ceilings.so (the
measurement kernels bench.py compares against) next to this file."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libawq.so")
CEILINGS_LIB = os.path.join(PKG, "libawq_ceilings.so")

SOURCES = ["awq_api.hip", "stats.hip", "gram.hip", "quant.hip", "loss.hip", "gemv.hip", "skinny.hip", "gemm.hip", "gemm_pipe.hip"]
CEILINGS_SOURCES = ["ceilings.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: no implicit multiply-add fusion, so the quantizer's fp32
#   operations round exactly as written (fused forms are spelled out in code).
# -packed-fp32-ops off: no v_pk_*_f32 instructions are generated.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]
# Per-source extras.  The pipelined W4A16 GEMM keeps its matrix-core
# accumulators in ordinary vector registers (measured faster than the
# accumulation-register form).
# The decode kernels are short enough (a few microseconds) that the kernel-argument
# load at each wave's start is on its critical path; gfx950 can preload the
# arguments into SGPRs at dispatch instead.
FILE_FLAGS = {"gemm_pipe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
              "gemv.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"],
              "skinny.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"]}


def flags_for(src: str) -> list:
    return FLAGS + FILE_FLAGS.get(os.path.basename(src), [])


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *flags_for(src), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if warn.strip() and os.environ.get("AWQ_BUILD_VERBOSE"):
        sys.stderr.write(warn + "\n")
    return obj


def _link(objs: list, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int | None = None) -> str:
    """Compiles every source, links libawq.so and libawq_ceilings.so; returns libawq.so's path."""
    os.makedirs(BUILD, exist_ok=True)
    sources = SOURCES + CEILINGS_SOURCES
    jobs = jobs or min(len(sources), 8)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = dict(zip(sources, ex.map(_compile, sources)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in CEILINGS_SOURCES], CEILINGS_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
