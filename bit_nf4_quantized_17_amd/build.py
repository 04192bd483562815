"""Build libqlora_nf4.so (gfx950) in-tree with hipcc, and the benchmark's
context kernels into libqlora_probes.so.

Usage: python -m bit_nf4_quantized_17_amd.build   (or build() from Python)

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled (-packed-fp32-ops) and fp32 denormals kept.  The encode
kernels are compiled with -ffp-contract=off so every float operation is the
single IEEE operation written.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqlora_nf4.so")

SOURCES = {
    "quant.hip": ["-ffp-contract=off"],
    "gemm.hip": [],
    "gemm_big.hip": [],
    "decode.hip": [],
    "merge.hip": [],
    "optim.hip": [],
    "capi.hip": [],
}

# context kernels of the benchmark, linked into a library of their own
PROBES = "probes.hip"
PROBES_LIB = os.path.join(HERE, "libqlora_probes.so")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = dict(SOURCES)
    jobs[PROBES] = []
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = dict(zip(jobs, ex.map(lambda kv: _compile(*kv), jobs.items())))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[PROBES]], PROBES_LIB)
    if verbose:
        print("built", LIB, "and", PROBES_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
