"""Build libfp4q.so in-tree with hipcc for gfx950.

    python block_scaled_fp4_e4m3_amd/build.py [--changed]

Every source under csrc/ is compiled to an object in _build/ (in parallel),
then linked into block_scaled_fp4_e4m3_amd/libfp4q.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfp4q.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["abi.cpp", "quantize.hip", "gemm.hip", "macaq.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # exact IEEE steps: no implicit contraction, FP32 denormals kept
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    # keep the compiler from forming packed FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature; drop that notice
    noise = [ln for ln in r.stderr.splitlines() if ln.strip() and "packed-fp32-ops" not in ln
             and "not a recognized feature" not in ln]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def _stale(src: str) -> bool:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src), os.path.join(os.path.dirname(PKG), "include", "fp4q.h")]
    deps += [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".hpp")]
    return any(os.path.getmtime(d) > os.path.getmtime(obj) for d in deps)


def build(verbose: bool = True, changed_only: bool = False) -> str:
    """Compile every source (or, with changed_only, those newer than their
    objects) and link libfp4q.so."""
    os.makedirs(BUILD, exist_ok=True)
    todo = [s for s in SOURCES if _stale(s)] if changed_only else SOURCES
    with ThreadPoolExecutor(max_workers=max(1, min(len(todo), os.cpu_count() or 1))) as ex:
        list(ex.map(_compile, todo))
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(changed_only="--changed" in sys.argv[1:])
