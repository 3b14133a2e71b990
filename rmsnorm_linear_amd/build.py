"""Build libflashnorm.so (gfx950) in-tree with hipcc.

    python -m rmsnorm_linear_amd.build        # or: python rmsnorm_linear_amd/build.py

Each source compiles to an object in ``_build/`` in parallel; the objects
link into ``rmsnorm_linear_amd/libflashnorm.so``.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libflashnorm.so")

# (source, object name, extra flags): the prefill GEMM compiles once per
# epilogue (FN_GEMM_EPI, the Epi values of kernels.hpp) so its many
# instantiations build in parallel.
N_GEMM_EPI = 6
SOURCES = ([("gemm_bf16.hip", f"gemm_bf16_e{e}", [f"-DFN_GEMM_EPI={e}"]) for e in range(N_GEMM_EPI)] +
           [(f, os.path.splitext(f)[0], []) for f in ("api.cpp", "gemm_f32.hip", "decode.hip", "rowwise.hip")])

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(spec) -> str:
    src, name, extra = spec
    obj = os.path.join(BUILD, name + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if noise:
        sys.stderr.write(noise + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
