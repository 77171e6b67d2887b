"""Build the HIP library ``libmoe_mi355x.so`` for gfx950 with hipcc.

Every source in ``csrc/`` is compiled separately (in parallel) into
``_build/`` and linked into the shared library next to this file.
``python -m sparse_mixture_experts_permute_amd.build`` runs it.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmoe_mi355x.so")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # no packed-fp32 instructions anywhere in device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    subprocess.check_call([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp] + objs)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


# A plain C program that calls the library (tests/c_abi): host code only, so
# gcc builds it against the HIP runtime and the in-tree library.
C_CALLER_SRC = os.path.join(os.path.dirname(HERE), "tests", "c_abi", "moe_c_caller.c")
C_CALLER = os.path.join(os.path.dirname(HERE), "tests", "c_abi", "moe_c_caller")


def build_c_caller(verbose: bool = True) -> str:
    rocm = os.path.dirname(os.path.dirname(HIPCC))  # the ROCm root (/opt/rocm)
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
           C_CALLER_SRC, "-o", C_CALLER, f"-L{HERE}", "-lmoe_mi355x", f"-L{rocm}/lib",
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../sparse_mixture_experts_permute_amd",
           f"-Wl,-rpath,{rocm}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed for {C_CALLER_SRC}:\n{r.stdout}{r.stderr}")
    if verbose:
        print(f"built {C_CALLER}")
    return C_CALLER


if __name__ == "__main__":
    build()
    build_c_caller()
