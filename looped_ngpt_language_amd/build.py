"""Build libdory.so (HIP kernels + host runtime) and its bounds-checked debug build
libdory_checked.so for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdory.so")
OBJ = os.path.join(ROOT, "_build")
SOURCES = ["k_rows.hip", "k_attn.hip", "k_gemm.hip", "k_gemv.hip", "k_sample.hip", "dory.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I" + os.path.join(ROOT, "include"),
         # no packed-fp32 instructions in device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]


# the bounds-checked debug build: page-table, page-id and RoPE-row guards in the attention
# kernels and a slot-region check in the host runtime (DORY_CHECKED=1)
CHECKED_LIB = os.path.join(HERE, "libdory_checked.so")
CHECKED_OBJ = os.path.join(OBJ, "checked")


def _compile(job) -> str:
    src, checked = job
    obj = os.path.join(CHECKED_OBJ if checked else OBJ, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    defs = ["-DDORY_CHECKED=1"] if checked else []
    cmd = [HIPCC, *lang, *FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    """Compile libdory.so and its checked debug build libdory_checked.so; returns the former's path."""
    os.makedirs(CHECKED_OBJ, exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + [(src, True) for src in SOURCES]
    with ThreadPoolExecutor(min(len(jobs), max(1, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(_compile, jobs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], CHECKED_LIB)
    if verbose:
        print(f"built {LIB} and {CHECKED_LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
