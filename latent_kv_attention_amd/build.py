"""Compile the HIP sources under csrc/ into libmla355.so for gfx950.

Usage: python -m latent_kv_attention_amd.build   (or call build()).
Each source is compiled in parallel to an object under _build/, then linked
into one shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libmla355.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["mla_abi.hip", "rope_tables.hip", "cache_write.hip", "absorb_q.hip", "flash_mla.hip", "up_v.hip",
           "heads_mha.hip", "proj_gemm.hip", "noalloc.hip"]

# The matrix-core ceiling probe (a measurement aid for bench.py) goes into a
# library of its own, so libmla355.so exports exactly what include/mla.h declares.
CEILING_SOURCE = "mfma_ceiling.hip"
CEILING_LIB_PATH = os.path.join(HERE, "libmla355_ceiling.so")

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU instructions.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# Per-source additions (none at present: the attention kernel orders its
# own operand reads and products with scheduling barriers).
SOURCE_FLAGS: dict = {}


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line and "not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link the library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        _run([hipcc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), *inc, "-c", os.path.join(CSRC, src), "-o", obj],
             verbose)
        return obj

    jobs = jobs or min(len(SOURCES) + 1, max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES + [CEILING_SOURCE]))
    for path, parts in ((LIB_PATH, objs[:-1]), (CEILING_LIB_PATH, objs[-1:])):
        tmp = path + ".tmp"
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *parts], verbose)
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
