"""Build libq4bq.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

    python -m q4_block_quantized_amd.build

Each source is compiled to an object in ``_build/`` (in parallel), then linked
into ``q4_block_quantized_amd/libq4bq.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libq4bq.so")

ARCH = "gfx950"
# measurement probes for the benchmark (not linked into the product library)
PROBE_SOURCE = "q4bq_probe.hip"
PROBE_LIB = os.path.join(PKG, "libq4bq_probe.so")
SOURCES = ["q4bq_api.cpp", "q4bq_quant.hip", "q4bq_gemv.hip", "q4bq_rows_x.hip", "q4bq_rows_act.hip",
           "q4bq_prefill.hip", "q4bq_q8w.hip", "q4bq_q8w_mm.hip", "q4bq_noalloc.hip", "q4bq_mma.hip", "q4bq_set.hip"]

# No fast-math anywhere: the quantizers need IEEE division and round-half-away.
# Packed fp32 instructions are switched off for all device code.
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results straight into VGPRs (no accumulator-register copies)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the q4bq HIP library cannot be built")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source, link libq4bq.so (the product library) and
    libq4bq_probe.so (the benchmark's peak-rate probes); returns the product
    library's path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES) + 1, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES + [PROBE_SOURCE]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
