"""Build libdhpt_gemm.so in-tree with hipcc for gfx950 (no GPU needed)."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdhpt_gemm.so")
# Profiling variant: the same kernels recording a per-wave timeline
# (-DDHPT_TIMELINE); loaded only by bench.py --timeline.
TIMELINE_LIB = os.path.join(PKG, "libdhpt_gemm_timeline.so")
ARCH = "gfx950"

SOURCES = ["gemm_api.cpp", "gemm_instances.hip", "gemm_dl_nn.hip", "gemm_dl_nn_epi.hip",
           "gemm_dl_tn.hip", "gemm_dl_tn_epi.hip", "gemm_ks.hip", "gemm_ks_epi.hip",
           "gemm_dl_f8_tn.hip", "gemm_dl_f8_tn_epi.hip", "gemm_dl_f8_nn.hip", "gemm_dl_f8_nn_epi.hip",
           "gemm_pk_nn.hip", "gemm_pk_nn_epi.hip", "gemm_pk_tn.hip", "gemm_pk_tn_epi.hip", "gemm_pp.hip",
           "gemm_sk.hip"]

# Packed-fp32 VALU ops stay disabled in every HIP translation unit.
HIP_FLAGS = ["-x", "hip", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
             "-Wall", "-Wno-unused-command-line-argument",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + INCLUDE, "-I" + CSRC]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False, extra_flags=None, timeline: bool = False) -> str:
    """Compile every source and link the shared library.  Always recompiles.
    timeline=True builds the profiling variant instead."""
    build_dir = os.path.join(PKG, "_build_timeline" if timeline else "_build")
    lib = TIMELINE_LIB if timeline else LIB
    extra_flags = list(extra_flags or []) + (["-DDHPT_TIMELINE"] if timeline else [])
    os.makedirs(build_dir, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc()] + HIP_FLAGS + list(extra_flags or []) + ["-c", os.path.join(CSRC, src),
                                                                  "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((cmd, obj))
    # one compiler process per translation unit, a few at a time
    workers = max(1, min(len(jobs), (os.cpu_count() or 2) // 2, 8))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda j: subprocess.run(j[0], check=True,
                                             stderr=None if verbose else subprocess.PIPE), jobs))
    objs = [obj for _, obj in jobs]
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, timeline="--timeline" in sys.argv))
