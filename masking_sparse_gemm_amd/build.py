"""Build libnm.so (the HIP kernels plus the C ABI) and libnm_probe.so (the matrix-core
rate probes of the benchmark) in-tree for gfx950 with hipcc.

Usage: ``python -m masking_sparse_gemm_amd.build`` (or ``build()`` from Python).
Sources compile in parallel to objects under ``_build/``, then link into
``masking_sparse_gemm_amd/libnm.so`` and ``masking_sparse_gemm_amd/libnm_probe.so``.
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
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libnm.so")
SOURCES = ["nm_api.hip", "nm_compress.hip", "nm_spmm.hip", "nm_spmm_sk.hip", "nm_srste.hip",
           "nm_tmask.hip", "nm_perm.hip"]
# the measurement probes (include/nm_probe.h) link into a library of their own
PROBE_SOURCES = ["nm_probe.hip"]
PROBE_LIB = os.path.join(HERE, "libnm_probe.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnm)")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        # never emit packed-fp32 VALU instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


def _stale(src: str, obj: str) -> bool:
    """The object is older than its source or any header of the package."""
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, h) for h in os.listdir(CSRC)
                                        if h.endswith(".h")] + [os.path.join(ROOT, "include", "nm.h")]
    return any(os.path.getmtime(d) > os.path.getmtime(obj) for d in deps)


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    if incremental and not _stale(src, obj):
        return obj
    cmd = [hipcc(), *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source (or, with incremental=True, only those whose object is stale)
    and link libnm.so."""
    os.makedirs(OBJ, exist_ok=True)
    every = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=len(every)) as ex:
        objs = dict(zip(every, ex.map(lambda src: _compile(src, incremental), every)))
    for lib, srcs in ((LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)):
        tmp = lib + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *[objs[s] for s in srcs],
               "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stderr}")
        os.replace(tmp, lib)
        if verbose:
            print(f"built {lib}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
    sys.exit(0)
