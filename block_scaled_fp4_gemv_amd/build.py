"""Build the HIP library libnvfp4gemv.so in-tree with hipcc for gfx950.

    python -m block_scaled_fp4_gemv_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("nvfp4_gemv.hip", "nvfp4_reblock.hip", "nvfp4_gemm_small_n.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libnvfp4gemv.so")
# the measurement helper (streaming-read reference for the bench): its own library
BENCH_SRCS = [os.path.join(PKG, "csrc", "bench", "stream_read.hip")]
BENCH_INCLUDE = os.path.join(PKG, "csrc", "bench")
BENCH_LIB = os.path.join(PKG, "libnvfp4bench.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # the direct-to-LDS copies name M0 in their clobber list on purpose
    "-Wno-inline-asm",
    # no packed-fp32 instructions: write plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # preload the leading kernel arguments into SGPRs (the GEMV kernel puts
    # the scalars its first loads depend on there)
    "-mllvm", "-amdgpu-kernarg-preload-count=14",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _build_lib(srcs, include, out, extra_flags, verbose):
    tmp = out + ".tmp"
    with tempfile.TemporaryDirectory(prefix="nvfp4_build_") as td:
        objs = [os.path.join(td, os.path.basename(src) + ".o") for src in srcs]
        cmds = [[hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-I", include, "-c", src, "-o", obj]
                for src, obj in zip(srcs, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            for r in ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), cmds):
                if r.returncode != 0:
                    sys.stderr.write(r.stdout + r.stderr)
                    raise subprocess.CalledProcessError(r.returncode, r.args)
        link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
    os.replace(tmp, out)
    return out


def build(extra_flags=None, out: str = LIB, verbose: bool = False) -> str:
    """Compile the HIP sources in csrc/ into ``out`` (one object per source,
    compiled in parallel, then linked), and the measurement helper into
    libnvfp4bench.so. Always recompiles."""
    with ThreadPoolExecutor(max_workers=2) as ex:
        f1 = ex.submit(_build_lib, SRCS, INCLUDE, out, extra_flags, verbose)
        f2 = ex.submit(_build_lib, BENCH_SRCS, BENCH_INCLUDE, BENCH_LIB, extra_flags, verbose)
        f1.result()
        f2.result()
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:], verbose=True))
