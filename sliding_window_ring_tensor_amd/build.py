"""Compile libswrt.so (HIP, gfx950) in place, next to this file.

    python -m sliding_window_ring_tensor_amd.build

All kernels and the C-ABI live in csrc/*.hip; the public header is
include/swrt.h at the repository root.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIBRARY = os.path.join(PKG, "libswrt.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # packed-fp32 instructions stay off in every kernel of this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: the attention kernel
    # rescales them on the VALU between products
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(out: str = LIBRARY, extra: tuple = (), verbose: bool = False) -> str:
    """Compile every csrc/*.hip (one compiler process per file, in parallel)
    and link them into one shared library; return its path."""
    tmp = out + ".tmp"
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="swrt_build_") as objdir:
        def compile_one(src: str) -> str:
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c", src,
                   "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            return obj

        jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            objs = list(pool.map(compile_one, srcs))
        link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
