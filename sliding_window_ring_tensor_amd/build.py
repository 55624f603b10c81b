"""Compile libswrt.so (HIP, gfx950) in place, next to this file.

    python -m sliding_window_ring_tensor_amd.build

All kernels and the C-ABI live in csrc/*.hip; the public header is
include/swrt.h at the repository root.
"""
from __future__ import annotations

import glob
import os
import re
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
    # every `#pragma unroll` tile loop unrolls in full: a fused tile of byte
    # targets (sixteen elements a word, each with its own scale) is past the
    # default size limit, and a rolled loop indexes its word array
    "-mllvm", "-pragma-unroll-threshold=65536",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


# the compiler's per-kernel resource remarks: a kernel name, then its figures
_RESOURCE = "-Rpass-analysis=kernel-resource-usage"
_NAME = re.compile(r"remark: Function Name: (\S+)")
_SCRATCH = re.compile(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)")


def scratch_kernels(remarks: str) -> list[tuple[str, int]]:
    """(kernel, bytes per lane) of every kernel whose resource remark reports
    private (scratch) memory."""
    found, name = [], None
    for line in remarks.splitlines():
        m = _NAME.search(line)
        if m:
            name = m.group(1)
            continue
        m = _SCRATCH.search(line)
        if m and int(m.group(1)) > 0:
            found.append((name, int(m.group(1))))
    return found


def build(out: str = LIBRARY, extra: tuple = (), verbose: bool = False) -> str:
    """Compile every csrc/*.hip (one compiler process per file, in parallel)
    and link them into one shared library; return its path.

    No kernel of the library may use scratch memory: every one keeps its
    state in registers and LDS, and a stack frame (a spill, or the argument
    block copied to private memory for an indexed access) costs a large
    multiple of a kernel's HBM time. The build reads the compiler's resource
    remarks and fails on any kernel that has one."""
    tmp = out + ".tmp"
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="swrt_build_") as objdir:
        def compile_one(src: str) -> str:
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            cmd = [HIPCC, *FLAGS, *extra, _RESOURCE, "-fno-caret-diagnostics", "-I",
                   os.path.join(ROOT, "include"), "-c",
                   src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            notes = [ln for ln in r.stderr.splitlines() if _RESOURCE not in ln]
            if notes:
                print("\n".join(notes), file=sys.stderr, flush=True)
            if r.returncode:
                raise subprocess.CalledProcessError(r.returncode, cmd)
            spills = scratch_kernels(r.stderr)
            if spills:
                raise RuntimeError(f"{os.path.basename(src)}: kernels with scratch memory: "
                                   + ", ".join(f"{n} ({b} B/lane)" for n, b in spills))
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
