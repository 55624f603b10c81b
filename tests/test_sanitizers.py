"""AddressSanitizer and UndefinedBehaviorSanitizer runs on the CPU.

* The oracle: tests/sanitize/oracle_fuzz.c calls every oracle entry point on
  random small shapes and edge cases with buffers of exactly the bytes a call
  may touch, built with gcc together with oracle/swrt_oracle.c (the sanitizer
  runtimes linked into the executable).
* The library's host code: the argument checks, plans and size arithmetic in
  front of every kernel launch. Every csrc/*.hip is compiled for the host only
  (the sanitizers on the host pass) and linked with tests/sanitize/host_fuzz.cpp,
  which calls each C-ABI entry point with made-up device addresses, exact host
  arrays and sizes from small values up to the extremes. No GPU is involved:
  a call that passes every check fails at its launch. Host-only objects still
  name their device code objects, which a host-only build does not produce;
  each gets an empty offload bundle in their place (nothing is launched).

Each run first checks that its sanitizer is live (a planted one-byte overrun
must be reported), then runs its rounds clean.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from sliding_window_ring_tensor_amd import build as swrt_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe, *args):
    return subprocess.run([exe, *args], capture_output=True, text=True, env=ENV, timeout=300)


def _check_live_and_clean(exe, rounds):
    bad = _run(exe, "--overrun")  # reported by ASan, or first by UBSan's object-size check
    assert bad.returncode != 0 and ("heap-buffer-overflow" in bad.stderr or
                                    "insufficient space" in bad.stderr), bad.stderr[-2000:]
    ok = _run(exe, str(rounds))
    assert ok.returncode == 0, (ok.stdout + ok.stderr)[-4000:]
    assert "runtime error" not in ok.stderr and "ERROR: AddressSanitizer" not in ok.stderr
    return ok.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_fuzz")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-Wall", "-Wextra",
                    "-Werror", *SAN_FLAGS, "-fsanitize=float-cast-overflow", "-static-libasan",
                    "-static-libubsan", os.path.join(SAN, "oracle_fuzz.c"),
                    os.path.join(ROOT, "oracle", "swrt_oracle.c"), "-o", exe, "-lm"],
                   check=True, capture_output=True)
    out = _check_live_and_clean(exe, 20000)
    m = re.search(r"ok (\d+), invalid (\d+)", out)
    assert m and int(m.group(1)) > 50000, out  # most calls reach the definitions' work


def test_host_validation_under_sanitizers(tmp_path):
    hipcc, clang = swrt_build.HIPCC, "/opt/rocm/llvm/bin/clang++"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not found")
    inc = os.path.join(ROOT, "include")
    host_san = [a for f in SAN_FLAGS for a in ("-Xarch_host", f)]
    srcs = swrt_build.sources() + [os.path.join(SAN, "host_fuzz.cpp")]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run([hipcc, "-x", "hip", "--cuda-host-only", "-O1", "-g", "-std=c++17",
                        *host_san, "-I", inc, "-c", src, "-o", obj],
                       check=True, capture_output=True)
        return obj

    with ThreadPoolExecutor(max_workers=8) as pool:
        objs = list(pool.map(compile_one, srcs))
    nm = shutil.which("nm") or "/opt/rocm/llvm/bin/llvm-nm"
    undef = subprocess.run([nm, "-u", *objs], check=True, capture_output=True, text=True).stdout
    names = sorted(set(re.findall(r"__hip_fatbin_[0-9a-f]+", undef)))
    stub = tmp_path / "bundles.c"
    stub.write_text("".join(f'__attribute__((aligned(4096))) const unsigned char {n}[32] = '
                            f'"__CLANG_OFFLOAD_BUNDLE__";\n' for n in names))
    subprocess.run(["gcc", "-c", str(stub), "-o", str(tmp_path / "bundles.o")], check=True)
    exe = str(tmp_path / "host_fuzz")
    subprocess.run([clang, *SAN_FLAGS, *objs, str(tmp_path / "bundles.o"), "-L/opt/rocm/lib",
                    "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                   check=True, capture_output=True)
    out = _check_live_and_clean(exe, 100000)
    m = re.search(r"launch (\d+)", out)
    assert m and int(m.group(1)) > 10000, out  # many calls pass every check
