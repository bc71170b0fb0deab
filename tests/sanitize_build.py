"""Sanitizer builds of the host-side C code -- TEST INFRASTRUCTURE ONLY.

The CPU oracle (plain C) is built with gcc and the library's host runtime
(h2o_runtime.cpp: validation, the schedule mirror, page and scratch
bookkeeping) with hipcc, host side only, each with AddressSanitizer and
UndefinedBehaviorSanitizer; the device code is linked in unchanged (no
sanitizer reaches the GPU).  test_sanitizers.py runs the CPU tests against
these builds in child processes that preload the matching sanitizer runtime.
"""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# gcc, one line, the oracle only
ORACLE_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
# hipcc: every sanitizer flag applies to the host compilation only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def oracle_runtime() -> str:
    """gcc's AddressSanitizer runtime, to preload before Python."""
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def host_runtime() -> str:
    """The ROCm clang AddressSanitizer runtime (it carries the UBSan handlers)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def build_oracle(out: str) -> str:
    from oracle.build import build
    return build(out=out, extra=ORACLE_SAN)


def build_library(out: str) -> str:
    """libh2o.so with the host runtime instrumented: h2o_runtime.cpp recompiled,
    linked with the device objects of the last normal build."""
    from kv_cache_eviction_h2o_amd import build as B
    objs = [os.path.join(B.BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    rt_obj = out + ".runtime.o"
    cmd = [B.HIPCC, *B.FLAGS, *HOST_SAN, "-c", os.path.join(B.CSRC, "h2o_runtime.cpp"), "-o", rt_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(r.stderr[-4000:])
    cmd = [B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *HOST_SAN, "-shared-libsan", "-o", out,
           *objs, rt_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(r.stderr[-4000:])
    return out
