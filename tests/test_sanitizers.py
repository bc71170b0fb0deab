"""The host-side C code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the oracle's pins, and the C ABI's host tests (validation, pool
sizing, workspace sizing, scratch sizing and rejections), each in a child
process that preloads the sanitizer runtime and loads an instrumented build
(sanitize_build.py).  Any sanitizer report fails the child."""
import os
import subprocess
import sys

import pytest

import sanitize_build as SB

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ASAN_OPTIONS = "detect_leaks=0:detect_odr_violation=0:abort_on_error=1:halt_on_error=1"


def _run_pytest(preload, env_extra, tests):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS=ASAN_OPTIONS,
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = SB.build_oracle(str(tmp_path / "liboracle_asan.so"))
    out = _run_pytest(SB.oracle_runtime(), {"H2O_ORACLE_LIB": lib}, ["tests/test_oracle_pins.py"])
    assert " passed" in out


def test_host_runtime_under_sanitizers(tmp_path):
    try:
        rt = SB.host_runtime()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    lib = SB.build_library(str(tmp_path / "libh2o_asan.so"))
    out = _run_pytest(rt, {"H2O_LIB": lib}, ["tests/test_abi.py"])
    assert " passed" in out


def test_sanitizer_setup_reports_a_planted_overflow(tmp_path):
    """Positive control on the CPU: a heap overflow planted in a tiny C file,
    built with the oracle's sanitizer flags and called from a child with the
    same preload, is reported; and the instrumented host runtime calls the
    AddressSanitizer report hooks."""
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\nint poke(int i) { int *a = malloc(16); a[i] = 1; int r = a[0]; free(a);"
                   " return r; }\n")
    so = tmp_path / "libplanted.so"
    subprocess.run(["gcc", "-shared", "-fPIC", "-O1", *SB.ORACLE_SAN, "-o", str(so), str(src)], check=True)
    code = f"import ctypes; ctypes.CDLL({str(so)!r}).poke(4)"
    env = dict(os.environ, LD_PRELOAD=SB.oracle_runtime(), ASAN_OPTIONS=ASAN_OPTIONS)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and ("heap-buffer-overflow" in r.stderr or "runtime error:" in r.stderr), \
        r.stderr[-2000:]
    try:
        SB.host_runtime()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    lib = SB.build_library(str(tmp_path / "libh2o_asan.so"))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_store" in syms and "__ubsan_handle" in syms
