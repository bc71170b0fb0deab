"""The C ABI from a plain C program (tests/c/h2o_c_check.c: include/h2o.h and
the HIP runtime only): decode steps on the matrix-core and FMA paths, fused and
step-then-compact, with the method's invariants checked after every step."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c", "h2o_c_check")


def test_c_client_invariants():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(EXE), "tests/c/h2o_c_check is missing: run __graft_entry__.build()"
    print("[c client] running tests/c/h2o_c_check", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=100)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and "c check ok" in r.stdout
