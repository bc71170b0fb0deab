"""The compiler's resource report of the last build: no decode-step, compaction
or prompt kernel uses scratch memory (a spill, or an argument block copied to
scratch because its address escaped into a call that was not inlined, turns
every access to it into a memory round trip), and the step kernels keep the
occupancy their launch shapes assume."""
import os

import pytest

from kv_cache_eviction_h2o_amd import build as B


@pytest.fixture(scope="module")
def res():
    if not all(os.path.exists(os.path.join(B.BUILD_DIR, os.path.splitext(s)[0] + ".o.resources.txt"))
               for s in B.SOURCES if s.endswith(".hip")):
        B.build()
    return B.kernel_resources()


def test_no_kernel_uses_scratch(res):
    assert len(res) > 100
    spilled = {k: v for k, v in res.items() if v.get("scratch", 0) != 0}
    assert not spilled, sorted(spilled)[:8]


def test_step_kernels_fit_their_workgroup(res):
    # a workgroup must fit one CU: 8 waves (2 per SIMD) for the matrix-core
    # step and the FMA step with groups of 1 or 2, 4 waves (1 per SIMD) for
    # the FMA step with groups of 4 or 8
    import re
    seen = 0
    for k, v in res.items():
        m = re.search(r"(mfma_)?step_kernelI.*?Li(\d)E", k)
        if not m or "step_kernel" not in k:
            continue
        need = 2 if (m.group(1) or int(m.group(2)) <= 2) else 1
        assert v["occupancy"] >= need, (k, v)
        seen += 1
    assert seen > 100
