"""The paged first step's window relink (window_remap, host and device share
it): for prompts of every length up to 5000 and a sample up to 70,000, with
and without sinks and at three budgets, the rule's page arithmetic holds and,
for random heavy-hitter sets, the holes of the front equal the rows that move.
Runs the rule itself, compiled for the host (hipcc), on the CPU."""
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PAGE = 16


def schedule(length, n_sink, num, den):
    k = length * num // den
    hh = (k - n_sink) // 2
    return k, hh, k - n_sink - hh


@pytest.fixture(scope="module")
def dump(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("wr") / "window_remap_dump")
    subprocess.run([hipcc, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "kv_cache_eviction_h2o_amd", "csrc"),
                    os.path.join(HERE, "c", "window_remap_dump.cpp"), "-o", exe], check=True,
                   capture_output=True)
    return exe


@pytest.mark.parametrize("n_sink,num,den", [(4, 1, 5), (0, 1, 5), (4, 1, 3), (4, 1, 10)])
def test_window_relink_rule(dump, n_sink, num, den):
    rng = np.random.default_rng(17 + n_sink + den)
    prompts = list(range(16, 5001)) + sorted(rng.integers(5001, 70000, 400).tolist())
    cases = []
    for p in prompts:
        t, n_att = p, p + 1  # the first decode step appends position p
        k, hh, w = schedule(t + 1, n_sink, num, den)
        e = max(0, n_att - k)
        cases.append((t, n_att, e, w))
    inp = "".join(f"{t} {n} {e} {n_sink} {num} {den}\n" for t, n, e, _ in cases)
    out = subprocess.run([dump], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
    relinked = 0
    for (t, n_att, e, w), line in zip(cases, out):
        ok, front, src, m = (int(x) for x in line.split())
        assert ok == int(w >= 32 and e >= 64 and e >= 2 * w), (t, n_att, e, w, line)
        if not ok:
            continue
        relinked += 1
        n2, a = n_att - e, n_att - w  # a: the window's first slot
        assert front % PAGE == 0 and src % PAGE == 0
        assert a <= src < a + PAGE  # the window's first whole page
        assert 0 < m <= n_att - src and front + m == n2
        assert src - front >= -(-m // PAGE) * PAGE  # relinked pages do not overlap their new entries
        for _ in range(2):
            # survivors: the sinks, the heavy hitters (any n2 - n_sink - w of the
            # candidates [n_sink, a)) and the window [a, n_att)
            keep = np.zeros(n_att, dtype=bool)
            keep[:n_sink] = True
            keep[a:] = True
            hh_n = n2 - n_sink - w
            keep[n_sink + rng.choice(a - n_sink, hh_n, replace=False)] = True
            assert keep.sum() == n2
            holes = int((~keep[:front]).sum())
            moved = int(keep[front:src].sum()) + (n_att - (src + m))
            assert holes == moved, (t, front, src, m, holes, moved)
    assert relinked > 0
