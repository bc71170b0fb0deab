"""Host byte accounting against the figures the pages print (no GPU)."""
import json
import os

import numpy as np
import pytest

from kv_cache_eviction_h2o_amd import metrics as M
from kv_cache_eviction_h2o_amd import workloads as WL

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _g(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_full_kv_cache_size_70b_32k():
    g = _g("kv_cache_size_70b_32k.json")
    per_tok = M.kv_bytes_per_token(g["n_layers"], g["n_kv_heads"], g["head_dim"], g["elem_bytes"])
    gb = per_tok * g["tokens"] / 1e9
    assert abs(gb - g["full_cache_gb"]) / g["full_cache_gb"] < g["rel_tol"]


def test_score_state_size():
    g = _g("score_state_size.json")
    one = M.score_state_bytes(g["tokens"], 1, g["score_bytes"]) / 1e6
    many = M.score_state_bytes(g["tokens"], g["batch"], g["score_bytes"]) / 1e6
    assert abs(one - g["single_mb"]) / g["single_mb"] < g["rel_tol"]
    assert abs(many - g["batch_mb"]) / g["batch_mb"] < g["rel_tol"]


def test_step_bytes_model():
    # one unit, bf16 D=128: 512 B of K+V per retained slot plus 8 B fp32 score RMW
    b1 = M.unit_step_bytes(1000, head_dim=128, kv_elem=2, group=1, score_bytes=4)
    b2 = M.unit_step_bytes(1001, head_dim=128, kv_elem=2, group=1, score_bytes=4)
    assert b2 - b1 == 512 + 8
    # fp32 D=64 rows are also 256 B; G=8 query heads add 2 * 8 * D * 4
    assert M.unit_step_bytes(10, head_dim=64, kv_elem=4, group=8, score_bytes=8) == \
        9 * 512 + 4 * 256 + 10 * 16 + 2 * 8 * 64 * 4
    tot = M.launch_bytes(np.array([10, 20]), n_kv_heads=3, head_dim=128, kv_elem=2, group=1,
                         score_bytes=4)
    assert tot == 3 * int(M.unit_step_bytes(10, head_dim=128, kv_elem=2, group=1, score_bytes=4)
                          + M.unit_step_bytes(20, head_dim=128, kv_elem=2, group=1, score_bytes=4))


@pytest.mark.parametrize("kw,lens,steps", [
    (dict(), [300, 517, 1100], 80),
    (dict(n_sink=0, budget_fixed=64, hh_fixed=0), [100, 333], 120),
    (dict(n_sink=20, budget_fixed=96, hh_fixed=76), [90, 260], 120),
    (dict(budget_fixed=200, hh_fixed=100), [40, 700], 150),
])
def test_block_count_mirror_matches_oracle(kw, lens, steps):
    """The host's count mirror under block eviction (which the library's page
    accounting shares: the number of candidate pages from the schedule alone)
    against oracle runs that choose pages from real scores."""
    import oracle as O
    from kv_cache_eviction_h2o_amd import synth as S
    w = WL.PAGED_BLOCK.scaled(batch=len(lens), n_q_heads=2, n_kv_heads=2, head_dim=64,
                              kv_dtype="f32", recipe=S.Recipe(seed=5, head_dim=64, kv_dtype="f32"), **kw)
    K, V = S.prompt_kv(w.recipe, 0, lens, 2)
    off = np.concatenate([[0], np.cumsum(lens)])
    cfg = O.cfg_from_workload(w)
    q, k, v = S.step_window(w.recipe, 0, lens, steps, 2, 2)
    for b, P in enumerate(lens):
        us = [O.Unit(cfg, b, h, K[off[b]:off[b + 1], h], V[off[b]:off[b + 1], h], P + steps + 1)
              for h in range(2)]
        mirror = M.retained_counts(w, P, steps)
        for s in range(steps):
            for h, u in enumerate(us):
                u.attend(q[s, b, h:h + 1], k[s, b, h], v[s, b, h])
            vic = O.block_select(us, page=16)
            assert len(vic) == 16 * mirror["pages"][s], f"seq {b} step {s}"
            for u in us:
                u.evict(vic)
            assert len(us[0].state()[0]) == mirror["count"][s], f"seq {b} step {s}"
