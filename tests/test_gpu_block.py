"""GPU parity of block-granular eviction (paged layout, whole 16-token pages)
against the fp64 oracle; see parity.run_block_parity for the acceptance rule.
Reduced shapes run the whole trace on every sequence; the full benchmark shape
runs in the benchmark's launch configuration with sampled sequences checked
against the oracle and every sequence checked for the properties that hold at
any size (parity.block_properties)."""
import numpy as np
import pytest

from kv_cache_eviction_h2o_amd import workloads as WL

pytestmark = pytest.mark.gpu

PB = WL.PAGED_BLOCK


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_eviction_h2o_amd import _lib
    _lib.load_library()


def P():
    import parity
    return parity


def _run(w, steps, lens, **kw):
    rep = P().run_block_parity(w, steps, lens=lens, **kw)
    P().block_properties(w, rep.cache, lens, steps)
    rep.cache.close()
    return rep


def test_block_paged_reduced_unfused():
    w = PB.scaled(batch=3, n_q_heads=4, n_kv_heads=4)
    rep = _run(w, 60, [300, 517, 1100], fused=False)
    assert rep.evictions > 0


def test_block_paged_reduced_fused():
    w = PB.scaled(batch=4, n_q_heads=4, n_kv_heads=4)
    rep = _run(w, 60, [64, 300, 517, 1100])
    assert rep.evictions > 0


def test_block_fused_equals_unfused():
    """h2o_step_compact and h2o_step + h2o_compact leave bit-identical state."""
    import torch
    p = P()
    w = PB.scaled(batch=3, n_q_heads=8, n_kv_heads=4)
    lens = [200, 700, 1500]
    steps = 50
    res = []
    for fused in (True, False):
        cache, _, _ = p.make_cache(w, lens, steps)
        q, k, v = p.S.step_window(w.recipe, 0, lens, steps, w.n_q_heads, w.n_kv_heads)
        qd = torch.from_numpy(q).cuda()
        kd, vd = p.to_dev(k, "bf16"), p.to_dev(v, "bf16")
        out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
        outs = []
        for i in range(steps):
            if fused:
                cache.step_compact(qd[i], kd[i], vd[i], out)
            else:
                cache.step(qd[i], kd[i], vd[i], out)
                cache.compact()
            outs.append(out.cpu().numpy().copy())
        res.append((cache.read_indices(), np.stack(outs), cache.info()))
        cache.close()
    (a, oa, ia), (b, ob, ib) = res
    assert ia == ib
    assert np.array_equal(oa, ob)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_block_gqa_group_of_eight_f64_fixed_budget():
    # the 4 + 512 + 512 cache manager with whole pages: prompt above the budget
    w = WL.LLAMA_GQA.scaled(name="llama2_70b_gqa_block", batch=2, prompt_len=1100, page_size=16,
                            selector="block")
    rep = _run(w, 40, [1100, 1100], fused=False)
    assert rep.evictions > 0


def test_block_no_sinks_no_heavy_hitters():
    # HH = 0: no token is important, so the oldest candidate pages go -- a
    # sliding window at page granularity
    w = PB.scaled(batch=2, n_q_heads=2, n_kv_heads=2, n_sink=0, budget_fixed=64, hh_fixed=0)
    rep = _run(w, 100, [100, 333], fused=False)
    assert rep.evictions > 0


def test_block_sinks_over_two_pages_and_zero_window():
    # 20 sinks hold two pages; W = 0 makes the newest full page a candidate
    w = PB.scaled(batch=2, n_q_heads=4, n_kv_heads=2, n_sink=20, budget_fixed=96, hh_fixed=76)
    rep = _run(w, 100, [90, 260], fused=False)
    assert rep.evictions > 0


def test_block_budget_above_length():
    w = PB.scaled(batch=2, n_q_heads=2, n_kv_heads=2, budget_fixed=4096, hh_fixed=2000)
    rep = _run(w, 40, [100, 333])
    assert rep.evictions == 0


def test_block_int8_rows():
    w = PB.scaled(name="paged_block_int8", batch=2, n_q_heads=4, n_kv_heads=4, kv_dtype="i8")
    rep = _run(w, 50, [300, 900], fused=False)
    assert rep.evictions > 0


def test_block_long_trace():
    # 2000 fused steps: pages evicted, pushed on the free stack and popped again
    rep = _run(PB.scaled(batch=3, n_q_heads=4, n_kv_heads=4), 2000, [700, 1500, 3000])
    assert rep.evictions > 0


def test_block_full_shape_sampled_sequences():
    """The benchmark's shape and launch configuration (64 sequences of 4k-64k
    prompts, 32 heads, fused entry point, device-drawn inputs): the two
    shortest sequences against the oracle at every step, then every sequence
    for the properties."""
    w = PB
    lens = WL.prompt_lengths(w)
    seqs = [int(x) for x in np.argsort(lens)[:2]]
    steps = 24
    rep = P().run_block_parity(w, steps, lens=lens, seqs=seqs, device_inputs=True, stored_rows=False,
                               read_every=4)
    from kv_cache_eviction_h2o_amd import metrics as M
    cap = int(max(M.retained_counts(w, p, steps)["count"].max() for p in lens))
    P().block_properties(w, rep.cache, lens, steps, cap=cap)
    rep.cache.close()
    assert rep.evictions > 0


def test_block_moving_sum_scores():
    """Block eviction ranks pages by heavy hitters of moving-sum scores (decay
    0.99 per step, fp32 and fp64): the same rule on the decayed scores."""
    for sd in ("f32", "f64"):
        w = PB.scaled(batch=3, n_q_heads=4, n_kv_heads=4, score_dtype=sd, score_decay=0.99)
        rep = _run(w, 60, [300, 517, 1100], fused=(sd == "f32"))
        assert rep.evictions > 0
