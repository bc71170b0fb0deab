"""GPU parity of h2o_snapkv_select (through the C ABI) against the oracle.

Votes (window rows' weights, per query head) are floating point: every element
|gpu - oracle| <= 2e-3 * oracle + 1e-9, and each head's votes add up to the
window length.  The selection from the votes is index work: the kept sets must
equal, bit for bit, the oracle's selection (orc_snapkv_select) applied to the
GPU's own votes, so that a near-tie in the votes cannot hide a selection bug.
"""
import numpy as np
import pytest

import oracle as O
from kv_cache_eviction_h2o_amd import synth as S
from kv_cache_eviction_h2o_amd import workloads as WL

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_eviction_h2o_amd import _lib
    _lib.load_library()


def run_snapkv(w, lens, window, pool, keep, vote_units=None, zero_q=False):
    import torch
    from kv_cache_eviction_h2o_amd import _lib as L
    print(f"[snapkv] {w.name} B={len(lens)} Hq={w.n_q_heads} Hkv={w.n_kv_heads} lens={lens[:6]} "
          f"window={window} pool={pool} keep={keep}{' zero q' if zero_q else ''}", flush=True)
    K, _ = S.prompt_kv(w.recipe, 0, lens, w.n_kv_heads)
    Q = S.prompt_queries(w.recipe, 0, lens, w.n_q_heads)
    if zero_q:
        Q = np.zeros_like(Q)
    cfg = L.config_from_workload(w.scaled(batch=len(lens)), max_len=max(lens) + 1)
    kd = torch.from_numpy(np.ascontiguousarray(K).view(np.int16)).view(torch.bfloat16).cuda()
    kept, count, votes = L.snapkv_select(cfg, lens, torch.from_numpy(Q).cuda(), kd, window, pool, keep)
    kept, count, votes = kept.cpu().numpy(), count.cpu().numpy(), votes.cpu().numpy()
    G, Hkv = w.group, w.n_kv_heads
    ocfg = O.make_cfg(head_dim=w.head_dim, group=G)
    off = np.concatenate([[0], np.cumsum(lens)])
    for b, P in enumerate(lens):
        wb = min(window, P)
        for h in range(Hkv):
            v = votes[off[b]:off[b + 1], h * G:(h + 1) * G].T  # [G][P]
            assert np.allclose(v.sum(axis=1), wb, rtol=1e-4, atol=0)
            want = O.snapkv_select(v, wb, pool, keep)
            n = int(count[b, h])
            assert n == len(want), (b, h, n, len(want))
            assert np.array_equal(kept[b, h, :n], want), (b, h)
            assert np.all(kept[b, h, n:] == -1)
    units = [(b, h) for b in range(len(lens)) for h in range(Hkv)] if vote_units is None else vote_units
    for b, h in units:
        P = lens[b]
        q = Q[off[b]:off[b + 1], h * G:(h + 1) * G].astype(np.float64)
        k = S.cache_to_f64(w.recipe, K[off[b]:off[b + 1], h])
        ref = O.colsum(ocfg, q, k, row_lo=P - min(window, P), per_head=True)
        got = votes[off[b]:off[b + 1], h * G:(h + 1) * G].T
        err = np.abs(got - ref)
        assert np.all(err <= TOL * ref + 1e-9), (b, h, float(err.max()))
    return kept, count


def test_snapkv_opt_layer_reduced():
    w = WL.OPT_LAYER.scaled(n_q_heads=4, n_kv_heads=4)
    kept, count = run_snapkv(w, [300, 517], window=32, pool=7, keep=64)
    assert np.all(count == 32 + 64)


@pytest.mark.parametrize("g", [2, 8])
def test_snapkv_gqa_union(g):
    w = WL.LLAMA_GQA.scaled(n_q_heads=2 * g, n_kv_heads=2)
    kept, count = run_snapkv(w, [700, 250], window=32, pool=7, keep=40)
    assert np.all(count >= 32 + 40) and np.all(count <= 32 + g * 40)


def test_snapkv_edge_cases():
    w = WL.OPT_LAYER.scaled(n_q_heads=2, n_kv_heads=2)
    # prompt no longer than the window, keep beyond the prefix, keep 0, pool 1
    _, c = run_snapkv(w, [20, 32, 33, 100], window=32, pool=7, keep=200)
    assert list(c[:, 0]) == [20, 32, 33, 100]
    _, c = run_snapkv(w, [50, 90], window=16, pool=1, keep=0)
    assert np.all(c == 16)


def test_snapkv_opt_layer_full_shape():
    w = WL.OPT_LAYER
    run_snapkv(w, WL.prompt_lengths(w), window=32, pool=7, keep=172, vote_units=[(0, 0), (5, 13), (7, 31)])


def test_snapkv_gqa_layer_full_shape():
    """The LLaMA-2-70B layer's prompts as the benchmark selects them (16 x 1024,
    8 KV heads, groups of 8, window 32, pool 7, 20 % kept per head): every
    unit's kept set against the oracle's selection of the GPU's votes, and the
    votes of three sampled units against the oracle's column sums."""
    w = WL.LLAMA_GQA
    lens = WL.prompt_lengths(w)
    keep = max(1, min(lens) // 5)
    run_snapkv(w, lens, window=32, pool=7, keep=keep, vote_units=[(0, 0), (9, 3), (15, 7)])


def test_snapkv_gqa_edge_cases():
    """G = 4 (each query head selected in its own workgroup, then the union):
    prompts no longer than the window, keep beyond the prefix, keep 0, pool 1."""
    w = WL.LLAMA_GQA.scaled(n_q_heads=8, n_kv_heads=2)
    _, c = run_snapkv(w, [20, 32, 33, 100], window=32, pool=7, keep=200)
    assert list(c[:, 0]) == [20, 32, 33, 100]
    _, c = run_snapkv(w, [50, 90], window=16, pool=1, keep=0)
    assert np.all(c == 16)


def test_snapkv_one_pass_bounds():
    """Prompts up to 1024 positions with windows up to 32 rows run in one pass
    (a workgroup of 8 waves of 128 keys per unit and query head): prompts at
    and around the wave and tile edges and a prompt of one position, windows
    of 32, 31 and 1 rows; then just past each bound (1025 positions, a 33-row
    window), where the two column-sum passes and the selection kernel run."""
    w = WL.OPT_LAYER.scaled(n_q_heads=2, n_kv_heads=2)
    run_snapkv(w, [1024, 1023, 897, 129, 128, 17, 1], window=32, pool=7, keep=100)
    run_snapkv(w, [1024, 513, 40], window=31, pool=5, keep=37)
    _, c = run_snapkv(w, [1024, 2], window=1, pool=3, keep=500)
    assert list(c[:, 0]) == [501, 2]
    run_snapkv(w, [1025, 1024], window=32, pool=7, keep=100)
    run_snapkv(w, [1024, 600], window=33, pool=7, keep=100)
    # selection boundaries: one prefix position dropped (P = 100: prefix 68,
    # keep 67), none (keep = the prefix), and a prefix shorter than keep
    _, c = run_snapkv(w, [100, 64], window=32, pool=3, keep=67)
    assert list(c[:, 0]) == [99, 64]
    _, c = run_snapkv(w, [100, 1024], window=32, pool=3, keep=68)
    assert list(c[:, 0]) == [100, 100]
    # the most sequences a call takes (128), ragged, one KV head each
    w1 = WL.OPT_LAYER.scaled(n_q_heads=1, n_kv_heads=1)
    lens = [33 + (37 * b) % 200 for b in range(128)]
    run_snapkv(w1, lens, window=32, pool=5, keep=20)


@pytest.mark.parametrize("g", [2, 8])
def test_snapkv_one_pass_groups(g):
    """Groups of query heads in one pass (a workgroup per unit and head, each
    head's bits OR-ed by the union kernel): 3 KV heads, so 9 units leave the
    last group of 8 units partial; ragged prompts at the bounds."""
    w = WL.LLAMA_GQA.scaled(n_q_heads=3 * g, n_kv_heads=3)
    _, c = run_snapkv(w, [1024, 600, 33], window=32, pool=7, keep=60)
    assert np.all(c >= 32 + 1) and np.all(c <= 32 + g * 60)
    run_snapkv(w, [1023, 129, 1], window=31, pool=5, keep=40)


@pytest.mark.parametrize("g,lens", [(1, [1024, 300]), (2, [700, 65]), (1, [1500, 40])])
def test_snapkv_all_votes_tied(g, lens):
    """Zero queries: every logit is 0, so every prefix position gets the same
    vote (each window row spreads its weight evenly over its keys) and the
    selection must keep the lowest positions, through every vote digit to the
    position digits.  The one-pass path (prompts up to 1024) and the two-pass
    path (1500)."""
    w = WL.LLAMA_GQA.scaled(n_q_heads=2 * g, n_kv_heads=2)
    keep = 50
    kept, count = run_snapkv(w, lens, window=32, pool=5, keep=keep, zero_q=True)
    for b, P in enumerate(lens):
        wb = min(32, P)
        want = list(range(min(keep, P - wb))) + list(range(P - wb, P))
        for h in range(2):
            assert list(kept[b, h, :count[b, h]]) == want, (b, h)


@pytest.mark.parametrize("g", [1, 4])
def test_snapkv_long_prefix_unstaged(g):
    """A prefix beyond the 4096 positions whose pooled votes the selection
    stages in LDS (its radix passes then read global memory), beside a short
    one that is staged."""
    w = WL.LLAMA_GQA.scaled(n_q_heads=2 * g, n_kv_heads=2)
    run_snapkv(w, [5000, 700], window=32, pool=7, keep=900)


@pytest.mark.parametrize("g", [1, 2])
def test_snapkv_prompt_beyond_48k_of_lds(g):
    """A 140,000-position prompt: the selection's bitmap and vote staging
    exceed 48 KB of LDS, so the kernel's dynamic LDS limit is raised first."""
    w = WL.LLAMA_GQA.scaled(n_q_heads=g, n_kv_heads=1)
    run_snapkv(w, [140000], window=32, pool=7, keep=28000)
