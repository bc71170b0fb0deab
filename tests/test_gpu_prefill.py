"""GPU parity of h2o_prefill_scores (through the C ABI) against the oracle's
causal-attention column sums (orc_colsum, rows from 0, summed over the group).

Acceptance: every element |gpu - oracle| <= 2e-3 * oracle + 1e-9 (the
tolerance of the decode step's scores); the column sums of each (sequence, KV
head) add up to G * P_b.
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


def run_prefill(w, lens, units=None, layer=0):
    import torch
    from kv_cache_eviction_h2o_amd import _lib as L
    print(f"[prefill] {w.name} B={len(lens)} Hq={w.n_q_heads} Hkv={w.n_kv_heads} lens={lens[:6]} "
          f"units={'all' if units is None else len(units)}", flush=True)
    K, _ = S.prompt_kv(w.recipe, layer, lens, w.n_kv_heads)
    Q = S.prompt_queries(w.recipe, layer, lens, w.n_q_heads)
    cfg = L.config_from_workload(w.scaled(batch=len(lens)), max_len=max(lens) + 1)
    kd = torch.from_numpy(np.ascontiguousarray(K).view(np.int16)).view(torch.bfloat16).cuda()
    qd = torch.from_numpy(Q).cuda()
    got = L.prefill_scores(cfg, lens, qd, kd).cpu().numpy()
    G, Hkv = w.group, w.n_kv_heads
    ocfg = O.make_cfg(head_dim=w.head_dim, group=G)
    off = np.concatenate([[0], np.cumsum(lens)])
    units = [(b, h) for b in range(len(lens)) for h in range(Hkv)] if units is None else units
    worst = 0.0
    for b, h in units:
        q = Q[off[b]:off[b + 1], h * G:(h + 1) * G].astype(np.float64)
        k = S.cache_to_f64(w.recipe, K[off[b]:off[b + 1], h])
        want = O.colsum(ocfg, q, k)
        g = got[off[b]:off[b + 1], h]
        err = np.abs(g - want)
        assert np.all(err <= TOL * want + 1e-9), (b, h, int(np.argmax(err - TOL * want)), float(err.max()))
        assert abs(g.sum() - G * lens[b]) <= 1e-4 * G * lens[b]
        worst = max(worst, float((err / np.maximum(want, 1e-30)).max()))
    print(f"[prefill] max relative error {worst:.2e}", flush=True)
    return got


def test_prefill_scores_opt_layer_reduced():
    w = WL.OPT_LAYER.scaled(n_q_heads=4, n_kv_heads=4)
    run_prefill(w, [300, 517])


@pytest.mark.parametrize("g", [2, 4, 8])
def test_prefill_scores_gqa_groups(g):
    w = WL.LLAMA_GQA.scaled(n_q_heads=2 * g, n_kv_heads=2)
    run_prefill(w, [700, 129])


@pytest.mark.parametrize("g", [1, 8])
def test_prefill_scores_ragged_short_prompts(g):
    # one position, fewer than one 8-row tile, exact tiles, one past a 64-key
    # block; prompts of at most 128 positions take the rows pass's window
    # tiling (one tile per wave; G = 8: four workgroups of two query heads)
    w = WL.OPT_LAYER.scaled(n_q_heads=2 * g, n_kv_heads=2)
    run_prefill(w, [1, 7, 8, 16, 33, 64, 65])


def test_prefill_scores_opt_layer_full_shape_sampled():
    w = WL.OPT_LAYER
    run_prefill(w, WL.prompt_lengths(w), units=[(0, 0), (3, 17), (7, 31)])


def test_prefill_scores_gqa_layer_full_shape_sampled():
    """The LLaMA-2-70B layer's prompts as the benchmark scores them (16 x 1024,
    8 KV heads, groups of 8: the rows pass runs each group as two workgroups
    of 4 heads), three units against the oracle element by element."""
    w = WL.LLAMA_GQA
    run_prefill(w, WL.prompt_lengths(w), units=[(0, 0), (9, 3), (15, 7)])


def test_prefill_scores_then_decode_parity():
    # the GPU's prefill scores seed both sides of a decode parity run
    import parity
    import torch
    from kv_cache_eviction_h2o_amd import _lib as L
    w = WL.OPT_LAYER.scaled(batch=2, n_q_heads=4, n_kv_heads=4)
    lens = [400, 333]
    K, _ = S.prompt_kv(w.recipe, 0, lens, w.n_kv_heads)
    Q = S.prompt_queries(w.recipe, 0, lens, w.n_q_heads)
    cfg = L.config_from_workload(w, max_len=max(lens) + 1)
    kd = torch.from_numpy(np.ascontiguousarray(K).view(np.int16)).view(torch.bfloat16).cuda()
    init = L.prefill_scores(cfg, lens, torch.from_numpy(Q).cuda(), kd).cpu().numpy()
    rep = parity.run_parity(w, 40, lens=lens, init_scores=init)
    assert rep.evictions > 0
