"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every ``pin_*`` takes a loaded oracle library and raises AssertionError (or the
oracle's own OracleError) when the oracle disagrees with the pin.  They are run
on the real oracle by test_oracle_pins.py and on deliberately broken copies of
it by test_oracle_mutants.py, which checks that each planted mistake is caught.

Independent references used here: torch's scaled_dot_product_attention and
softmax (fp64, CPU), torch.topk, numpy.lexsort, numpy.random.Philox, brute
force over subsets, closed forms the pages state (StreamingLLM's sinks + window,
the sliding window, full attention when nothing is evicted), and fixtures under
tests/golden/.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
M64 = 1 << 64


def _unit(lib, cfg, pk, pv, cap, b=0, h=0, init=None):
    return O.Unit(cfg, b, h, pk, pv, cap, init_scores=init, lib=lib)


def _sdpa(q, Kr, Vr, scale=None):
    """torch fp64 attention of G queries over one shared K/V: q [G][D], Kr/Vr [n][D]."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, :, None, :]
    G = qt.shape[1]
    kt = torch.from_numpy(np.asarray(Kr, np.float64))[None, None].expand(1, G, -1, -1)
    vt = torch.from_numpy(np.asarray(Vr, np.float64))[None, None].expand(1, G, -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[0, :, 0, :].numpy()


def _softmax_rows(q, Kr, scale):
    s = torch.from_numpy(np.asarray(q, np.float64)) @ torch.from_numpy(np.asarray(Kr, np.float64)).T
    return torch.softmax(s * scale, dim=-1).numpy()


def _philox_np(ctr, key):
    """numpy's Philox4x64-10 block at counter ctr (numpy bumps its counter first)."""
    c0, c1, c2, c3 = (int(x) for x in ctr)
    v = (c0 + c1 * M64 + c2 * M64 ** 2 + c3 * M64 ** 3 - 1) % M64 ** 4
    c = np.array([(v >> (64 * i)) % M64 for i in range(4)], dtype=np.uint64)
    g = np.random.Philox(key=np.array([k % M64 for k in key], dtype=np.uint64), counter=c)
    return [int(x) for x in g.random_raw(4)]


# ---------------------------------------------------------------- attention
def pin_attention_full_cache(lib):
    """Budget >= length: nothing is evicted and every step is plain decode
    attention over all positions (torch SDPA), its weights are torch softmax
    rows, and each position's score is the sum of its weights over steps and
    query heads."""
    rng = np.random.default_rng(11)
    D, G, P, steps = 16, 3, 9, 12
    for scale in (0.0, 0.3):
        cfg = O.make_cfg(head_dim=D, group=G, scale=scale, n_sink=4, budget_fixed=1000,
                         hh_fixed=992)
        pk, pv = rng.standard_normal((P, D)), rng.standard_normal((P, D))
        u = _unit(lib, cfg, pk, pv, P + steps)
        Kall, Vall = [*pk], [*pv]
        acc = np.zeros(P + steps)
        sc = scale if scale else 1.0 / np.sqrt(D)
        for s in range(steps):
            q = rng.standard_normal((G, D))
            k, v = rng.standard_normal(D), rng.standard_normal(D)
            Kall.append(k)
            Vall.append(v)
            out, probs = u.attend(q, k, v, want_probs=True)
            ref = _sdpa(q, np.array(Kall), np.array(Vall), scale=scale if scale else None)
            assert np.max(np.abs(out - ref)) < 1e-12, "attention output != torch SDPA"
            rows = _softmax_rows(q, np.array(Kall), sc)
            assert np.max(np.abs(probs - rows)) < 1e-14, "weights != torch softmax"
            assert np.max(np.abs(probs.sum(axis=1) - 1.0)) < 1e-12
            acc[:len(Kall)] += rows.sum(axis=0)
            vic, _ = u.select()
            assert len(vic) == 0, "evicted although budget >= length"
            u.evict(vic)
            u.check()
        pos, scores, em = u.state()
        assert list(pos) == list(range(P + steps)), "full cache lost a position"
        assert np.max(np.abs(scores - acc)) < 1e-12, "scores != summed softmax weights"
        assert em == 0.0


# ------------------------------------------------- scores + selection, H2O
def _budget_20pct(length, n_sink=4):
    K = length // 5
    HH = (K - n_sink) // 2
    return K, HH, K - n_sink - HH


def pin_scores_and_selection_recomputed(lib):
    """20 % budget over a ragged trace: the test keeps its own scores (torch
    softmax over the retained set, summed over the group's query heads) and its
    own selection (numpy.lexsort: score ascending, then position descending,
    over the candidates outside sinks and recent window).  The oracle must
    agree on the retained set, every score and the evicted mass, and the mass
    must add up to G * steps.  Then the same with a moving sum (decay 0.85:
    every retained score is multiplied by the decay once per step before the
    step's weights are added)."""
    _recomputed(lib, 1.0)
    _recomputed(lib, 0.85)


def _recomputed(lib, lam):
    rng = np.random.default_rng(12)
    D, G, P, steps = 8, 2, 57, 41
    cfg = O.make_cfg(head_dim=D, group=G, n_sink=4, budget_num=1, budget_den=5, decay=lam)
    pk, pv = rng.standard_normal((P, D)), rng.standard_normal((P, D))
    pk[3] += 2.5  # a heavy direction on a few keys
    u = _unit(lib, cfg, pk, pv, P + steps)
    Kall, live = [*pk], set(range(P))
    score = {p: 0.0 for p in range(P)}
    evicted = 0.0
    scale = 1.0 / np.sqrt(D)
    for s in range(steps):
        t = P + s
        q = rng.standard_normal((G, D)) + 0.5
        k, v = rng.standard_normal(D), rng.standard_normal(D)
        Kall.append(k)
        live.add(t)
        score[t] = 0.0
        R = sorted(live)
        rows = _softmax_rows(q, np.array([Kall[p] for p in R]), scale)
        for i, p in enumerate(R):
            score[p] = lam * score[p] + rows[:, i].sum()
        out = u.attend(q, k, v)
        length = t + 1
        K, HH, W = _budget_20pct(length)
        e = len(R) - K
        vic_ref = []
        if e > 0:
            cands = [p for p in R if 4 <= p < length - W]
            order = np.lexsort((-np.array(cands), np.array([score[p] for p in cands])))
            vic_ref = [cands[i] for i in order[:e]]
        vic, _ = u.select()
        assert sorted(vic) == sorted(vic_ref), f"step {s}: victims differ"
        u.evict(vic)
        u.check()
        for p in vic_ref:
            live.discard(p)
            evicted += score[p]
        pos, sc, em = u.state()
        assert list(pos) == sorted(live)
        assert np.max(np.abs(sc - np.array([score[p] for p in pos]))) < 1e-12
        assert abs(em - evicted) < 1e-12
        if lam == 1.0:
            assert abs(sc.sum() + em - G * (s + 1)) < 1e-9, "retained + evicted mass != G*steps"
        assert len(pos) <= K


def pin_streaming_llm_and_sliding_window(lib):
    """No heavy hitters: 4 sinks + the last W positions (StreamingLLM, the
    attention-sinks page sec. 4.1); no sinks either: the last W only (sliding
    window, sec. 2.1).  Closed forms, whatever the values."""
    rng = np.random.default_rng(13)
    D, P, steps = 6, 30, 25
    for n_sink, W in ((4, 8), (0, 10)):
        cfg = O.make_cfg(head_dim=D, n_sink=n_sink, budget_fixed=n_sink + W, hh_fixed=0)
        u = _unit(lib, cfg, rng.standard_normal((P, D)), rng.standard_normal((P, D)), P + steps)
        for s in range(steps):
            u.step(rng.standard_normal((1, D)), rng.standard_normal(D), rng.standard_normal(D))
            length = P + s + 1
            pos, _, _ = u.state()
            expect = list(range(n_sink)) + list(range(length - W, length))
            assert list(pos) == expect, f"sinks={n_sink} W={W} step {s}"


def pin_greedy_equals_bruteforce(lib):
    """H2O's greedy step (the H2O summary page): with an additive set score,
    the evicted set must be the one that leaves the largest retained score.
    Brute force over every e-subset of the candidates, on tiny inputs."""
    rng = np.random.default_rng(14)
    D, P, steps = 4, 12, 10
    cfg = O.make_cfg(head_dim=D, n_sink=1, budget_fixed=8, hh_fixed=3)
    u = _unit(lib, cfg, rng.standard_normal((P, D)), rng.standard_normal((P, D)), P + steps)
    for s in range(steps):
        u.attend(rng.standard_normal((1, D)) * 1.5, rng.standard_normal(D), rng.standard_normal(D))
        length = P + s + 1
        pos, sc, _ = u.state()
        W = 8 - 1 - 3
        cands = [(p, x) for p, x in zip(pos, sc) if 1 <= p < length - W]
        e = len(pos) - 8
        best, best_kept = None, -np.inf
        for sub in itertools.combinations(range(len(cands)), max(e, 0)):
            kept = sum(x for i, (_, x) in enumerate(cands) if i not in sub)
            if kept > best_kept:
                best, best_kept = sub, kept
        vic, _ = u.select()
        assert sorted(vic) == sorted(cands[i][0] for i in best), f"step {s}"
        u.evict(vic)


def pin_topk_middle_region(lib):
    """The cache-manager listing of the StreamingLLM-vs-H2O article: keep the
    first n_sink rows, the last n_recent rows and torch.topk(middle scores,
    n_heavy) of the rows in between.  At a bulk eviction from a full prompt
    the oracle must keep exactly that set."""
    rng = np.random.default_rng(15)
    D, P = 8, 40
    cfg = O.make_cfg(head_dim=D, n_sink=4, budget_fixed=15, hh_fixed=6)
    u = _unit(lib, cfg, rng.standard_normal((P, D)), rng.standard_normal((P, D)), P + 4,
              init=rng.random(P))
    u.attend(rng.standard_normal((1, D)), rng.standard_normal(D), rng.standard_normal(D))
    pos, sc, _ = u.state()
    length = P + 1
    mid = torch.from_numpy(sc[4:length - 5])
    hh = (torch.topk(mid, 6).indices + 4).tolist()
    expect = sorted(list(range(4)) + hh + list(range(length - 5, length)))
    vic, _ = u.select()
    u.evict(vic)
    pos, _, _ = u.state()
    assert list(pos) == expect


def pin_tie_break_lower_position_kept(lib):
    """Equal scores: the lower position is retained (ties resolved by
    numpy.lexsort on (score, -position)).  Identical keys give every token the
    same weight, so all candidates tie."""
    D, P = 4, 20
    key = np.array([0.5, -1.0, 0.25, 2.0])
    pk = np.tile(key, (P, 1))
    pv = np.arange(P * D, dtype=np.float64).reshape(P, D)
    cfg = O.make_cfg(head_dim=D, n_sink=2, budget_fixed=8, hh_fixed=3)
    u = _unit(lib, cfg, pk, pv, P + 2)
    u.attend(np.ones((1, D)), key, np.zeros(D))
    pos, sc, _ = u.state()
    assert np.all(sc == sc[0])
    length = P + 1
    cands = np.array([p for p in pos if 2 <= p < length - 3])
    order = np.lexsort((-cands, sc[cands]))
    e = len(pos) - 8
    vic, _ = u.select()
    assert sorted(vic) == sorted(cands[order[:e]].tolist())
    u.evict(vic)
    pos, _, _ = u.state()
    assert list(pos) == [0, 1, 2, 3, 4, 18, 19, 20]


# ------------------------------------------------------------ Random selector
def pin_philox_matches_numpy(lib):
    """The oracle's own Philox4x64-10 against numpy.random.Philox."""
    for key in ([5, 0], [0xC4, 0], [2 ** 63 + 7, 99]):
        for ctr in ([0, 0, 0, 0], [3, 7, 4223, 2050], [2 ** 64 - 1, 5, 6, 7], [31, 7, 32767, 32766]):
            assert O.philox4x64_10(ctr, key, lib=lib) == _philox_np(ctr, key)


def pin_random_victims_are_smallest_philox_words(lib):
    """Random Attention: the prompt is kept; when the generated tokens reach
    K + r, the r evicted are those with the smallest Philox word 0 at counter
    (sequence, head, step, position), key (seed, 0) -- computed here with
    numpy's Philox -- ties to the higher position."""
    rng = np.random.default_rng(16)
    D, P, Kk, r, seed = 4, 5, 6, 3, 0xC4
    b, h = 3, 1
    cfg = O.make_cfg(head_dim=D, group=2, selector=O.ORC_RANDOM, rand_k=Kk, rand_r=r, seed=seed)
    u = _unit(lib, cfg, rng.standard_normal((P, D)), rng.standard_normal((P, D)), P + 40, b=b, h=h)
    events = 0
    for s in range(40):
        t = P + s
        u.attend(rng.standard_normal((2, D)), rng.standard_normal(D), rng.standard_normal(D))
        pos, _, _ = u.state()
        gen = [p for p in pos if p >= P]
        vic, _ = u.select()
        if len(gen) == Kk + r:
            words = np.array([_philox_np([b, h, t, p], [seed, 0])[0] for p in gen], dtype=np.uint64)
            order = np.lexsort((-np.array(gen), words))
            assert sorted(vic) == sorted(np.array(gen)[order[:r]].tolist())
            events += 1
        else:
            assert len(vic) == 0
        u.evict(vic)
        u.check()
        pos, _, _ = u.state()
        assert set(range(P)) <= set(pos), "prompt token evicted"
        assert len([p for p in pos if p >= P]) < Kk + r
    assert events == 11


def pin_random_uniform_and_independent(lib):
    """Per head, uniform: every one of the K + r candidates is evicted with
    probability r / (K + r); two heads of one sequence choose independently
    (expected overlap r^2 / (K + r))."""
    D, Kk, r = 2, 12, 4
    n_units = 1200
    counts = np.zeros(Kk + r)
    overlaps = []
    cfg = O.make_cfg(head_dim=D, selector=O.ORC_RANDOM, rand_k=Kk, rand_r=r, seed=77)
    z = np.zeros(D)
    for b in range(n_units // 2):
        sets = []
        for h in range(2):
            u = _unit(lib, cfg, np.zeros((1, D)), np.zeros((1, D)), Kk + r + 2, b=b, h=h)
            for s in range(Kk + r):
                u.attend(np.zeros((1, D)), z, z)
            vic, _ = u.select()
            assert len(vic) == r
            counts[np.asarray(vic) - 1] += 1
            sets.append(set(vic.tolist()))
        overlaps.append(len(sets[0] & sets[1]))
    p = r / (Kk + r)
    expect = n_units * p
    sd = np.sqrt(n_units * p * (1 - p))
    assert np.all(np.abs(counts - expect) < 5 * sd), counts
    chi2 = float(np.sum((counts - expect) ** 2 / (expect * (1 - p))))
    assert chi2 < 45.0, chi2  # 15 dof; p ~ 1e-4
    mean_overlap = np.mean(overlaps)
    hyper_sd = np.sqrt(r * p * (1 - p) * (Kk / (Kk + r - 1)) / len(overlaps))
    assert abs(mean_overlap - r * p) < 5 * hyper_sd, mean_overlap


# ------------------------------------------------------------- golden files
def pin_golden_streaming_layout(lib):
    """tests/golden/streaming_llm_layout.json: the sink + window layout the
    attention-sinks page draws in sec. 4.1."""
    with open(os.path.join(GOLDEN, "streaming_llm_layout.json")) as f:
        g = json.load(f)
    rng = np.random.default_rng(17)
    D, N, W, S = 4, g["length"], g["window"], g["n_sink"]
    P = N - 1
    cfg = O.make_cfg(head_dim=D, n_sink=S, budget_fixed=S + W, hh_fixed=0)
    u = _unit(lib, cfg, rng.standard_normal((P, D)), rng.standard_normal((P, D)), N)
    u.step(rng.standard_normal((1, D)), rng.standard_normal(D), rng.standard_normal(D))
    pos, _, _ = u.state()
    assert list(pos) == g["retained"]


def pin_golden_cache_manager_sizes(lib):
    """tests/golden/cache_manager_defaults.json: the StreamingLLM-vs-H2O
    article's manager (4 sinks, 512 heavy hitters, 512 recent) leaves the
    cache unchanged while the length is within 4 + 512 + 512, and past it
    keeps exactly 4 sink, 512 heavy-hitter and 512 recent rows."""
    with open(os.path.join(GOLDEN, "cache_manager_defaults.json")) as f:
        g = json.load(f)
    S, HH, R = g["num_sink_tokens"], g["num_heavy_hitters"], g["num_recent_tokens"]
    cap = g["max_capacity"]
    rng = np.random.default_rng(18)
    D = 2
    P = cap - 1
    cfg = O.make_cfg(head_dim=D, n_sink=S, budget_fixed=cap, hh_fixed=HH)
    u = _unit(lib, cfg, rng.standard_normal((P, D)), rng.standard_normal((P, D)), cap + 3)
    u.step(rng.standard_normal((1, D)), rng.standard_normal(D), rng.standard_normal(D))
    pos, _, _ = u.state()
    assert list(pos) == list(range(cap)), "evicted at length == capacity"
    for _ in range(2):
        u.step(rng.standard_normal((1, D)), rng.standard_normal(D), rng.standard_normal(D))
        length = u.length()
        pos, _, _ = u.state()
        assert len(pos) == cap
        sinks = [p for p in pos if p < S]
        recent = [p for p in pos if p >= length - R]
        heavy = [p for p in pos if S <= p < length - R]
        assert (len(sinks), len(heavy), len(recent)) == tuple(g["layout_sizes"])


def pin_colsum_identical_keys(lib):
    """Identical keys make every causal row uniform: row i gives 1/(i+1) to each
    j <= i, so column j collects H(P) - H(max(j, row_lo)) per query head (H the
    harmonic numbers); the total is G * (P - row_lo) (each row sums to one)."""
    D, G, P = 16, 3, 23
    cfg = O.make_cfg(head_dim=D, group=G)
    rng = np.random.default_rng(11)
    k = np.tile(rng.standard_normal(D), (P, 1))
    q = rng.standard_normal((P, G, D)) * 3.0
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, P + 1))])
    for row_lo in (0, 7):
        out = O.colsum(cfg, q, k, row_lo=row_lo, lib=lib)
        per = O.colsum(cfg, q, k, row_lo=row_lo, per_head=True, lib=lib)
        want = np.array([H[P] - H[max(j, row_lo)] for j in range(P)])
        assert np.allclose(out, G * want, rtol=0, atol=1e-12)
        assert np.allclose(per, np.tile(want, (G, 1)), rtol=0, atol=1e-12)
        assert abs(out.sum() - G * (P - row_lo)) < 1e-9


def pin_colsum_equals_decode_accumulation(lib):
    """Scoring the prompt's causal rows is the decode accumulation run over the
    prompt: a unit started from the first token and stepped over positions
    1..P-1 with a budget it never reaches holds, for every position j, the sum
    over rows i >= max(j, 1) of row i's weight on j -- column sums from row 1."""
    D, G, P = 32, 2, 40
    rng = np.random.default_rng(12)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    k = rng.standard_normal((P, D))
    k[[0, 5, 17, 30]] += 2.5 * u
    v = rng.standard_normal((P, D))
    q = rng.standard_normal((P, G, D)) + 1.5 * u
    dec = O.make_cfg(head_dim=D, group=G, budget_fixed=P + 8, hh_fixed=2)
    unit = _unit(lib, dec, k[:1], v[:1], P + 1)
    for t in range(1, P):
        unit.step(q[t], k[t], v[t])
    pos, sc, em = unit.state()
    assert list(pos) == list(range(P)) and em == 0.0
    want = O.colsum(O.make_cfg(head_dim=D, group=G), q, k, row_lo=1, lib=lib)
    assert np.allclose(sc, want, rtol=1e-12, atol=1e-14)
    per = O.colsum(O.make_cfg(head_dim=D, group=G), q, k, row_lo=1, per_head=True, lib=lib)
    assert np.allclose(per.sum(axis=0), want, rtol=1e-12, atol=1e-14)


def pin_snapkv_pooling_and_union(lib):
    """A vote spike at j0 pooled with kernel 7 covers [j0 - 3, j0 + 3] (clipped at the
    prefix ends); keep = 7 keeps exactly that range; two heads with spikes at
    different places keep the union of both ranges; the window is always kept."""
    P, w = 40, 6
    Pp = P - w
    window = list(range(Pp, P))
    v = np.zeros((1, P))
    v[0, 12] = 1.0
    assert list(O.snapkv_select(v, w, 7, 7, lib=lib)) == list(range(9, 16)) + window
    # clipped at position 0: pooled 1 on 0..3, then the zeros go lowest position first
    v = np.zeros((1, P))
    v[0, 0] = 0.5
    assert list(O.snapkv_select(v, w, 7, 6, lib=lib)) == list(range(0, 6)) + window
    # window votes never enter the pooling: a spike 6 before the window pools onto
    # Pp-9..Pp-3, and keep = 4 takes the lowest four of that range, not the last
    # prefix positions next to the window's large votes
    v = np.zeros((1, P))
    v[0, Pp - 6] = 2.0
    v[0, Pp:] = 9.0
    assert list(O.snapkv_select(v, w, 7, 4, lib=lib)) == list(range(Pp - 9, Pp - 5)) + window
    v = np.zeros((2, P))
    v[0, 5] = 1.0
    v[1, 25] = 1.0
    assert list(O.snapkv_select(v, w, 7, 7, lib=lib)) == list(range(2, 9)) + list(range(22, 29)) + window


def pin_snapkv_topk_matches_library(lib):
    """Random votes: pooled by scipy's maximum_filter1d (constant -inf border),
    top-k per head by numpy's stable sort of the negated pooled votes, union + window."""
    from scipy.ndimage import maximum_filter1d
    rng = np.random.default_rng(21)
    G, P, w, pool, keep = 3, 60, 10, 7, 9
    v = rng.random((G, P))
    Pp = P - w
    want = set(range(Pp, P))
    for g in range(G):
        pooled = maximum_filter1d(v[g, :Pp], size=pool, mode="constant", cval=-np.inf)
        want |= set(np.argsort(-pooled, kind="stable")[:keep].tolist())
    assert list(O.snapkv_select(v, w, pool, keep, lib=lib)) == sorted(want)
    # keep >= prefix: everything kept
    assert list(O.snapkv_select(v, w, pool, Pp + 3, lib=lib)) == list(range(P))


def pin_snapkv_ties_keep_lower_positions(lib):
    """Equal votes everywhere: each head keeps the `keep` lowest positions."""
    v = np.ones((2, 30))
    assert list(O.snapkv_select(v, 4, 5, 3, lib=lib)) == [0, 1, 2] + list(range(26, 30))


def pin_snapkv_votes_are_window_weights(lib):
    """The votes of orc_snapkv are the window rows' weights: per head they add up
    to w (each row sums to one) and equal orc_colsum from row P - w."""
    D, G, P, w = 16, 2, 50, 8
    rng = np.random.default_rng(22)
    q = rng.standard_normal((P, G, D)) * 2.0
    k = rng.standard_normal((P, D))
    cfg = O.make_cfg(head_dim=D, group=G)
    kept, votes = O.snapkv(cfg, q, k, w, 7, 5, lib=lib)
    assert np.allclose(votes.sum(axis=1), w, rtol=0, atol=1e-10)
    assert np.allclose(votes, O.colsum(cfg, q, k, row_lo=P - w, per_head=True, lib=lib), rtol=0, atol=0)
    assert list(kept) == list(O.snapkv_select(votes, w, 7, 5, lib=lib))


def pin_int8_rows(lib):
    """Int8 row quantisation (oracle.quantize_rows): the bounds and special cases
    the definition fixes -- scale = max|x| / 127; the largest element maps to
    +-127; every element is reproduced within half a scale step; signs and zeros
    are kept; a zero row has scale 0; scaling a row by a power of two scales the
    scale alone; a row already on the grid (integers up to 127 times a step) is
    stored exactly."""
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((64, 128)) * np.exp(rng.uniform(-4, 4, (64, 1)))).astype(np.float32)
    x[5] = 0.0
    x[6, :] = 0.0
    x[6, 17] = -3.5
    codes, scale = O.quantize_rows(x)
    a = np.max(np.abs(x), axis=1)
    assert np.array_equal(scale, (a / np.float32(127.0)).astype(np.float32))
    assert scale[5] == 0.0 and not codes[5].any()
    assert codes[6, 17] == -127 and np.count_nonzero(codes[6]) == 1
    big = np.argmax(np.abs(x), axis=1)
    nz = a > 0
    assert np.all(np.abs(codes[nz, big[nz]]) == 127)
    err = np.abs(O.dequantize_rows(codes, scale) - x.astype(np.float64))
    assert np.all(err <= 0.5 * scale[:, None].astype(np.float64) * (1 + 1e-6))
    assert np.all((codes > 0) <= (x > 0)) and np.all((codes < 0) <= (x < 0))
    c2, s2 = O.quantize_rows(x * np.float32(8.0))
    assert np.array_equal(c2, codes) and np.array_equal(s2, scale * np.float32(8.0))
    grid = rng.integers(-127, 128, (8, 128)).astype(np.float32)
    grid[:, 0] = 127.0
    cg, sg = O.quantize_rows(grid * np.float32(0.25))
    assert np.all(sg == np.float32(0.25)) and np.array_equal(cg.astype(np.float32), grid)


# --------------------------------------------------- block-granular eviction
def _block_expect(length, live, scores, n_sink, K, HH, page):
    """Brute force for one block-eviction decision: importance per block from
    each head's HH best candidate tokens (numpy.lexsort on (position, -score)),
    then the m-subset of candidate blocks with the least total importance,
    equal totals going to the lexicographically first (oldest) block list."""
    W = K - n_sink - HH
    n = int(np.count_nonzero(live))
    if n <= K:
        return []
    nb = (length + page - 1) // page
    cand = [k for k in range(nb)
            if (k + 1) * page <= length and all(live[k * page:(k + 1) * page])
            and k * page >= n_sink and (k + 1) * page - 1 < length - W]
    imp = {k: 0 for k in cand}
    toks = np.array([p for k in cand for p in range(k * page, (k + 1) * page)], dtype=np.int64)
    for sc in scores:
        if toks.size == 0:
            break
        order = np.lexsort((toks, -np.asarray(sc)[toks]))
        for p in toks[order[:max(0, min(HH, toks.size))]]:
            imp[int(p) // page] += 1
    m = min(len(cand), -(-(n - K) // page))
    best = min(itertools.combinations(cand, m), key=lambda sub: (sum(imp[k] for k in sub), sub))
    return [p for k in sorted(best) for p in range(k * page, (k + 1) * page)]


def pin_block_bruteforce(lib):
    """Block-granular eviction ("Attention Sinks and KV cache eviction",
    section 5: blocks with the lowest share of important tokens go first),
    against brute force over every m-subset of candidate blocks on tiny inputs:
    random retained sets (holes make a block ineligible), 1 to 3 heads, scores
    rounded to one decimal so that ties occur, pages of 2 and 3."""
    rng = np.random.default_rng(41)
    for trial in range(60):
        page = 2 + trial % 2
        length = int(rng.integers(12, 22))
        n_sink = int(rng.integers(0, 3))
        HH = int(rng.integers(0, 6))
        W = int(rng.integers(0, 5))
        K = n_sink + HH + W
        live = (rng.random(length) < 0.85).astype(np.uint8)
        live[:n_sink] = 1
        live[length - W:] = 1
        heads = int(rng.integers(1, 4))
        scores = np.round(rng.random((heads, length)), 1)
        cfg = O.make_cfg(head_dim=4, selector=O.ORC_BLOCK, n_sink=n_sink, budget_fixed=max(K, 1),
                         hh_fixed=HH)
        if K < 1:
            continue
        got = O.block_rank(cfg, length, live, scores, page=page, lib=lib)
        want = _block_expect(length, live, scores, n_sink, K, HH, page)
        assert list(got) == want, f"trial {trial}: {list(got)} vs {want}"


def pin_block_equal_scores(lib):
    """All scores equal: each head's heavy hitters are its HH oldest candidate
    tokens, so the first HH // page candidate blocks are fully important, one
    is partly, and the rest have importance zero; the victims are the oldest
    zero-importance blocks, and when more must go the partly important block
    follows before the fully important ones (oldest first among those)."""
    page, n_sink, HH, W = 4, 2, 10, 5
    K = n_sink + HH + W
    length = 40
    live = np.ones(length, dtype=np.uint8)
    cfg = O.make_cfg(head_dim=4, selector=O.ORC_BLOCK, n_sink=n_sink, budget_fixed=K, hh_fixed=HH)
    blocks = lambda ks: [p for k in ks for p in range(4 * k, 4 * k + 4)]
    # candidates: blocks 1..7 (block 0 holds sinks, block 8 reaches position 35 of the
    # window [35, 40)); importance over 3 heads: b1 = b2 = 12, b3 = 6, b4..b7 = 0;
    # n - K = 23 -> 6 blocks: the four zeros, then b3, then b1 (older than b2)
    got = O.block_rank(cfg, length, live, np.ones((3, length)), page=page, lib=lib)
    assert list(got) == blocks((1, 3, 4, 5, 6, 7))
    live2 = live.copy()
    live2[20:28] = 0  # blocks 5 and 6 already gone: n - K = 15 -> 4 of 1, 2, 3, 4, 7
    got = O.block_rank(cfg, length, live2, np.ones((3, length)), page=page, lib=lib)
    assert list(got) == blocks((1, 3, 4, 7))
    # n <= K: nothing goes
    live3 = np.zeros(length, dtype=np.uint8)
    live3[:K] = 1
    assert O.block_rank(cfg, length, live3, np.ones((1, length)), page=page, lib=lib).size == 0


def pin_block_page1_single_head_is_h2o(lib):
    """With pages of one token and one head, the block rule is H2O's token rule:
    once H2O runs, the retained set is sinks + candidates + the whole window, so
    the unimportant candidates are exactly the n - K lowest-scored ones.  An H2O
    unit and a block unit fed the same steps keep the same positions."""
    rng = np.random.default_rng(42)
    D, P, steps = 8, 30, 40
    pk, pv = rng.standard_normal((P, D)), rng.standard_normal((P, D))
    kw = dict(head_dim=D, n_sink=2, budget_fixed=14, hh_fixed=5)
    uh = _unit(lib, O.make_cfg(**kw), pk, pv, P + steps)
    ub = _unit(lib, O.make_cfg(selector=O.ORC_BLOCK, **kw), pk, pv, P + steps)
    for s in range(steps):
        q, k, v = rng.standard_normal((1, D)) * 2, rng.standard_normal(D), rng.standard_normal(D)
        uh.step(q, k, v)
        ub.attend(q, k, v)
        ub.evict(O.block_select([ub], page=1, lib=lib))
        ub.check()
        ph, sh, eh = uh.state()
        pb, sb, eb = ub.state()
        assert list(ph) == list(pb), f"step {s}"
        assert np.array_equal(sh, sb) and abs(eh - eb) <= 1e-12 * max(1.0, eh), f"step {s}"


def pin_block_run_invariants(lib):
    """A run of block eviction over two heads (units stepped, then
    orc_block_select on both): victims are the brute-force choice on the two
    units' scores, and they are whole blocks the units share, never
    a sink's block and never one reaching into the recent window; each step
    leaves n <= K unless no candidate block is left; and the evicted mass plus
    the retained scores add up to the total weight handed out (one per query
    head per step, plus the prompt's initial scores)."""
    rng = np.random.default_rng(43)
    D, G, P, steps, page = 8, 2, 80, 60, 4
    K, HH = 40, 24
    W = K - 3 - HH
    cfg = O.make_cfg(head_dim=D, group=G, selector=O.ORC_BLOCK, n_sink=3, budget_fixed=K, hh_fixed=HH)
    units = []
    for h in range(2):
        init = rng.random(P)
        units.append(_unit(lib, cfg, rng.standard_normal((P, D)), rng.standard_normal((P, D)),
                           P + steps, h=h, init=init))
    total0 = [float(np.sum(u.state()[1])) for u in units]
    evicted_blocks = 0
    for s in range(steps):
        for u in units:
            u.attend(rng.standard_normal((G, D)) * 2, rng.standard_normal(D), rng.standard_normal(D))
        length = P + s + 1
        pre = units[0].state()[0]
        vic = O.block_select(units, page=page, lib=lib)
        live = np.zeros(length, dtype=np.uint8)
        live[pre] = 1
        scores = np.zeros((len(units), length))
        for i, u in enumerate(units):
            pos_i, sc_i, _ = u.state()
            scores[i, pos_i] = sc_i
        assert list(vic) == _block_expect(length, live, scores, 3, K, HH, page), f"step {s}"
        assert len(vic) % page == 0
        for i in range(0, len(vic), page):
            blk = vic[i:i + page]
            assert blk[0] % page == 0 and list(blk) == list(range(blk[0], blk[0] + page))
            assert blk[0] >= 3 and blk[-1] < length - W
        for u in units:
            u.evict(vic)
            u.check()
        evicted_blocks += len(vic) // page
        post = units[0].state()[0]
        left = [k for k in range(length // page)
                if all(p in set(post.tolist()) for p in range(k * page, k * page + page))
                and k * page >= 3 and k * page + page - 1 < length - W]
        assert len(post) <= K or not left, f"step {s}: {len(post)} > {K} with {len(left)} candidates"
        assert len(pre) - len(post) == len(vic)
        for i, u in enumerate(units):
            _, sc, em = u.state()
            assert abs(float(np.sum(sc)) + em - total0[i] - G * (s + 1)) < 1e-9
    assert evicted_blocks > 5


# ------------------------------------------------ many units on threads
def pin_step_many_equals_sequential(lib):
    """orc_step_many (the CPU baseline's threaded driver) over N units equals N
    plain orc_step calls, bit for bit, whatever the thread count: outputs,
    retained positions, scores and evicted mass after every step.  A stride or
    join slip that skips or repeats a unit changes one of them."""
    rng = np.random.default_rng(29)
    D, G, P, steps, N = 8, 2, 14, 6, 7
    cfg = O.make_cfg(head_dim=D, group=G, n_sink=2, budget_fixed=10, hh_fixed=4)
    pk = [rng.standard_normal((P, D)) for _ in range(N)]
    pv = [rng.standard_normal((P, D)) for _ in range(N)]
    ins = [[(rng.standard_normal((G, D)), rng.standard_normal(D), rng.standard_normal(D))
            for _ in range(N)] for _ in range(steps)]
    ref = [_unit(lib, cfg, pk[i], pv[i], P + steps + 1, b=i, h=i % 3) for i in range(N)]
    ref_out = [[u.step(*ins[s][i]) for i, u in enumerate(ref)] for s in range(steps)]
    for nthreads in (1, 3, N + 2):
        us = [_unit(lib, cfg, pk[i], pv[i], P + steps + 1, b=i, h=i % 3) for i in range(N)]
        for s in range(steps):
            outs = O.step_many(us, [x[0] for x in ins[s]], [x[1] for x in ins[s]], [x[2] for x in ins[s]],
                               nthreads)
            for i in range(N):
                assert np.array_equal(outs[i], ref_out[s][i]), f"{nthreads} threads: unit {i} output"
        for i in range(N):
            a, b = us[i].state(), ref[i].state()
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2], \
                f"{nthreads} threads: unit {i} state"


# ------------------------------------------------- compressed score state
def pin_f16_rounding_matches_numpy(lib):
    """orc_round_f16 (binary16 storage of the scores) against numpy's float64
    -> float16 conversion, a library routine that rounds once, to nearest with
    ties to even: random values over the whole exponent range (subnormal,
    normal, overflowing), exact midpoints between neighbouring binary16 values
    and their fp64 neighbours, negative values, and the edges (0, the smallest
    subnormal and half of it, 65504, 65520)."""
    rng = np.random.default_rng(31)
    x = np.ldexp(rng.random(20000) + 0.5, rng.integers(-30, 18, 20000))
    h16 = np.arange(0, 0x7BFF, 7, dtype=np.uint16).view(np.float16)
    lo, hi = h16.astype(np.float64), np.nextafter(h16, np.float16(np.inf)).astype(np.float64)
    mids = (lo + hi) / 2  # exact: both have at most 11 significant bits
    edges = np.array([0.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25, 6.1e-5, 65504.0, 65519.99, 65520.0, 1e6])
    allx = np.concatenate([x, -x[:200], mids, np.nextafter(mids, 0.0), np.nextafter(mids, np.inf), edges])
    with np.errstate(over="ignore"):
        want = allx.astype(np.float16).astype(np.float64)
    got = O.round_f16(allx, lib=lib)
    assert np.array_equal(got, want), f"{int(np.sum(got != want))} values rounded differently from numpy"
    assert O.round_f16(np.array([np.nan]), lib=lib)[0] != O.round_f16(np.array([np.nan]), lib=lib)[0]


def pin_decay_closed_forms(lib):
    """Moving sum with decay lam, in closed form.  With zero queries every
    retained token takes the weight 1/n_att from each of the G query heads, and
    with no heavy hitters (4 sinks + window W, StreamingLLM) n_att = K + 1 at
    every step; a token that has taken m steps' weights then holds the
    geometric series G/(K+1) (1 - lam^m) / (1 - lam) (G m/(K+1) for lam = 1):
    the sinks m = T after T steps, a generated token m = T - s after its
    append at step s, and each step evicts the token leaving the window, the
    prompt's at m = s + 1 and the generated ones at m = W + 1.  Binary16
    storage (G = 1): every sink score equals numpy's float16 replay of
    s <- f16(lam s + 1/(K+1)), and initial scores enter rounded.  Adopting
    given scores (orc_set_scores) replaces them and refuses a position not
    retained."""
    rng = np.random.default_rng(33)
    D, K, W, steps = 4, 12, 8, 30
    P = K
    pk, pv = rng.standard_normal((P, D)), rng.standard_normal((P, D))
    for G, lam in ((2, 1.0), (2, 0.9), (3, 0.75)):
        cfg = O.make_cfg(head_dim=D, group=G, n_sink=4, budget_fixed=K, hh_fixed=0, decay=lam)
        u = _unit(lib, cfg, pk, pv, P + steps)

        def geo(m):
            return G / (K + 1) * (m if lam == 1.0 else (1 - lam ** m) / (1 - lam))
        for s in range(steps):
            u.step(np.zeros((G, D)), rng.standard_normal(D), rng.standard_normal(D))
            T = s + 1
            pos, sc, em = u.state()
            ages = np.array([T - (p - P) if p >= P else T for p in pos])
            ref = np.array([geo(a) for a in ages])
            assert np.max(np.abs(sc - ref) / ref) < 1e-12, f"G={G} decay={lam} step {s}: scores"
            em_ref = sum(geo(min(i + 1, W + 1)) for i in range(T))
            assert abs(em - em_ref) <= 1e-12 * em_ref, f"G={G} decay={lam} step {s}: evicted mass"
    lam = 0.9375
    init = rng.random(P) * 3.0
    cfg = O.make_cfg(head_dim=D, group=1, n_sink=4, budget_fixed=K, hh_fixed=0, decay=lam, score_f16=True)
    u = _unit(lib, cfg, pk, pv, P + steps, init=init)
    _, sc0, _ = u.state()
    assert np.array_equal(sc0, init.astype(np.float16).astype(np.float64)), "initial scores not rounded"
    sink = init[:4].astype(np.float16).astype(np.float64)
    for s in range(steps):
        u.step(np.zeros((1, D)), rng.standard_normal(D), rng.standard_normal(D))
        sink = (lam * sink + 1.0 / (K + 1)).astype(np.float16).astype(np.float64)
        _, sc, _ = u.state()
        assert np.array_equal(sc[:4], sink), f"binary16 step {s}: sink scores"
    pos, sc, _ = u.state()
    u.set_scores(pos[:3], [0.5, 0.25, 0.125])
    assert list(u.state()[1][:3]) == [0.5, 0.25, 0.125]
    try:
        u.set_scores([P + steps - W - 1], [1.0])  # evicted long ago
    except O.OracleError:
        pass
    else:
        raise AssertionError("set_scores accepted a position that is not retained")


ALL_PINS = [
    pin_f16_rounding_matches_numpy,
    pin_decay_closed_forms,
    pin_step_many_equals_sequential,
    pin_attention_full_cache,
    pin_scores_and_selection_recomputed,
    pin_streaming_llm_and_sliding_window,
    pin_greedy_equals_bruteforce,
    pin_topk_middle_region,
    pin_tie_break_lower_position_kept,
    pin_philox_matches_numpy,
    pin_random_victims_are_smallest_philox_words,
    pin_random_uniform_and_independent,
    pin_golden_streaming_layout,
    pin_golden_cache_manager_sizes,
    pin_colsum_identical_keys,
    pin_colsum_equals_decode_accumulation,
    pin_snapkv_pooling_and_union,
    pin_snapkv_topk_matches_library,
    pin_snapkv_ties_keep_lower_positions,
    pin_snapkv_votes_are_window_weights,
    pin_int8_rows,
    pin_block_bruteforce,
    pin_block_equal_scores,
    pin_block_page1_single_head_is_h2o,
    pin_block_run_invariants,
]
