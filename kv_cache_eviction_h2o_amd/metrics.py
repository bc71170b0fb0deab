"""Byte accounting of the decode step (host arithmetic, no device work).

Algorithmic bytes of one step for one (sequence, KV head) unit holding n_att
retained slots after the append, with row = D x element bytes:
  K and V rows read         (n_att - 1) * 2 * row   (the new token arrives as input)
  new k, v read + written   2 * 2 * row
  cumulative score RMW      n_att * 2 * score_bytes (H2O; none for Random)
  q read, output written    2 * G * D * 4
Not counted (implementation overhead): slot positions read for the candidate
mask, block-table reads, LDS traffic.

Cache-size arithmetic follows the pages: KV bytes per token = 2 (K and V) x
layers x KV heads x head dim x element bytes ("Attention Sinks and KV cache
eviction", sec. 1.1); per-token cumulative-score state = score bytes per token
(sec. 6.2).
"""
from __future__ import annotations

import numpy as np


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * n_layers * n_kv_heads * head_dim * elem_bytes


def score_state_bytes(n_tokens: int, batch: int = 1, score_bytes: int = 4) -> int:
    return n_tokens * batch * score_bytes


def unit_step_bytes(n_att, *, head_dim: int, kv_elem: int, group: int, score_bytes: int,
                    int8_rows: bool = False):
    """Algorithmic bytes of one unit-step (n_att may be an array): the retained K and V
    rows read once, the new token's rows read from the input and written to the cache,
    each score read and written, q read and the output written.  int8_rows: stored rows
    are head_dim int8 codes plus a 4-byte scale; the inputs stay head_dim * kv_elem."""
    row_in = head_dim * kv_elem
    row = head_dim + 4 if int8_rows else row_in
    n = np.asarray(n_att, dtype=np.int64)
    return (n - 1) * 2 * row + 2 * row_in + 2 * row + n * 2 * score_bytes + 2 * group * head_dim * 4


def launch_bytes(n_att_per_seq, *, n_kv_heads: int, head_dim: int, kv_elem: int, group: int,
                 score_bytes: int, int8_rows: bool = False) -> int:
    """Algorithmic bytes of one step launch: every head of sequence b holds n_att[b] slots."""
    per = unit_step_bytes(n_att_per_seq, head_dim=head_dim, kv_elem=kv_elem, group=group,
                          score_bytes=score_bytes, int8_rows=int8_rows)
    return int(np.sum(per) * n_kv_heads)


PAGE = 16


def schedule(w, length: int):
    """Budget K, heavy hitters HH and recent window W at a sequence length (the
    workload's fixed or proportional budget; the same rule as the library's)."""
    if w.budget_fixed > 0:
        K, HH = w.budget_fixed, w.hh_fixed
    else:
        K = length * w.budget_num // w.budget_den
        HH = (K - w.n_sink) // 2
    return K, HH, K - w.n_sink - HH


def retained_counts(w, P: int, n_steps: int) -> dict:
    """Host mirror of one sequence's counts over n_steps decode steps (prompt P):
    n_att (slots attended at each step, after the append), count (retained
    after the step), and for block eviction pages (pages evicted at the step)
    and cand (candidate pages it ranked).  H2O keeps min(n_att, K_t); Random
    Attention drops r at each event; block eviction drops whole pages: with
    n_att > K_t, min(candidates, ceil((n_att - K_t) / 16)) of them, where the
    candidates are the pages past the sinks' pages that end before the recent
    window, less those already evicted (all of which lay before it)."""
    n_att = np.empty(n_steps, dtype=np.int64)
    count = np.empty(n_steps, dtype=np.int64)
    pages = np.zeros(n_steps, dtype=np.int64)
    cand = np.zeros(n_steps, dtype=np.int64)
    c, evicted = P, 0
    js = (w.n_sink + PAGE - 1) // PAGE
    for s in range(n_steps):
        length = P + s + 1
        n = c + 1
        n_att[s] = n
        if w.selector == "h2o":
            c = min(n, schedule(w, length)[0])
        elif w.selector == "block":
            K, _, W = schedule(w, length)
            if n > K:
                nc = max(0, (length - W) // PAGE - js) - evicted
                m = min(nc, -(-(n - K) // PAGE))
                if m > 0:
                    pages[s], cand[s] = m, nc
                    evicted += m
                    n -= m * PAGE
            c = n
        else:
            c = n - (w.rand_r if n - P == w.rand_k + w.rand_r else 0)
        count[s] = c
    return {"n_att": n_att, "count": count, "pages": pages, "cand": cand}


def block_launch_bytes(cand, pages, n_att, *, n_kv_heads: int, score_bytes: int) -> int:
    """Algorithmic bytes of the block-eviction launches after one step, over the
    sequences that lose pages (arrays per such sequence): each head's candidate
    scores read once, its per-page important counts written and read back, the
    sequence's block-table row read and written, and per freed page the slots'
    scores read and positions written."""
    cand = np.asarray(cand, dtype=np.int64)
    pages = np.asarray(pages, dtype=np.int64)
    rows = (np.asarray(n_att, dtype=np.int64) + PAGE - 1) // PAGE
    per_seq = (n_kv_heads * cand * PAGE * score_bytes + 2 * n_kv_heads * cand + 2 * rows * 4
               + n_kv_heads * pages * PAGE * (score_bytes + 4) + pages * 4)
    return int(per_seq.sum())
