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
