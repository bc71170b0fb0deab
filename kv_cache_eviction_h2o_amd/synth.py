"""Seeded synthetic inputs for the H2O decode step (queries, keys, values).

This module only draws numbers.  It holds none of the method's arithmetic:
no attention, no scores, no selection.  Both the GPU path's tests and the CPU
oracle are fed from here, so the two sides see bit-identical inputs.

Recipe (the value structure the pages describe: a few heavy-hitter tokens whose
cumulative attention follows a power law, "H2O: Heavy-Hitter Oracle", summary
of observations; attention sinks at the first four positions, "Attention Sinks
and KV cache eviction", section 3):

* ``u`` is one seeded unit vector in R^D, shared by every layer and head.
* Keys:   k[p] = N(0,1)^D + m(p) * u.  m(p) = 2.0 at positions 0..3, and at a
  seeded Bernoulli(frac) subset of the other positions; elsewhere 0.  With a
  Zipf exponent set, the subset's magnitudes are 2.0 * Z with Z drawn from a
  Zipf law bounded to {1..zipf_n}.  The boost mask is per (layer, sequence,
  position) and shared by all heads of that sequence.
* Values: v[p] = N(0,1)^D.
* Queries: q[t] = N(0,1)^D + 2.0 * u for every query head and step.
* K/V are rounded to the cache dtype (bf16 by round-to-nearest-even) here, on
  the host, so both sides consume the same rounded values.

Streams are counter based: every block of 256 rows of one
(kind, layer, sequence, head) stream has its own numpy Philox key, so any
window of any unit can be regenerated on its own.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

KIND_U, KIND_BOOST, KIND_K, KIND_V, KIND_Q = 1, 2, 3, 4, 5
CHUNK = 256


@dataclass(frozen=True)
class Recipe:
    seed: int
    head_dim: int
    kv_dtype: str = "bf16"          # "f32" or "bf16"
    boost_frac: float = 0.02        # Bernoulli fraction of boosted key positions
    boost_mag: float = 2.0
    zipf_s: float | None = None     # power-law exponent of boost magnitudes
    zipf_n: int = 16                # Zipf support {1..zipf_n}
    n_fixed_boost: int = 4          # positions 0..n-1 are always boosted by boost_mag
    q_boost: float = 2.0


def stream_key(seed: int, kind: int, layer: int, b: int, h: int, chunk: int) -> np.ndarray:
    """Philox key of one 256-row block: word 0 = seed, word 1 = packed stream id.

    Packing (injective): kind 8 bits | layer 12 | sequence 12 | head 12 | block 20.
    """
    if not (0 <= kind < 256 and 0 <= layer < 4096 and 0 <= b < 4096 and 0 <= h < 4096
            and 0 <= chunk < (1 << 20)):
        raise ValueError("stream coordinates out of range")
    w1 = (kind << 56) | (layer << 44) | (b << 32) | (h << 20) | chunk
    return np.array([seed & 0xFFFFFFFFFFFFFFFF, w1], dtype=np.uint64)


def _gen(seed, kind, layer, b, h, chunk) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=stream_key(seed, kind, layer, b, h, chunk)))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def unit_vector(r: Recipe) -> np.ndarray:
    z = _gen(r.seed, KIND_U, 0, 0, 0, 0).standard_normal(r.head_dim, dtype=np.float64)
    return (z / np.sqrt(np.dot(z, z))).astype(np.float32)


def _zipf_cdf(s: float, n: int) -> np.ndarray:
    w = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def boost_magnitudes(r: Recipe, layer: int, b: int, p0: int, p1: int) -> np.ndarray:
    """m(p) for positions [p0, p1) of sequence b (float32, shared by all heads)."""
    out = np.zeros(max(0, p1 - p0), dtype=np.float32)
    if p1 <= p0:
        return out
    cdf = _zipf_cdf(r.zipf_s, r.zipf_n) if r.zipf_s is not None else None
    for c in range(p0 // CHUNK, (p1 - 1) // CHUNK + 1):
        g = _gen(r.seed, KIND_BOOST, layer, b, 0, c)
        hit = g.random(CHUNK) < r.boost_frac
        mag = np.full(CHUNK, r.boost_mag, dtype=np.float64)
        if cdf is not None:
            z = np.searchsorted(cdf, g.random(CHUNK), side="right") + 1
            mag = r.boost_mag * z
        pos = c * CHUNK + np.arange(CHUNK)
        m = np.where(hit, mag, 0.0)
        m = np.where(pos < r.n_fixed_boost, r.boost_mag, m)
        lo, hi = max(p0, c * CHUNK), min(p1, (c + 1) * CHUNK)
        out[lo - p0:hi - p0] = m[lo - c * CHUNK:hi - c * CHUNK]
    return out


def normal_rows(r: Recipe, kind: int, layer: int, b: int, h: int, p0: int, p1: int) -> np.ndarray:
    """Rows [p0, p1) of one N(0,1) stream, float32 [p1-p0][D]."""
    D = r.head_dim
    out = np.empty((max(0, p1 - p0), D), dtype=np.float32)
    if p1 <= p0:
        return out
    for c in range(p0 // CHUNK, (p1 - 1) // CHUNK + 1):
        blk = _gen(r.seed, kind, layer, b, h, c).standard_normal((CHUNK, D), dtype=np.float32)
        lo, hi = max(p0, c * CHUNK), min(p1, (c + 1) * CHUNK)
        out[lo - p0:hi - p0] = blk[lo - c * CHUNK:hi - c * CHUNK]
    return out


def _to_cache_dtype(r: Recipe, x: np.ndarray) -> np.ndarray:
    if r.kv_dtype == "bf16":
        return bf16_bits(x)
    if r.kv_dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(r.kv_dtype)


def cache_to_f64(r: Recipe, x: np.ndarray) -> np.ndarray:
    """Exact widening of cache-dtype values (uint16 bf16 bits or float32) to float64."""
    if r.kv_dtype == "bf16":
        return bf16_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def keys(r: Recipe, layer: int, b: int, h: int, p0: int, p1: int, u=None, mag=None) -> np.ndarray:
    u = unit_vector(r) if u is None else u
    mag = boost_magnitudes(r, layer, b, p0, p1) if mag is None else mag
    x = normal_rows(r, KIND_K, layer, b, h, p0, p1) + mag[:, None] * u[None, :]
    return _to_cache_dtype(r, x)


def values(r: Recipe, layer: int, b: int, h: int, p0: int, p1: int) -> np.ndarray:
    return _to_cache_dtype(r, normal_rows(r, KIND_V, layer, b, h, p0, p1))


def queries(r: Recipe, layer: int, b: int, g: int, p0: int, p1: int, u=None) -> np.ndarray:
    u = unit_vector(r) if u is None else u
    return normal_rows(r, KIND_Q, layer, b, g, p0, p1) + np.float32(r.q_boost) * u[None, :]


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _cache_np_dtype(r: Recipe):
    return np.uint16 if r.kv_dtype == "bf16" else np.float32


def prompt_kv(r: Recipe, layer: int, prompt_lens, n_kv_heads: int):
    """Packed prompts: K and V as [sum P_b][Hkv][D] in the cache dtype (bf16 as uint16 bits)."""
    lens = [int(x) for x in prompt_lens]
    D = r.head_dim
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    K = np.empty((int(off[-1]), n_kv_heads, D), dtype=_cache_np_dtype(r))
    V = np.empty_like(K)
    u = unit_vector(r)

    def work(b):
        mag = boost_magnitudes(r, layer, b, 0, lens[b])
        for h in range(n_kv_heads):
            K[off[b]:off[b + 1], h] = keys(r, layer, b, h, 0, lens[b], u=u, mag=mag)
            V[off[b]:off[b + 1], h] = values(r, layer, b, h, 0, lens[b])

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(len(lens))))
    return K, V


def prompt_queries(r: Recipe, layer: int, prompt_lens, n_q_heads: int) -> np.ndarray:
    """Packed prompt queries [sum P_b][Hq][D] float32: position p of sequence b has
    the query a decode step at position p would have (the same stream)."""
    lens = [int(x) for x in prompt_lens]
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    Q = np.empty((int(off[-1]), n_q_heads, r.head_dim), dtype=np.float32)
    u = unit_vector(r)

    def work(b):
        for g in range(n_q_heads):
            Q[off[b]:off[b + 1], g] = queries(r, layer, b, g, 0, lens[b], u=u)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(len(lens))))
    return Q


def step_window(r: Recipe, layer: int, t0, n_steps: int, n_q_heads: int, n_kv_heads: int):
    """Inputs of n_steps decode steps; sequence b's first step appends position t0[b].

    Returns q [n_steps][B][Hq][D] float32, k and v [n_steps][B][Hkv][D] in the cache dtype.
    """
    t0 = [int(x) for x in t0]
    B, D = len(t0), r.head_dim
    q = np.empty((n_steps, B, n_q_heads, D), dtype=np.float32)
    k = np.empty((n_steps, B, n_kv_heads, D), dtype=_cache_np_dtype(r))
    v = np.empty_like(k)
    u = unit_vector(r)

    def work(b):
        p0, p1 = t0[b], t0[b] + n_steps
        mag = boost_magnitudes(r, layer, b, p0, p1)
        for g in range(n_q_heads):
            q[:, b, g] = queries(r, layer, b, g, p0, p1, u=u)
        for h in range(n_kv_heads):
            k[:, b, h] = keys(r, layer, b, h, p0, p1, u=u, mag=mag)
            v[:, b, h] = values(r, layer, b, h, p0, p1)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(B)))
    return q, k, v


def uniform_lengths(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """n integer lengths uniform on [lo, hi] (inclusive), from their own Philox stream."""
    g = np.random.Generator(np.random.Philox(key=np.array([seed, 0xFFFF], dtype=np.uint64)))
    return g.integers(lo, hi + 1, size=n).astype(np.int32)


# ---------------------------------------------------------------------------
# Device-side drawing of the same recipe, for workloads too large to draw on
# the host (the benchmark's many layer instances).  The normals come from
# torch's seeded GPU generator, so the values differ from the numpy streams
# above; the structure (u, boost mask and magnitudes, rounding) is identical.
def _torch_seed(seed: int, kind: int, layer: int, b: int, block: int = 0) -> int:
    w1 = int(stream_key(seed, kind, layer, b, 0, block)[1])
    return (seed * 0x9E3779B97F4A7C15 + w1) & 0x7FFFFFFFFFFFFFFF


def device_prompt_kv(r: Recipe, layer: int, prompt_lens, n_kv_heads: int, device="cuda"):
    """Packed prompts [sum P_b][Hkv][D] as torch device tensors (bf16 or fp32)."""
    import torch
    lens = [int(x) for x in prompt_lens]
    D = r.head_dim
    dt = torch.bfloat16 if r.kv_dtype == "bf16" else torch.float32
    u = torch.from_numpy(unit_vector(r)).to(device)
    K = torch.empty((sum(lens), n_kv_heads, D), dtype=dt, device=device)
    V = torch.empty_like(K)
    off = 0
    for b, P in enumerate(lens):
        mag = torch.from_numpy(boost_magnitudes(r, layer, b, 0, P)).to(device)
        g = torch.Generator(device=device)
        g.manual_seed(_torch_seed(r.seed, KIND_K, layer, b))
        k = torch.randn((P, n_kv_heads, D), generator=g, device=device, dtype=torch.float32)
        K[off:off + P] = (k + mag[:, None, None] * u).to(dt)
        g.manual_seed(_torch_seed(r.seed, KIND_V, layer, b))
        V[off:off + P] = torch.randn((P, n_kv_heads, D), generator=g, device=device,
                                     dtype=torch.float32).to(dt)
        off += P
    return K, V


def device_prompt_queries(r: Recipe, layer: int, prompt_lens, n_q_heads: int, device="cuda"):
    """Packed prompt queries [sum P_b][Hq][D] fp32 as a torch device tensor."""
    import torch
    lens = [int(x) for x in prompt_lens]
    u = torch.from_numpy(unit_vector(r)).to(device)
    Q = torch.empty((sum(lens), n_q_heads, r.head_dim), dtype=torch.float32, device=device)
    off = 0
    for b, P in enumerate(lens):
        g = torch.Generator(device=device)
        g.manual_seed(_torch_seed(r.seed, KIND_Q, layer, b, 1 << 19))
        Q[off:off + P] = torch.randn((P, n_q_heads, r.head_dim), generator=g, device=device) + r.q_boost * u
        off += P
    return Q


def device_step_window(r: Recipe, layer: int, t0, n_steps: int, n_q_heads: int, n_kv_heads: int,
                       device="cuda"):
    """Inputs of n_steps decode steps as device tensors:
    q [n][B][Hq][D] fp32, k and v [n][B][Hkv][D] in the cache dtype."""
    import torch
    t0 = [int(x) for x in t0]
    B, D = len(t0), r.head_dim
    dt = torch.bfloat16 if r.kv_dtype == "bf16" else torch.float32
    u = torch.from_numpy(unit_vector(r)).to(device)
    g = torch.Generator(device=device)
    blk = t0[0] % (1 << 20)  # the window's first position names its streams
    g.manual_seed(_torch_seed(r.seed, KIND_Q, layer, 0, blk))
    q = torch.randn((n_steps, B, n_q_heads, D), generator=g, device=device) + r.q_boost * u
    mag = torch.stack([torch.from_numpy(boost_magnitudes(r, layer, b, t0[b], t0[b] + n_steps))
                       for b in range(B)], dim=1).to(device)  # [n][B]
    g.manual_seed(_torch_seed(r.seed, KIND_K, layer, 4095, blk))
    k = torch.randn((n_steps, B, n_kv_heads, D), generator=g, device=device)
    k = (k + mag[:, :, None, None] * u).to(dt)
    g.manual_seed(_torch_seed(r.seed, KIND_V, layer, 4095, blk))
    v = torch.randn((n_steps, B, n_kv_heads, D), generator=g, device=device).to(dt)
    return q.contiguous(), k.contiguous(), v.contiguous()
