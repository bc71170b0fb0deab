"""ctypes wrapper of the fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  It never imports the GPU package.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from .build import LIB, build

# a test may point the wrapper at another build of the same source (a sanitizer build)
LIB = os.environ.get("H2O_ORACLE_LIB") or LIB

ORC_H2O, ORC_RANDOM, ORC_BLOCK = 0, 1, 2
_dp = C.POINTER(C.c_double)
_ip = C.POINTER(C.c_int32)


class OrcCfg(C.Structure):
    _fields_ = [("head_dim", C.c_int), ("group", C.c_int), ("scale", C.c_double),
                ("selector", C.c_int), ("n_sink", C.c_int), ("budget_fixed", C.c_int),
                ("hh_fixed", C.c_int), ("budget_num", C.c_int), ("budget_den", C.c_int),
                ("rand_k", C.c_int), ("rand_r", C.c_int), ("seed", C.c_uint64),
                ("decay", C.c_double), ("score_f16", C.c_int)]


def _bind(lib):
    lib.orc_new.restype = C.c_void_p
    lib.orc_new.argtypes = [C.POINTER(OrcCfg), C.c_int, C.c_int, C.c_int, C.c_int, _dp, _dp, _dp]
    lib.orc_free.argtypes = [C.c_void_p]
    lib.orc_colsum.restype = C.c_int
    lib.orc_block_select.restype = C.c_int
    lib.orc_block_rank.restype = C.c_int
    lib.orc_block_rank.argtypes = [C.POINTER(OrcCfg), C.c_int, C.c_int, C.c_int, C.POINTER(C.c_ubyte), _dp, _ip]
    lib.orc_block_select.argtypes = [C.POINTER(C.c_void_p), C.c_int, C.c_int, _ip]
    lib.orc_snapkv_select.restype = C.c_int
    lib.orc_snapkv_select.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, _dp, _ip]
    lib.orc_snapkv.restype = C.c_int
    lib.orc_snapkv.argtypes = [C.POINTER(OrcCfg), C.c_int, C.c_int, C.c_int, C.c_int, _dp, _dp, _dp, _ip]
    lib.orc_colsum.argtypes = [C.POINTER(OrcCfg), C.c_int, C.c_int, _dp, _dp, C.c_int, _dp]
    lib.orc_schedule.argtypes = [C.POINTER(OrcCfg), C.c_int, _ip, _ip, _ip]
    lib.orc_attend.restype = C.c_int
    lib.orc_attend.argtypes = [C.c_void_p, _dp, _dp, _dp, _dp, _dp]
    lib.orc_select.restype = C.c_int
    lib.orc_select.argtypes = [C.c_void_p, _ip, _dp]
    lib.orc_evict.restype = C.c_int
    lib.orc_evict.argtypes = [C.c_void_p, _ip, C.c_int]
    lib.orc_check.restype = C.c_int
    lib.orc_check.argtypes = [C.c_void_p]
    lib.orc_step.restype = C.c_int
    lib.orc_step.argtypes = [C.c_void_p, _dp, _dp, _dp, _dp]
    lib.orc_state.restype = C.c_int
    lib.orc_state.argtypes = [C.c_void_p, _ip, _dp, _dp]
    lib.orc_score_of.restype = C.c_double
    lib.orc_score_of.argtypes = [C.c_void_p, C.c_int]
    lib.orc_length.restype = C.c_int
    lib.orc_length.argtypes = [C.c_void_p]
    lib.orc_step_many.restype = C.c_int
    lib.orc_step_many.argtypes = [C.POINTER(C.c_void_p), C.c_int, C.POINTER(_dp),
                                  C.POINTER(_dp), C.POINTER(_dp), C.POINTER(_dp), C.c_int]
    lib.orc_philox4x64_10.argtypes = [C.POINTER(C.c_uint64), C.POINTER(C.c_uint64),
                                      C.POINTER(C.c_uint64)]
    lib.orc_round_f16.restype = C.c_double
    lib.orc_round_f16.argtypes = [C.c_double]
    lib.orc_round_f16_many.restype = None
    lib.orc_round_f16_many.argtypes = [_dp, _dp, C.c_int]
    lib.orc_set_scores.restype = C.c_int
    lib.orc_set_scores.argtypes = [C.c_void_p, _ip, _dp, C.c_int]
    return lib


_LIBS: dict = {}


def load(path: str = LIB):
    """Load (building first if absent) an oracle shared library."""
    if path not in _LIBS:
        if not os.path.exists(path):
            build(out=path)
        _LIBS[path] = _bind(C.CDLL(path))
    return _LIBS[path]


def _p(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def make_cfg(*, head_dim, group=1, scale=0.0, selector=ORC_H2O, n_sink=4, budget_fixed=0,
             hh_fixed=0, budget_num=1, budget_den=5, rand_k=0, rand_r=0, seed=0, decay=1.0,
             score_f16=False) -> OrcCfg:
    return OrcCfg(head_dim, group, scale, selector, n_sink, budget_fixed, hh_fixed,
                  budget_num, budget_den, rand_k, rand_r, seed & 0xFFFFFFFFFFFFFFFF, float(decay),
                  1 if score_f16 else 0)


def cfg_from_workload(w, **over) -> OrcCfg:
    """Oracle parameters of a workload description (attributes read by name)."""
    sel = {"random": ORC_RANDOM, "block": ORC_BLOCK}.get(w.selector, ORC_H2O)
    kw = dict(head_dim=w.head_dim, group=w.n_q_heads // w.n_kv_heads, selector=sel,
              n_sink=w.n_sink, budget_fixed=w.budget_fixed, hh_fixed=w.hh_fixed,
              budget_num=w.budget_num, budget_den=w.budget_den, rand_k=w.rand_k,
              rand_r=w.rand_r, seed=w.recipe.seed, decay=getattr(w, "score_decay", 1.0),
              score_f16=getattr(w, "score_dtype", "f32") == "f16")
    kw.update(over)
    return make_cfg(**kw)


def schedule(cfg: OrcCfg, length: int, lib=None):
    lib = lib or load()
    K, HH, W = C.c_int32(), C.c_int32(), C.c_int32()
    lib.orc_schedule(C.byref(cfg), length, C.byref(K), C.byref(HH), C.byref(W))
    return K.value, HH.value, W.value


def colsum(cfg: OrcCfg, q, k, row_lo: int = 0, per_head: bool = False, lib=None) -> np.ndarray:
    """Causal-attention column sums of one unit's prompt (orc_colsum): q [P][G][D],
    k [P][D] -> [P] (summed over the group) or [G][P] (per_head)."""
    lib = lib or load()
    G, D = cfg.group, cfg.head_dim
    q = _f64(q).reshape(-1, G, D)
    P = q.shape[0]
    k = _f64(k).reshape(P, D)
    out = np.empty((G, P) if per_head else (P,), dtype=np.float64)
    rc = lib.orc_colsum(C.byref(cfg), P, int(row_lo), _p(q), _p(k), 1 if per_head else 0, _p(out))
    if rc != 0:
        raise OracleError(f"orc_colsum failed ({rc})")
    return out


def snapkv_select(votes, w: int, pool: int, keep: int, lib=None) -> np.ndarray:
    """SnapKV's kept positions of one unit from its votes [G][P] (orc_snapkv_select)."""
    lib = lib or load()
    v = _f64(votes)
    G, P = v.shape
    kept = np.empty(P, dtype=np.int32)
    n = lib.orc_snapkv_select(G, P, int(w), int(pool), int(keep), _p(v), kept.ctypes.data_as(_ip))
    if n < 0:
        raise OracleError(f"orc_snapkv_select failed ({n})")
    return kept[:n].copy()


def snapkv(cfg: OrcCfg, q, k, w: int, pool: int, keep: int, lib=None):
    """(kept positions, votes [G][P]) of one unit's prompt (orc_snapkv)."""
    lib = lib or load()
    G, D = cfg.group, cfg.head_dim
    q = _f64(q).reshape(-1, G, D)
    P = q.shape[0]
    k = _f64(k).reshape(P, D)
    votes = np.empty((G, P), dtype=np.float64)
    kept = np.empty(P, dtype=np.int32)
    n = lib.orc_snapkv(C.byref(cfg), P, int(w), int(pool), int(keep), _p(q), _p(k), _p(votes),
                       kept.ctypes.data_as(_ip))
    if n < 0:
        raise OracleError(f"orc_snapkv failed ({n})")
    return kept[:n].copy(), votes


def quantize_rows(x):
    """Int8 K/V rows with one scale per row: x [n][D] (any float dtype, taken as
    float32) -> (codes int8 [n][D], scale float32 [n]).

    Definition (the pages name INT8 K/V storage without fixing a scheme -- "KV
    cache eviction policies" page, section on alternatives used together with
    eviction (INT4/INT8 K/V, orthogonal to eviction); "Attention Sinks and KV
    cache eviction", sec. 1.2 (compressing each token's K/V by quantisation)):
    per row, in float32,
    a = max |x_d|, scale = a / 127, code_d = rint(x_d / scale) (round half to
    even) clamped to [-127, 127]; a row of zeros has scale 0 and codes 0.  The
    row stands for code_d * scale."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("rows [n][D] expected")
    a = np.max(np.abs(x), axis=1)
    scale = (a / np.float32(127.0)).astype(np.float32)
    codes = np.zeros(x.shape, dtype=np.int8)
    nz = scale > 0
    if np.any(nz):
        q = np.rint(x[nz] / scale[nz, None]).astype(np.float32)
        codes[nz] = np.clip(q, -127, 127).astype(np.int8)
    return codes, scale


def dequantize_rows(codes, scale) -> np.ndarray:
    """float64 rows code * scale (exact)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[:, None]


def block_select(units, page: int = 16, lib=None) -> np.ndarray:
    """Victim positions (whole blocks) of one sequence's KV-head units (orc_block_select)."""
    lib = lib or load()
    arr = (C.c_void_p * len(units))(*[u.ptr for u in units])
    vic = np.empty(units[0].length() + 1, dtype=np.int32)
    e = lib.orc_block_select(arr, len(units), int(page), vic.ctypes.data_as(_ip))
    if e < 0:
        raise OracleError(f"orc_block_select failed ({e})")
    return vic[:e].copy()


def block_rank(cfg: OrcCfg, length: int, live, scores, page: int = 16, lib=None) -> np.ndarray:
    """orc_block_rank: the block rule on given scores [n_heads][length] over the
    retained set live[length] (nonzero = retained); victim positions."""
    lib = lib or load()
    lv = np.ascontiguousarray(live, dtype=np.uint8).reshape(-1)
    sc = _f64(scores).reshape(-1, int(length))
    assert lv.size == length
    vic = np.empty(int(length) + 1, dtype=np.int32)
    e = lib.orc_block_rank(C.byref(cfg), int(length), int(page), sc.shape[0],
                           lv.ctypes.data_as(C.POINTER(C.c_ubyte)), _p(sc), vic.ctypes.data_as(_ip))
    if e < 0:
        raise OracleError(f"orc_block_rank failed ({e})")
    return vic[:e].copy()


def philox4x64_10(ctr, key, lib=None):
    lib = lib or load()
    c = (C.c_uint64 * 4)(*[int(x) & 0xFFFFFFFFFFFFFFFF for x in ctr])
    k = (C.c_uint64 * 2)(*[int(x) & 0xFFFFFFFFFFFFFFFF for x in key])
    o = (C.c_uint64 * 4)()
    lib.orc_philox4x64_10(c, k, o)
    return [int(x) for x in o]


def round_f16(x, lib=None) -> np.ndarray:
    """orc_round_f16 elementwise: the nearest IEEE binary16 values, as float64."""
    lib = lib or load()
    a = _f64(x).ravel().copy()
    out = np.empty_like(a)
    lib.orc_round_f16_many(_p(a), _p(out), len(a))
    return out.reshape(np.shape(x))


class OracleError(RuntimeError):
    pass


class Unit:
    """One (sequence, KV head) unit of the oracle."""

    def __init__(self, cfg: OrcCfg, b: int, h: int, prompt_k, prompt_v, cap: int,
                 init_scores=None, lib=None):
        self.lib = lib or load()
        self.cfg = cfg
        self.D, self.G = cfg.head_dim, cfg.group
        pk, pv = _f64(prompt_k).reshape(-1, self.D), _f64(prompt_v).reshape(-1, self.D)
        self.prompt_len = pk.shape[0]
        self.cap = int(cap)
        sc = None if init_scores is None else _f64(init_scores)
        self._keep = (pk, pv, sc)
        self.ptr = self.lib.orc_new(C.byref(cfg), b, h, self.prompt_len, self.cap, _p(pk), _p(pv),
                                    _p(sc) if sc is not None else None)
        if not self.ptr:
            raise OracleError("orc_new rejected the configuration")

    def __del__(self):
        if getattr(self, "ptr", None):
            self.lib.orc_free(self.ptr)
            self.ptr = None

    def length(self) -> int:
        return self.lib.orc_length(self.ptr)

    def attend(self, q, k, v, want_probs=False):
        q, k, v = _f64(q).reshape(self.G, self.D), _f64(k).reshape(self.D), _f64(v).reshape(self.D)
        out = np.empty((self.G, self.D), dtype=np.float64)
        probs = None
        if want_probs:
            n_max = self.length() + 1
            probs = np.empty(self.G * n_max, dtype=np.float64)
        n = self.lib.orc_attend(self.ptr, _p(q), _p(k), _p(v), _p(out),
                                _p(probs) if probs is not None else None)
        if n < 0:
            raise OracleError(f"orc_attend failed ({n})")
        if want_probs:
            return out, probs[:self.G * n].reshape(self.G, n)
        return out

    def select(self):
        vic = np.empty(self.length() + 1, dtype=np.int32)
        tau = C.c_double()
        e = self.lib.orc_select(self.ptr, vic.ctypes.data_as(_ip), C.byref(tau))
        if e < 0:
            raise OracleError(f"orc_select failed ({e})")
        return vic[:e].copy(), tau.value

    def evict(self, victims):
        vic = np.ascontiguousarray(victims, dtype=np.int32)
        rc = self.lib.orc_evict(self.ptr, vic.ctypes.data_as(_ip), len(vic))
        if rc != 0:
            raise OracleError(f"orc_evict rejected the victim set ({rc})")

    def check(self):
        rc = self.lib.orc_check(self.ptr)
        if rc != 0:
            raise OracleError(f"oracle invariant violated ({rc})")

    def step(self, q, k, v):
        q, k, v = _f64(q).reshape(self.G, self.D), _f64(k).reshape(self.D), _f64(v).reshape(self.D)
        out = np.empty((self.G, self.D), dtype=np.float64)
        rc = self.lib.orc_step(self.ptr, _p(q), _p(k), _p(v), _p(out))
        if rc != 0:
            raise OracleError(f"orc_step failed ({rc})")
        return out

    def state(self):
        n_max = self.length()
        pos = np.empty(max(1, n_max), dtype=np.int32)
        sc = np.empty(max(1, n_max), dtype=np.float64)
        em = C.c_double()
        n = self.lib.orc_state(self.ptr, pos.ctypes.data_as(_ip), _p(sc), C.byref(em))
        return pos[:n].copy(), sc[:n].copy(), em.value

    def set_scores(self, pos, scores):
        """Adopt these scores for retained positions pos (lockstep with an
        implementation whose stored scores are rounded differently)."""
        p = np.ascontiguousarray(pos, dtype=np.int32)
        sc = _f64(scores)
        if self.lib.orc_set_scores(self.ptr, p.ctypes.data_as(_ip), _p(sc), len(p)) != 0:
            raise OracleError("orc_set_scores: a position is not retained")

    def score_of(self, pos: int) -> float:
        return self.lib.orc_score_of(self.ptr, int(pos))


def step_many(units, qs, ks, vs, nthreads: int):
    """orc_step on many units at once (POSIX threads); returns outputs [n][G][D]."""
    lib = units[0].lib
    n = len(units)
    qs = [_f64(x) for x in qs]
    ks = [_f64(x) for x in ks]
    vs = [_f64(x) for x in vs]
    outs = [np.empty((u.G, u.D), dtype=np.float64) for u in units]
    arr = lambda xs: (_dp * n)(*[_p(x) for x in xs])
    ptrs = (C.c_void_p * n)(*[u.ptr for u in units])
    rc = lib.orc_step_many(ptrs, n, arr(qs), arr(ks), arr(vs), arr(outs), nthreads)
    if rc != 0:
        raise OracleError(f"orc_step_many failed ({rc})")
    return outs
