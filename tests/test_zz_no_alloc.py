"""h2o_snapkv_select_noalloc (the SnapKV selection on the library's fixed
per-device scratch, for callers that cannot allocate) against
h2o_snapkv_select on the same inputs, through the C ABI: kept positions,
kept counts and votes bit for bit, on two calls in a row (the second smaller),
with the votes in the caller's buffer and in the scratch; and a call whose
scratch need exceeds the fixed size is refused before anything runs."""
import ctypes as C

import numpy as np
import pytest

from kv_cache_eviction_h2o_amd import synth as S
from kv_cache_eviction_h2o_amd import workloads as WL

pytestmark = pytest.mark.gpu

FIXED = 64 << 20  # bytes of the library's scratch array


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_eviction_h2o_amd import _lib
    _lib.load_library()


def _inputs(w, lens):
    import torch
    K, _ = S.prompt_kv(w.recipe, 0, lens, w.n_kv_heads)
    Q = S.prompt_queries(w.recipe, 0, lens, w.n_q_heads)
    kd = torch.from_numpy(np.ascontiguousarray(K).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(Q).cuda(), kd


def _call(fn, cfg, lens, q, k, window, pool, keep, with_votes):
    import torch
    from kv_cache_eviction_h2o_amd import _lib as L
    G = cfg.n_q_heads // cfg.n_kv_heads
    cap = max(min(P, min(window, P) + G * min(keep, P - min(window, P))) for P in lens)
    total = sum(lens)
    votes = torch.full((total, cfg.n_q_heads), -1.0, dtype=torch.float64, device="cuda")
    kept = torch.full((cfg.batch, cfg.n_kv_heads, cap), -7, dtype=torch.int32, device="cuda")
    count = torch.full((cfg.batch, cfg.n_kv_heads), -7, dtype=torch.int32, device="cuda")
    arr = (C.c_int32 * len(lens))(*lens)
    sh = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = fn(C.byref(cfg), arr, window, pool, keep, C.c_void_p(q.data_ptr()), C.c_void_p(k.data_ptr()),
            C.c_void_p(votes.data_ptr()) if with_votes else None, C.c_void_p(kept.data_ptr()),
            C.c_void_p(count.data_ptr()), cap, sh)
    assert rc == L.H2O_OK, L.load_library().h2o_last_error(None).decode()
    torch.cuda.synchronize()
    return kept.cpu().numpy(), count.cpu().numpy(), votes.cpu().numpy()


def test_noalloc_matches_snapkv_select_two_calls():
    from kv_cache_eviction_h2o_amd import _lib as L
    lib = L.load_library()
    cases = [  # the first call larger than the second
        (WL.LLAMA_GQA.scaled(batch=3, n_q_heads=32, n_kv_heads=4), [3000, 1777, 2500], 32, 7, 400),
        (WL.OPT_LAYER.scaled(batch=2, n_q_heads=4, n_kv_heads=4), [600, 333], 16, 5, 60),
    ]
    for with_votes in (True, False):
        for w, lens, window, pool, keep in cases:
            cfg = L.config_from_workload(w, max_len=max(lens) + 1)
            q, k = _inputs(w, lens)
            ref = _call(lib.h2o_snapkv_select, cfg, lens, q, k, window, pool, keep, with_votes)
            got = _call(lib.h2o_snapkv_select_noalloc, cfg, lens, q, k, window, pool, keep, with_votes)
            print(f"[no-alloc] {w.name} B={len(lens)} G={w.group} lens={lens} votes in "
                  f"{'caller buffer' if with_votes else 'scratch'}: kept {int(ref[1].sum())}", flush=True)
            assert np.array_equal(got[1], ref[1]), "kept counts differ"
            assert np.array_equal(got[0], ref[0]), "kept positions differ"
            if with_votes:
                assert np.array_equal(got[2], ref[2]), "votes differ"
            assert ref[1].min() >= min(window, min(lens))


def test_noalloc_refuses_scratch_above_the_fixed_size():
    from kv_cache_eviction_h2o_amd import _lib as L
    lib = L.load_library()
    w = WL.OPT_LAYER.scaled(batch=8)
    lens = [16384] * 8  # votes and pooled votes in scratch: 2 x 8 B x 131072 x 32 = 64 MiB + the passes
    cfg = L.config_from_workload(w, max_len=16385)
    arr = (C.c_int32 * 8)(*lens)
    p = C.c_void_p(256)  # never touched: the size check comes before anything is enqueued
    rc = lib.h2o_snapkv_select_noalloc(C.byref(cfg), arr, 32, 7, 100, p, p, None, p, p, 16384, None)
    assert rc == L.H2O_EINVAL
    msg = lib.h2o_last_error(None).decode()
    assert "scratch" in msg and str(FIXED) in msg
