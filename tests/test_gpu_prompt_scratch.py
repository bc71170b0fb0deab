"""The prompt calls' scratch (h2o_prefill_scores, h2o_snapkv_select): one
grow-only device buffer per device, reused by every call and ordered across
streams.  The column sums and the selection are deterministic, so a call
interleaved with others -- of other sizes, on another stream, with no host wait
in between -- must return the same bits as the same call made alone.  SnapKV
without a votes buffer (votes in the scratch) must keep the same positions as
with one.  The values themselves are checked against the oracle in
test_gpu_prefill.py and test_gpu_snapkv.py."""
import ctypes as C

import numpy as np
import pytest

from kv_cache_eviction_h2o_amd import synth as S
from kv_cache_eviction_h2o_amd import workloads as WL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_eviction_h2o_amd import _lib
    _lib.load_library()


def _inputs(w, lens, layer):
    import torch
    from kv_cache_eviction_h2o_amd import _lib as L
    K, _ = S.prompt_kv(w.recipe, layer, lens, w.n_kv_heads)
    Q = S.prompt_queries(w.recipe, layer, lens, w.n_q_heads)
    kd = torch.from_numpy(np.ascontiguousarray(K).view(np.int16)).view(torch.bfloat16).cuda()
    qd = torch.from_numpy(Q).cuda()
    cfg = L.config_from_workload(w.scaled(batch=len(lens)), max_len=max(lens) + 1)
    return cfg, qd, kd


def test_prefill_calls_interleaved_on_two_streams():
    import torch
    from kv_cache_eviction_h2o_amd import _lib as L
    w = WL.OPT_LAYER.scaled(n_q_heads=8, n_kv_heads=8)
    cases = [[300, 517], [2048, 1500, 1024], [64], [4096, 4096]]  # the last grows the scratch
    ins = [_inputs(w, lens, layer=i) for i, lens in enumerate(cases)]
    alone = []
    for (cfg, qd, kd), lens in zip(ins, cases):
        alone.append(L.prefill_scores(cfg, lens, qd, kd).clone())
        torch.cuda.synchronize()
    print(f"[scratch] prefill cases {[len(x) for x in cases]} computed alone", flush=True)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = [torch.full_like(a, -1.0) for a in alone for _ in range(2)]
    torch.cuda.synchronize()  # the fills run on the default stream
    # every case twice, alternating streams, largest last on the second pass
    order = [(i, r) for r in range(2) for i in range(len(cases))]
    for n, (i, r) in enumerate(order):
        cfg, qd, kd = ins[i]
        L.prefill_scores(cfg, cases[i], qd, kd, out=outs[2 * i + r], stream=s1 if n % 2 == 0 else s2)
    torch.cuda.synchronize()
    for i in range(len(cases)):
        for r in range(2):
            assert torch.equal(outs[2 * i + r], alone[i]), (i, r)


def test_snapkv_votes_in_scratch_and_two_streams():
    import torch
    from kv_cache_eviction_h2o_amd import _lib as L
    lib = L.load_library()
    w = WL.LLAMA_GQA.scaled(n_q_heads=16, n_kv_heads=2)
    cases = [([700, 250], 40), ([3000, 1200, 64], 300)]
    ref = []
    for i, (lens, keep) in enumerate(cases):
        cfg, qd, kd = _inputs(w, lens, layer=10 + i)
        kept, count, votes = L.snapkv_select(cfg, lens, qd, kd, 32, 7, keep)
        torch.cuda.synchronize()
        ref.append((cfg, qd, kd, kept.clone(), count.clone()))
    print("[scratch] snapkv cases computed alone", flush=True)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    runs = list(zip(cases, ref)) * 2
    got = [(torch.full_like(r[3], -7), torch.full_like(r[4], -7)) for _, r in runs]
    torch.cuda.synchronize()  # the fills run on the default stream
    for n, ((lens, keep), (cfg, qd, kd, kept, count)) in enumerate(runs):
        k2, c2 = got[n]
        lens_c = (C.c_int32 * len(lens))(*lens)
        st = s1 if n % 2 == 0 else s2
        rc = lib.h2o_snapkv_select(C.byref(cfg), lens_c, 32, 7, keep, C.c_void_p(qd.data_ptr()),
                                   C.c_void_p(kd.data_ptr()), None, C.c_void_p(k2.data_ptr()),
                                   C.c_void_p(c2.data_ptr()), int(kept.shape[2]), C.c_void_p(st.cuda_stream))
        assert rc == 0, lib.h2o_last_error(None).decode()
    torch.cuda.synchronize()
    for n, (k2, c2) in enumerate(got):
        _, _, _, kept, count = ref[n % len(cases)]
        assert torch.equal(c2, count), n
        assert torch.equal(k2, kept), n


def _growth_check():
    """Run in a fresh process (the scratch then starts empty): each call is
    larger than the last and on the other stream, so each grows the scratch,
    releasing the old buffer behind the other stream's work."""
    import torch
    from kv_cache_eviction_h2o_amd import _lib as L
    L.load_library()
    w = WL.OPT_LAYER.scaled(n_q_heads=4, n_kv_heads=4)
    cases = [[100], [600, 300], [1500, 1500], [3000, 2000, 1000]]
    ins = [_inputs(w, lens, layer=20 + i) for i, lens in enumerate(cases)]
    outs = [torch.empty((sum(lens), w.n_kv_heads), dtype=torch.float64, device="cuda") for lens in cases]
    torch.cuda.synchronize()  # the input copies run on the default stream
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    got = []
    for n, ((cfg, qd, kd), lens) in enumerate(zip(ins, cases)):
        got.append(L.prefill_scores(cfg, lens, qd, kd, out=outs[n], stream=s1 if n % 2 == 0 else s2))
    torch.cuda.synchronize()
    for (cfg, qd, kd), lens, g in zip(ins, cases, got):
        alone = L.prefill_scores(cfg, lens, qd, kd)
        torch.cuda.synchronize()
        assert torch.equal(g, alone), lens
    print("growth check ok", flush=True)


def test_prefill_scratch_growth_across_streams_fresh_process():
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.abspath(__file__)], cwd=root, capture_output=True, text=True,
                       timeout=100, env={**os.environ, "PYTHONPATH": root})
    assert r.returncode == 0 and "growth check ok" in r.stdout, (r.stdout[-2000:], r.stderr[-2000:])


if __name__ == "__main__":
    _growth_check()
