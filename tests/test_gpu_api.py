"""Error paths of the C ABI on a live context: every rejected call returns its
status before anything is enqueued and leaves the context as it was.  Two
contexts take the same valid calls; one also takes the rejected ones, and the
two must end bit-identical (outputs, positions, scores, evicted mass)."""
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


def _setup(w, lens, steps, **cfg_over):
    import parity
    import torch
    from kv_cache_eviction_h2o_amd import _lib as L
    K, V = S.prompt_kv(w.recipe, 0, lens, w.n_kv_heads)
    # max_len admits exactly `steps` steps of the longest prompt
    cfg = L.config_from_workload(w, max_len=max(lens) + steps, **cfg_over)
    if w.page_size and not cfg.max_pages:
        cfg.max_pages = L.pages_needed(lens, steps, cfg)
    mk = lambda: L.H2OCache(cfg, lens, parity.to_dev(K, w.recipe.kv_dtype), parity.to_dev(V, w.recipe.kv_dtype))
    q, k, v = S.step_window(w.recipe, 0, lens, steps, w.n_q_heads, w.n_kv_heads)
    qd = torch.from_numpy(q).cuda()
    kd, vd = parity.to_dev(k, w.recipe.kv_dtype), parity.to_dev(v, w.recipe.kv_dtype)
    return cfg, mk, qd, kd, vd


def _same(a, b):
    pa, ca, sa, ea = a.read_indices()
    pb, cb, sb, eb = b.read_indices()
    assert np.array_equal(ca, cb) and np.array_equal(pa, pb)
    assert np.array_equal(sa, sb) and np.array_equal(ea, eb)
    assert a.info() == b.info()


@pytest.mark.parametrize("wname", ["gqa_tiles", "opt_rows", "paged"])
def test_rejected_calls_leave_the_context_unchanged(wname):
    import torch
    from kv_cache_eviction_h2o_amd import _lib as L
    w = {"gqa_tiles": WL.LLAMA_GQA.scaled(batch=2, budget_fixed=100, hh_fixed=48),
         "opt_rows": WL.OPT_LAYER.scaled(batch=2, n_q_heads=4, n_kv_heads=4),
         "paged": WL.PAGED_MIXED.scaled(batch=2, n_q_heads=4, n_kv_heads=4)}[wname]
    lens, steps = [150, 90], 14
    cfg, mk, qd, kd, vd = _setup(w, lens, steps)
    a, b = mk(), mk()
    lib = a.lib
    oa = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    ob = torch.empty_like(oa)
    # a buffer whose start is 4 bytes past an aligned address, for each argument in turn
    qx = torch.empty(qd[0].numel() + 4, dtype=torch.float32, device="cuda")
    sh = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptr = lambda t: C.c_void_p(t.data_ptr())
    for i in range(steps):
        if i == 2:  # misaligned q, k_new, v_new, out: rejected by both entry points
            for fn in (lib.h2o_step, lib.h2o_step_compact):
                args = [ptr(qd[i]), ptr(kd[i]), ptr(vd[i]), ptr(ob)]
                for j in range(4):
                    bad = list(args)
                    bad[j] = C.c_void_p(qx.data_ptr() + 4)
                    assert fn(b.ctx, *bad, sh) == L.H2O_EINVAL
                    assert "16-byte aligned" in lib.h2o_last_error(b.ctx).decode()
        if i == 4:  # nothing pending
            assert lib.h2o_compact(b.ctx, sh) == L.H2O_ESTATE
        if i == 6 or i == 9:  # a step pending: a second step, and reads, are refused
            a.step(qd[i], kd[i], vd[i], oa)
            b.step(qd[i], kd[i], vd[i], ob)
            for fn in (lib.h2o_step, lib.h2o_step_compact):
                assert fn(b.ctx, ptr(qd[i]), ptr(kd[i]), ptr(vd[i]), ptr(ob), sh) == L.H2O_ESTATE
            with pytest.raises(L.H2OError) as ex:
                b.read_indices()
            assert ex.value.code == L.H2O_ESTATE
            a.compact()
            b.compact()
        else:
            a.step_compact(qd[i], kd[i], vd[i], oa)
            b.step_compact(qd[i], kd[i], vd[i], ob)
        assert torch.equal(oa, ob), i
    # a read with too small a cap
    with pytest.raises(L.H2OError) as ex:
        b.read_indices(cap=1)
    assert ex.value.code == L.H2O_EINVAL
    _same(a, b)
    # the next step would pass max_len
    assert lib.h2o_step_compact(b.ctx, ptr(qd[0]), ptr(kd[0]), ptr(vd[0]), ptr(ob), sh) == L.H2O_EINVAL
    assert "max_len" in lib.h2o_last_error(b.ctx).decode()
    _same(a, b)
    a.close()
    b.close()


def test_page_pool_exhaustion_is_refused_and_recoverable_state():
    """Paged layout with a pool exactly as large as the prompts' pages and a
    budget above every length: the first step that needs a new page is
    refused with H2O_ENOMEM, and the context still reads back unchanged."""
    import torch
    from kv_cache_eviction_h2o_amd import _lib as L
    w = WL.PAGED_MIXED.scaled(batch=2, n_q_heads=4, n_kv_heads=4, budget_fixed=4096, hh_fixed=2000)
    lens = [32, 20]  # 2 + 2 pages; sequence 0 needs a third page at its first step
    cfg, mk, qd, kd, vd = _setup(w, lens, 4, max_pages=4)
    c = mk()
    before = c.read_indices()
    assert c.info()[1:] == (0, 4)
    o = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    for fused in (True, False):
        with pytest.raises(L.H2OError) as ex:
            (c.step_compact if fused else c.step)(qd[0], kd[0], vd[0], o)
        assert ex.value.code == L.H2O_ENOMEM
        assert c.info()[1:] == (0, 4)
    after = c.read_indices()
    for x, y in zip(before, after):
        assert np.array_equal(x, y)
    c.close()


@pytest.mark.parametrize("wname", ["opt_rows", "gqa_tiles", "paged", "block", "random", "int8"])
def test_workspace_context_matches_library_allocated(wname):
    """A context whose state lives in a caller's workspace (filled with 0xAB
    first, so nothing may rely on zeroed memory) steps bit-identically to one
    whose state the library allocates; a workspace one byte short is refused."""
    import torch
    from kv_cache_eviction_h2o_amd import _lib as L
    w = {"opt_rows": WL.OPT_LAYER.scaled(batch=2, n_q_heads=4, n_kv_heads=4),
         "gqa_tiles": WL.LLAMA_GQA.scaled(batch=2, budget_fixed=100, hh_fixed=48),
         "paged": WL.PAGED_MIXED.scaled(batch=2, n_q_heads=4, n_kv_heads=4),
         "block": WL.PAGED_BLOCK.scaled(batch=2, n_q_heads=4, n_kv_heads=4),
         "random": WL.RANDOM_ATTN.scaled(batch=2, n_q_heads=8, n_kv_heads=2, rand_k=24, rand_r=8),
         "int8": WL.OPT_LAYER_I8.scaled(batch=2, n_q_heads=4, n_kv_heads=4)}[wname]
    lens, steps = ([400, 150] if wname != "random" else [40, 30]), 40
    import parity
    K, V = S.prompt_kv(w.recipe, 0, lens, w.n_kv_heads)
    cfg = L.config_from_workload(w, max_len=max(lens) + steps + 1)
    if w.page_size:
        cfg.max_pages = L.pages_needed(lens, steps, cfg)
    dk, dv = parity.to_dev(K, w.recipe.kv_dtype), parity.to_dev(V, w.recipe.kv_dtype)
    n = L.workspace_size(cfg, lens)
    print(f"[workspace] {wname}: {n} bytes", flush=True)
    with pytest.raises(L.H2OError) as ex:
        L.H2OCache(cfg, lens, dk, dv, workspace=torch.empty(n - 1, dtype=torch.uint8, device="cuda"))
    assert ex.value.code == L.H2O_EINVAL and "h2o_workspace_size" in str(ex.value)
    ws = torch.full((n,), 0xAB, dtype=torch.uint8, device="cuda")
    a = L.H2OCache(cfg, lens, dk, dv)
    b = L.H2OCache(cfg, lens, dk, dv, workspace=ws)
    q, k, v = S.step_window(w.recipe, 0, lens, steps, w.n_q_heads, w.n_kv_heads)
    qd = torch.from_numpy(q).cuda()
    kd, vd = parity.to_dev(k, w.recipe.kv_dtype), parity.to_dev(v, w.recipe.kv_dtype)
    oa = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    ob = torch.empty_like(oa)
    for i in range(steps):
        if i % 3 == 2:
            for c, o in ((a, oa), (b, ob)):
                c.step(qd[i], kd[i], vd[i], o)
                c.compact()
        else:
            a.step_compact(qd[i], kd[i], vd[i], oa)
            b.step_compact(qd[i], kd[i], vd[i], ob)
        assert torch.equal(oa, ob), i
    _same(a, b)
    for x, y in zip(a.read_kv(), b.read_kv()):
        assert (x is None and y is None) or np.array_equal(x, y)
    a.close()
    b.close()
    assert int(ws[:16].sum()) >= 0  # the caller's memory is still the caller's


def _two_thread_check():
    """Two contexts stepped at once from two host threads, each on its own
    stream, then twins of both stepped one after the other on one thread: every
    step's outputs and the final states must be bit-identical.  Both kernels keep
    more than the default 48 KB of dynamic LDS (their logits: the matrix-core
    kernel 8 heads x 1728 slots, the FMA kernel 1 head x 14101 slots), so in a
    fresh process the two threads race to raise the same launch limits."""
    import threading

    import torch
    ws = [WL.LLAMA_GQA.scaled(batch=2, budget_fixed=1700, hh_fixed=800),
          WL.OPT_LAYER.scaled(batch=2, n_q_heads=2, n_kv_heads=2, budget_fixed=14000, hh_fixed=7000)]
    lens = [[1750, 1600], [14100, 9000]]
    steps = 24
    setups = [_setup(w, l, steps) for w, l in zip(ws, lens)]
    outs = [[None] * steps for _ in ws]
    caches = [mk() for (_, mk, _, _, _) in setups]
    torch.cuda.synchronize()
    errors = []

    def drive(i):
        try:
            _, _, qd, kd, vd = setups[i]
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                o = torch.empty((ws[i].batch, ws[i].n_q_heads, ws[i].head_dim), dtype=torch.float32,
                                device="cuda")
                for s in range(steps):
                    caches[i].step_compact(qd[s], kd[s], vd[s], o)
                    outs[i][s] = o.clone()
            st.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    th = [threading.Thread(target=drive, args=(i,)) for i in range(len(ws))]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errors, errors
    for i, w in enumerate(ws):
        _, mk, qd, kd, vd = setups[i]
        twin = mk()
        o = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
        for s in range(steps):
            twin.step_compact(qd[s], kd[s], vd[s], o)
            assert torch.equal(o, outs[i][s]), f"context {i} step {s}: outputs differ"
        _same(caches[i], twin)
    print("two-thread check ok", flush=True)


def test_two_threads_drive_two_contexts():
    """_two_thread_check in a fresh process, so that the dynamic-LDS launch
    limits start unraised and both threads reach them together."""
    import os
    import subprocess
    import sys
    tests = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(tests)
    code = (f"import sys; sys.path[:0] = [{root!r}, {tests!r}]; "
            "import test_gpu_api as t; t._two_thread_check()")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "two-thread check ok" in r.stdout, (r.stdout[-2000:], r.stderr[-3000:])
