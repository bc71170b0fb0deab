"""The C-ABI library on the CPU: it loads, exports what include/h2o.h declares,
its struct layout matches the binding, and it validates before touching a device."""
import ctypes as C
import os
import re
import subprocess

import pytest

from kv_cache_eviction_h2o_amd import _lib as L
from kv_cache_eviction_h2o_amd.build import INCLUDE, LIB, build

HEADER = os.path.join(INCLUDE, "h2o.h")
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        build()
    return L.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(h2o_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree_on_symbols():
    assert declared_functions() == sorted(L.SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (h2o_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_config_struct_layout_matches_c(tmp_path):
    fields = [f for f, _ in L.H2OConfig._fields_]
    prog = ["#include <stdio.h>", "#include <stddef.h>", '#include "h2o.h"', "int main(void){",
            'printf("%zu\\n", sizeof(h2o_config));']
    prog += [f'printf("%zu\\n", offsetof(h2o_config, {f}));' for f in fields]
    prog += ["return 0;}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(prog))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", INCLUDE, "-o", str(exe), str(src)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == C.sizeof(L.H2OConfig)
    assert vals[1:] == [getattr(L.H2OConfig, f).offset for f in fields]


def _init(lib, cfg, lens):
    ctx = C.c_void_p()
    arr = (C.c_int32 * len(lens))(*lens)
    rc = lib.h2o_init(C.byref(ctx), C.byref(cfg), arr, C.c_void_p(16), C.c_void_p(16), None, None)
    return rc, ctx


GOOD = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, kv_dtype="bf16", score_dtype="f32",
            budget_fixed=64, hh_fixed=28, max_len=4096)


@pytest.mark.parametrize("bad,msg", [
    (dict(n_q_heads=7), "multiple"),
    (dict(n_q_heads=6), "group size"),
    (dict(n_q_heads=32, n_kv_heads=2), "group size"),
    (dict(head_dim=64), "head_dim"),
    (dict(kv_dtype="f32", head_dim=128), "head_dim"),
    (dict(kv_dtype="i8", head_dim=64), "head_dim"),
    (dict(hh_fixed=61), "hh_fixed"),
    (dict(budget_fixed=0, budget_num=3, budget_den=2), "proportional"),
    (dict(budget_fixed=0, budget_num=1, budget_den=500), "below n_sink"),
    (dict(selector="random", rand_r=0), "Random"),
    (dict(page_size=8), "page_size"),
    (dict(page_size=16, max_pages=0), "max_pages"),
    (dict(page_size=16, kv_dtype="f32", head_dim=64, max_pages=64), "bf16"),
    (dict(max_len=100), "max_len"),
    (dict(scale=-1.0), "scale"),
    (dict(selector="block"), "paged layout"),
    (dict(selector="block", page_size=16, max_pages=64, n_q_heads=2048, n_kv_heads=2048), "1024 KV heads"),
    (dict(selector="block", page_size=16, max_pages=64, hh_fixed=61), "hh_fixed"),
    (dict(selector="block", page_size=16, max_pages=64, score_dtype="bf16"), "score_dtype"),
    (dict(selector="block", page_size=16, max_pages=64, score_dtype="f16"), "H2O selector"),
    (dict(score_dtype="i8"), "score_dtype"),
    (dict(score_decay=1.5), "score_decay"),
    (dict(score_decay=-0.5), "score_decay"),
    (dict(selector="block", page_size=16, max_pages=64, budget_fixed=0, budget_num=1, budget_den=5,
          max_len=500000), "5120 pages"),
])
def test_invalid_config_rejected_before_device(lib, bad, msg):
    cfg = L.make_config(**{**GOOD, **bad})
    rc, ctx = _init(lib, cfg, [100, 200])
    assert rc == L.H2O_EINVAL
    assert not ctx.value
    assert msg in lib.h2o_last_error(None).decode()


def test_invalid_prompt_lengths_rejected(lib):
    cfg = L.make_config(**GOOD)
    assert _init(lib, cfg, [0, 10])[0] == L.H2O_EINVAL
    assert _init(lib, cfg, [10, 4096])[0] == L.H2O_EINVAL


def test_null_arguments(lib):
    assert lib.h2o_step(None, None, None, None, None, None) == L.H2O_EINVAL
    assert lib.h2o_step_compact(None, None, None, None, None, None) == L.H2O_EINVAL
    assert lib.h2o_compact(None, None) == L.H2O_EINVAL
    assert lib.h2o_info(None, None, None, None) == L.H2O_EINVAL
    lib.h2o_destroy(None)
    cfg = L.make_config(**GOOD)
    arr = (C.c_int32 * 2)(10, 20)
    assert lib.h2o_init(None, C.byref(cfg), arr, None, None, None, None) == L.H2O_EINVAL
    ctx = C.c_void_p()
    assert lib.h2o_init(C.byref(ctx), C.byref(cfg), arr, None, None, None, None) == L.H2O_EINVAL


def test_init_rejects_misaligned_device_pointers(lib):
    cfg = L.make_config(**GOOD)
    arr = (C.c_int32 * 2)(10, 20)
    ctx = C.c_void_p()
    for k, v, s in ((20, 16, None), (16, 8, None), (16, 16, 4)):
        rc = lib.h2o_init(C.byref(ctx), C.byref(cfg), arr, C.c_void_p(k), C.c_void_p(v),
                          C.c_void_p(s) if s else None, None)
        assert rc == L.H2O_EINVAL and not ctx.value
        assert "16-byte aligned" in lib.h2o_last_error(None).decode()


def test_c_client_compiles_against_the_header(tmp_path):
    """The C client check (run on a GPU by test_gpu_c_client.py) builds with gcc
    against include/h2o.h and the library, warning-free."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("c_build", os.path.join(HERE, "c", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    r = subprocess.run(mod.command(str(tmp_path / "h2o_c_check")) + ["-Werror"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_workspace_size_host_logic(lib):
    """h2o_workspace_size validates like h2o_init, needs no device, covers at
    least the K and V rows of every slot, and grows with the batch."""
    cfg = L.make_config(**GOOD)
    n2 = L.workspace_size(cfg, [100, 200])
    assert n2 >= 2 * 2 * 2 * 200 * 256  # K and V, 2 sequences x 2 KV heads x >= 200 slots x 256 B
    cfg3 = L.make_config(**{**GOOD, "batch": 3})
    assert L.workspace_size(cfg3, [100, 200, 300]) > n2
    paged = L.make_config(**{**GOOD, "page_size": 16, "max_pages": 64})
    assert L.workspace_size(paged, [100, 200]) >= 64 * 2 * 16 * 256 * 2
    with pytest.raises(L.H2OError) as ex:
        L.workspace_size(L.make_config(**{**GOOD, "page_size": 16, "max_pages": 4}), [100, 200])
    assert ex.value.code == L.H2O_ENOMEM
    with pytest.raises(L.H2OError) as ex:
        L.workspace_size(L.make_config(**{**GOOD, "n_q_heads": 7}), [100, 200])
    assert ex.value.code == L.H2O_EINVAL


def test_init_rejects_misaligned_workspace(lib):
    cfg = L.make_config(**GOOD)
    cfg.workspace = 4096 + 128
    cfg.workspace_bytes = 1 << 30
    rc, ctx = _init(lib, cfg, [10, 20])
    assert rc == L.H2O_EINVAL and not ctx.value
    assert "256-byte aligned" in lib.h2o_last_error(None).decode()


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    mod = importlib.import_module("kv_cache_eviction_h2o_amd._lib")
    saved = mod._lib
    try:
        mod._lib = None
        with pytest.raises(RuntimeError, match="missing"):
            mod.load_library(str(tmp_path / "nope.so"))
    finally:
        mod._lib = saved


def test_contiguous_unit_past_32bit_descriptor_rejected(lib):
    """Contiguous units are read through 32-bit buffer descriptors: a unit whose
    K rows reach 2^31 bytes is refused (the paged layout has no such limit)."""
    big = dict(budget_fixed=(1 << 23), hh_fixed=1000, max_len=(1 << 23) + 10)
    rc, ctx = _init(lib, L.make_config(**{**GOOD, **big}), [100, 200])
    assert rc == L.H2O_EINVAL and not ctx.value
    assert "2^31 bytes" in lib.h2o_last_error(None).decode()
    ok = dict(budget_fixed=(1 << 23) - 2, hh_fixed=1000, max_len=(1 << 23) + 10)
    n = C.c_uint64()
    arr = (C.c_int32 * 2)(100, 200)
    assert lib.h2o_workspace_size(C.byref(L.make_config(**{**GOOD, **ok})), arr, C.byref(n)) == L.H2O_OK
    paged = dict(big, page_size=16, max_pages=64)
    assert lib.h2o_workspace_size(C.byref(L.make_config(**{**GOOD, **paged})), arr, C.byref(n)) == L.H2O_OK


def _pool_mirror(w, lens, steps):
    """Sum over sequences of the most pages each holds: ceil(P / 16) after the
    prompt, ceil(n_att / 16) while a step runs (metrics' host mirror)."""
    from kv_cache_eviction_h2o_amd import metrics as M
    tot = 0
    for P in lens:
        n_att = M.retained_counts(w, P, steps)["n_att"]
        tot += max((P + 15) // 16, int(((n_att + 15) // 16).max()) if steps else 0)
    return tot


@pytest.mark.parametrize("selector", ["h2o", "block", "random"])
def test_page_pool_sizing_matches_mirror(lib, selector):
    """h2o_pool_pages equals the sum of each sequence's largest page count under
    the selector's schedule (host mirror in metrics.retained_counts)."""
    from kv_cache_eviction_h2o_amd import workloads as WL
    if selector == "random":
        w = WL.RANDOM_ATTN.scaled(batch=3, n_q_heads=8, n_kv_heads=2, rand_k=64, rand_r=16, page_size=16)
    else:
        w = WL.PAGED_MIXED.scaled(batch=3, n_q_heads=4, n_kv_heads=4, selector=selector)
    lens, steps = [40, 1500, 4097], 300
    cfg = L.config_from_workload(w, max_len=max(lens) + steps + 1, max_pages=1)
    assert L.pages_needed(lens, steps, cfg) == _pool_mirror(w, lens, steps)
    assert L.pages_needed(lens, 0, cfg) == sum((p + 15) // 16 for p in lens)


def test_page_pool_sizing_rejects(lib):
    base = {**GOOD, "budget_fixed": 0, "budget_num": 1, "budget_den": 5, "page_size": 16, "max_len": 5000}
    arr = (C.c_int32 * 2)(100, 200)
    n = C.c_int32()
    assert lib.h2o_pool_pages(C.byref(L.make_config(**{**base, "page_size": 0})), arr, 10, C.byref(n)) == L.H2O_EINVAL
    assert "paged layout" in lib.h2o_last_error(None).decode()
    assert lib.h2o_pool_pages(C.byref(L.make_config(**base)), arr, -1, C.byref(n)) == L.H2O_EINVAL
    assert lib.h2o_pool_pages(C.byref(L.make_config(**base)), arr, 4900, C.byref(n)) == L.H2O_EINVAL
    assert "max_len" in lib.h2o_last_error(None).decode()
    assert lib.h2o_pool_pages(C.byref(L.make_config(**base)), arr, 10, None) == L.H2O_EINVAL
    assert lib.h2o_pool_pages(C.byref(L.make_config(**base)), arr, 10, C.byref(n)) == L.H2O_OK and n.value > 0


def _prefill(lib, cfg, lens, ptr=16):
    arr = (C.c_int32 * len(lens))(*lens)
    p = C.c_void_p(ptr) if ptr else None
    return lib.h2o_prefill_scores(C.byref(cfg), arr, p, p, p, None)


@pytest.mark.parametrize("bad,lens,msg", [
    (dict(), [0, 10], ">= 1"),
    (dict(n_q_heads=7), [10, 10], "multiple"),
    (dict(n_q_heads=32, n_kv_heads=2), [10, 10], "group size"),
    (dict(head_dim=64), [10, 10], "head_dim 128"),
    (dict(kv_dtype="f32"), [10, 10], "bf16"),
    (dict(scale=-1.0), [10, 10], "scale"),
    (dict(batch=129), [10] * 129, "128 sequences"),
])
def test_prefill_scores_rejects_before_device(lib, bad, lens, msg):
    cfg = L.make_config(**{**GOOD, **bad})
    assert _prefill(lib, cfg, lens) == L.H2O_EINVAL
    assert msg in lib.h2o_last_error(None).decode()


def test_prefill_scores_rejects_misaligned_pointers(lib):
    cfg = L.make_config(**GOOD)
    assert _prefill(lib, cfg, [10, 10], ptr=20) == L.H2O_EINVAL
    assert "16-byte aligned" in lib.h2o_last_error(None).decode()


def test_prefill_scores_null_arguments(lib):
    cfg = L.make_config(**GOOD)
    assert lib.h2o_prefill_scores(None, None, None, None, None, None) == L.H2O_EINVAL
    assert _prefill(lib, cfg, [10, 10], ptr=0) == L.H2O_EINVAL
    assert "null" in lib.h2o_last_error(None).decode()


def _snap(lib, cfg, lens, window=32, pool=7, keep=16, cap=4096, ptr=16):
    arr = (C.c_int32 * len(lens))(*lens)
    p = C.c_void_p(ptr) if ptr else None
    return lib.h2o_snapkv_select(C.byref(cfg), arr, window, pool, keep, p, p, None, p, p, cap, None)


@pytest.mark.parametrize("kw,msg", [
    (dict(window=0), "window"),
    (dict(pool=4), "odd"),
    (dict(pool=0), "odd"),
    (dict(keep=-1), "keep"),
    (dict(cap=10), "cap"),
    (dict(ptr=0), "null"),
    (dict(ptr=24), "16-byte aligned"),
])
def test_snapkv_select_rejects_before_device(lib, kw, msg):
    cfg = L.make_config(**GOOD)
    assert _snap(lib, cfg, [100, 200], **kw) == L.H2O_EINVAL
    assert msg in lib.h2o_last_error(None).decode()


def _align256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("B,P,Hq,Hkv", [(8, 16384, 32, 32), (128, 1024, 64, 8)])
def test_snapkv_noalloc_scratch_need_matches_the_header(lib, B, P, Hq, Hkv):
    """h2o_snapkv_select_noalloc refuses, on the host and before any device
    call, a call whose scratch need passes the fixed 64 MiB, and names the
    need: with the votes in scratch it is 8 sum P Hq bytes, plus the per-head
    kept bitmaps for groups, plus -- unless the call runs in one pass (every
    prompt up to 1024 positions, window up to 32) -- the pooled votes and the
    column-sum passes' window q tiles and row statistics (4160 B Hkv G T)."""
    G, w = Hq // Hkv, 32
    cfg = L.make_config(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=128, kv_dtype="bf16",
                        score_dtype="f32", budget_fixed=64, hh_fixed=28, max_len=P + 1)
    arr = (C.c_int32 * B)(*([P] * B))
    p = C.c_void_p(256)  # never touched: the size check comes before anything is enqueued
    rc = lib.h2o_snapkv_select_noalloc(C.byref(cfg), arr, w, 7, 100, p, p, None, p, p, P, None)
    assert rc == L.H2O_EINVAL
    msg = lib.h2o_last_error(None).decode()
    need = _align256(8 * B * P * Hq)  # the votes
    if G > 1:
        need += _align256(4 * B * Hq * ((P + 127) // 128 * 4))
    if P > 1024:
        T = (P + 7) // 8 - (P - w) // 8
        need += _align256(8 * B * P * Hq) + _align256(B * Hkv * T * G * 256 * 16) + _align256(B * Hkv * T * G * 64)
    assert need > 64 << 20 and f"needs {need} bytes" in msg, (need, msg)
