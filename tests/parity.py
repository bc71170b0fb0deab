"""GPU path vs CPU oracle, step by step, on the same seeded inputs.

Acceptance (per step, per checked (sequence, KV head) unit):
* attention output: for each query head, max_d |gpu - oracle| <= 2e-3 * max_d |oracle|;
* retained set: equal to the oracle's, except that a different victim set is
  accepted when it has the same size, only evictable tokens, and every token in
  the symmetric difference has an oracle score within 1e-5 of the oracle's
  e-th smallest candidate score (a near-tie the fp32 path may resolve either
  way); the oracle then adopts the GPU's set so later steps stay comparable.
  Random Attention has no exemption: its sets must be identical;
* cumulative scores of the retained tokens: |gpu - oracle| <= 2e-3 * oracle + 1e-9;
* evicted mass: |gpu - oracle| <= 2e-3 * max(1, oracle);
* binary16 scores (the compressed state): the GPU rounds its fp32 update and
  the oracle its fp64 update, so a stored value may sit one binary16 unit in
  the last place (ulp) away: every score must be within one ulp of the
  oracle's, a different victim set is accepted when every token in the
  symmetric difference lies within two ulps (plus the gap above) of the
  oracle's e-th smallest score, and after each checked step the oracle adopts
  the GPU's stored scores (lockstep, as for adopted victims) so that the next
  step starts from the same state -- the check is then of each step's update
  and selection, which is what a rounded state can be held to;
* stored rows (after the last step): every retained position's K and V row as
  the library holds it equals, bit for bit, the generator's row for that
  position -- its bf16 / fp32 bits, or for int8 storage the oracle's
  quantisation of it (codes and scale).  This pins the compaction: a row moved
  to the wrong slot or half-moved would show here.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass, field

import numpy as np

import oracle as O
from kv_cache_eviction_h2o_amd import synth as S
from kv_cache_eviction_h2o_amd import workloads as WL

OUT_TOL = 2e-3
SCORE_TOL = 2e-3
GAP = 1e-5


def ulp16(x) -> np.ndarray:
    """Spacing of IEEE binary16 values at |x|: 2^(e - 10) for a leading bit 2^e
    (e >= -14), 2^-24 below (subnormals)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return np.ldexp(1.0, (e - 10).astype(np.int64))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_rows(w: WL.Workload, x) -> np.ndarray:
    """The fp64 rows the oracle attends over for generator rows x (recipe dtype):
    the exact values, or for int8 storage their quantise-dequantise image."""
    if w.kv_dtype == "i8":
        x2 = S.bf16_to_f32(np.asarray(x)).reshape(-1, w.head_dim)
        return O.dequantize_rows(*O.quantize_rows(x2)).reshape(np.shape(x))
    return S.cache_to_f64(w.recipe, x)


def to_dev(x, kv_dtype):
    import torch
    if kv_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


@dataclass
class ParityReport:
    steps: int = 0
    units: int = 0
    adopted: int = 0
    max_out_err: float = 0.0
    max_score_err: float = 0.0
    evictions: int = 0
    max_swapped: int = 0
    notes: list = field(default_factory=list)


def make_cache(w: WL.Workload, lens, n_steps: int, layer: int = 0, init_scores=None):
    import torch
    from kv_cache_eviction_h2o_amd import _lib as L
    K, V = S.prompt_kv(w.recipe, layer, lens, w.n_kv_heads)
    max_len = max(lens) + n_steps + 1
    cfg = L.config_from_workload(w, max_len=max_len)
    if w.page_size:
        cfg.max_pages = L.pages_needed(lens, n_steps, cfg)
    isc = None
    if init_scores is not None:
        isc = torch.from_numpy(np.ascontiguousarray(init_scores, dtype=np.float64)).cuda()
    cache = L.H2OCache(cfg, lens, to_dev(K, w.recipe.kv_dtype), to_dev(V, w.recipe.kv_dtype), init_scores=isc)
    return cache, K, V


def _oracle_threads(n_units: int) -> int:
    import os
    return max(1, min(16, os.cpu_count() or 1, n_units))


def run_parity(w: WL.Workload, n_steps: int, *, lens=None, units=None, fused=True, layer=0,
               init_scores=None, read_every=1, check_steps=(), check_scores=True, device_inputs=False,
               stored_rows=True, properties=False, max_swapped=None, zero_q=False) -> ParityReport:
    """Run n_steps on the GPU and in the oracle (for `units`, default all).

    Checked steps: every read_every-th, those in check_steps, and the last.
    device_inputs: prompts and steps drawn on the device (the benchmark's
    generator, for full-size batches); the checked units' rows are copied back
    for the oracle, and reads are sized by the host mirror of the counts.
    stored_rows: check the stored rows of the checked units at the end.
    properties: after the last step, check every unit for what holds at any
    size (h2o_properties).
    max_swapped: at most this many tokens of a unit-step may differ from the
    oracle's victims under the near-tie rule (a check stricter than the rule:
    when scores are far below the absolute gap, as after the bulk first step of
    long prompts, the rule alone would accept any candidate).
    zero_q: every decode query is zero, so every step weighs its slots equally
    and tokens present over the same steps hold exactly equal scores (the
    tie rule decides).
    The oracle steps its units on POSIX threads (orc_step_many) between checked
    steps, and attends them on a thread pool at checked steps."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    lens = list(lens) if lens is not None else WL.prompt_lengths(w)
    B, Hq, Hkv, G, D = w.batch, w.n_q_heads, w.n_kv_heads, w.group, w.head_dim
    assert len(lens) == B
    say(f"[parity] {w.name} B={B} Hq={Hq} Hkv={Hkv} D={D} lens={lens[:6]}{'...' if B > 6 else ''} "
        f"steps={n_steps} fused={fused} units={'all' if units is None else len(units)}")
    off = np.concatenate([[0], np.cumsum(lens)])
    units = [(b, h) for b in range(B) for h in range(Hkv)] if units is None else list(units)
    assert not (zero_q and device_inputs)
    if device_inputs:
        from kv_cache_eviction_h2o_amd import _lib as L
        from kv_cache_eviction_h2o_amd import metrics as M
        assert init_scores is None
        pk, pv = S.device_prompt_kv(w.recipe, layer, lens, Hkv)
        cfg = L.config_from_workload(w, max_len=max(lens) + n_steps + 1)
        if w.page_size:
            cfg.max_pages = L.pages_needed(lens, n_steps, cfg)
        cache = L.H2OCache(cfg, lens, pk, pv)
        seqs = sorted({b for b, _ in units})
        K = _Rows(off, {b: _host_bits(pk[off[b]:off[b + 1]]) for b in seqs})
        V = _Rows(off, {b: _host_bits(pv[off[b]:off[b + 1]]) for b in seqs})
        del pk, pv
        cap = int(max(M.retained_counts(w, P, n_steps)["count"].max() for P in lens))
    else:
        cache, K, V = make_cache(w, lens, n_steps, layer, init_scores)
        cap = cache.info()[0]
    ocfg = O.cfg_from_workload(w)
    orc = {}
    for (b, h) in units:
        isc = None if init_scores is None else init_scores[off[b]:off[b + 1], h]
        orc[(b, h)] = O.Unit(ocfg, b, h, oracle_rows(w, K[off[b]:off[b + 1], h]),
                             oracle_rows(w, V[off[b]:off[b + 1], h]),
                             lens[b] + n_steps + 1, init_scores=isc)
    rep = ParityReport(units=len(units))
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    win = 256
    gen_k, gen_v = [], []  # generated rows of the decode steps, for the stored-row check
    check_steps = set(check_steps)
    f16 = w.score_dtype == "f16" and w.selector == "h2o"
    assert not f16 or read_every == 1, "binary16 scores are checked in lockstep: every step"
    nthr = _oracle_threads(len(units))
    pool = ThreadPoolExecutor(nthr)
    ulist = [orc[bh] for bh in units]
    for s0 in range(0, n_steps, win):
        ns = min(win, n_steps - s0)
        t0 = [p + s0 for p in lens]
        if device_inputs:
            qd, kd, vd = S.device_step_window(w.recipe, layer, t0, ns, Hq, Hkv)
            q, k, v = qd.cpu().numpy(), _host_bits(kd), _host_bits(vd)
        else:
            q, k, v = S.step_window(w.recipe, layer, t0, ns, Hq, Hkv)
            if zero_q:
                q = np.zeros_like(q)
            qd = torch.from_numpy(q).cuda()
            kd, vd = to_dev(k, w.recipe.kv_dtype), to_dev(v, w.recipe.kv_dtype)
        gen_k.append(k)
        gen_v.append(v)
        for i in range(ns):
            s = s0 + i
            if fused:
                cache.step_compact(qd[i], kd[i], vd[i], out)
            else:
                cache.step(qd[i], kd[i], vd[i], out)
                cache.compact()
            check = (s % read_every == 0) or s in check_steps or s == n_steps - 1
            if not check:
                # the oracle still has to take the step (its own choice)
                O.step_many(ulist, [q[i, b, h * G:(h + 1) * G] for (b, h) in units],
                            [oracle_rows(w, k[i, b, h]) for (b, h) in units],
                            [oracle_rows(w, v[i, b, h]) for (b, h) in units], nthr)
                continue
            o_gpu = out.cpu().numpy()
            pos, cnt, sc, em = cache.read_indices(cap)
            o_refs = list(pool.map(lambda bh: orc[bh].attend(q[i, bh[0], bh[1] * G:(bh[1] + 1) * G],
                                                             oracle_rows(w, k[i, bh[0], bh[1]]),
                                                             oracle_rows(w, v[i, bh[0], bh[1]])), units))
            for ui, (b, h) in enumerate(units):
                u = orc[(b, h)]
                o_ref = o_refs[ui]
                og = o_gpu[b, h * G:(h + 1) * G].astype(np.float64)
                err = np.max(np.abs(og - o_ref), axis=1) / np.maximum(np.max(np.abs(o_ref), axis=1), 1e-30)
                rep.max_out_err = max(rep.max_out_err, float(err.max()))
                assert np.all(err <= OUT_TOL), f"step {s} unit {(b, h)}: output rel err {err.max():.3g}"
                pre_pos, _, _ = u.state()
                vic, tau = u.select()
                n = int(cnt[b])
                gpos = pos[b, h, :n]
                gset = set(gpos.tolist())
                assert gset <= set(pre_pos.tolist()), f"step {s} unit {(b, h)}: GPU retains unknown positions"
                gvic = sorted(set(pre_pos.tolist()) - gset)
                if sorted(vic.tolist()) != gvic:
                    diff = set(vic.tolist()) ^ set(gvic)
                    gap = GAP + (2 * float(ulp16(tau)) if f16 else 0.0)
                    ok = (w.selector == "h2o" and len(gvic) == len(vic)
                          and all(abs(u.score_of(p) - tau) < gap for p in diff))
                    assert ok, (f"step {s} unit {(b, h)}: victims differ: oracle-only "
                                f"{sorted(set(vic.tolist()) - set(gvic))[:8]} gpu-only "
                                f"{sorted(set(gvic) - set(vic.tolist()))[:8]} tau={tau}")
                    assert max_swapped is None or len(diff) // 2 <= max_swapped, \
                        f"step {s} unit {(b, h)}: {len(diff) // 2} victims swapped under the near-tie rule"
                    rep.max_swapped = max(rep.max_swapped, len(diff) // 2)
                    u.evict(np.array(gvic, dtype=np.int32))
                    rep.adopted += 1
                else:
                    u.evict(vic)
                u.check()
                rep.evictions += len(gvic)
                o_pos, o_sc, o_em = u.state()
                assert np.array_equal(o_pos, gpos), f"step {s} unit {(b, h)}: retained sets differ"
                if check_scores and w.selector == "h2o":
                    g_sc = sc[b, h, :n]
                    serr = np.abs(g_sc - o_sc)
                    if f16:
                        assert np.all(serr <= ulp16(o_sc) * (1 + 1e-12)), \
                            f"step {s} unit {(b, h)}: binary16 scores more than one ulp apart"
                        assert np.array_equal(g_sc, g_sc.astype(np.float16).astype(np.float64)), \
                            f"step {s} unit {(b, h)}: stored scores are not binary16 values"
                    assert np.all(serr <= SCORE_TOL * np.abs(o_sc) + 1e-9), \
                        f"step {s} unit {(b, h)}: score err {np.max(serr / (np.abs(o_sc) + 1e-9)):.3g}"
                    rep.max_score_err = max(rep.max_score_err,
                                            float(np.max(serr / np.maximum(np.abs(o_sc), 1e-30))))
                    assert abs(em[b, h] - o_em) <= SCORE_TOL * max(1.0, o_em), \
                        f"step {s} unit {(b, h)}: evicted mass {em[b, h]} vs {o_em}"
                if f16:  # lockstep: the next step starts from the GPU's stored scores
                    u.set_scores(gpos, sc[b, h, :n])
            rep.steps += 1
    pool.shutdown()
    if stored_rows:
        check_stored_rows(w, cache, units, lens, K, V, gen_k, gen_v, cap=cap)
    if properties:
        h2o_properties(w, cache, lens, n_steps, cap=cap)
    cache.close()
    say(f"[parity] ok: checked {rep.steps} steps x {rep.units} units, max out err "
        f"{rep.max_out_err:.2e}, max score err {rep.max_score_err:.2e}, evictions {rep.evictions}, "
        f"near-ties adopted {rep.adopted} (most tokens swapped in one: {rep.max_swapped})")
    return rep


def check_stored_rows(w, cache, units, lens, K, V, gen_k, gen_v, cap=None):
    """The library's stored rows of every retained position against the generator."""
    pos, cnt, _, _ = cache.read_indices(cap)
    kr, vr, ks, vs = cache.read_kv(cap)
    off = np.concatenate([[0], np.cumsum(lens)])
    gk = np.concatenate(gen_k) if gen_k else None  # [steps][B][Hkv][D]
    gv = np.concatenate(gen_v) if gen_v else None
    for (b, h) in units:
        n = int(cnt[b])
        for i, p in enumerate(pos[b, h, :n]):
            P = lens[b]
            kx = K[off[b] + p, h] if p < P else gk[p - P, b, h]
            vx = V[off[b] + p, h] if p < P else gv[p - P, b, h]
            if w.kv_dtype == "i8":
                for x, rows, sc, name in ((kx, kr, ks, "K"), (vx, vr, vs, "V")):
                    codes, scale = O.quantize_rows(S.bf16_to_f32(x).reshape(1, -1))
                    assert np.array_equal(rows[b, h, i], codes[0]), f"unit {(b, h)} pos {p}: stored {name} codes"
                    assert sc[b, h, i] == scale[0], f"unit {(b, h)} pos {p}: stored {name} scale"
            else:
                assert np.array_equal(kr[b, h, i], kx), f"unit {(b, h)} pos {p}: stored K row"
                assert np.array_equal(vr[b, h, i], vx), f"unit {(b, h)} pos {p}: stored V row"


def run_block_parity(w: WL.Workload, n_steps: int, *, lens=None, seqs=None, fused=True, layer=0,
                     init_scores=None, read_every=1, check_scores=True, device_inputs=False,
                     stored_rows=True) -> ParityReport:
    """Block-granular eviction: GPU path vs oracle for whole sequences (every KV
    head of each checked sequence, since the pages that go depend on all of
    them).  Per checked step and sequence: outputs, retained positions (the
    same for every head, whole pages), scores and evicted mass as in
    run_parity.  The GPU's victim pages must be the oracle's; unfused runs also
    read the step's pending state (after the append, before any page goes) and
    check it against the oracle, and a different page choice is accepted only
    when the oracle's rule applied to the GPU's own pre-eviction scores picks
    exactly the GPU's pages (a near-tie that fp32 scores resolve the other way);
    the oracle then adopts them.

    device_inputs: prompts and steps drawn on the device (the benchmark's
    generator, for full-size batches); the checked sequences' rows are copied
    back for the oracle.  The cache is left open in the report (rep.cache) for
    further checks; the caller closes it."""
    import torch
    from kv_cache_eviction_h2o_amd import metrics as M
    assert w.selector == "block" and w.page_size == 16
    lens = list(lens) if lens is not None else WL.prompt_lengths(w)
    B, Hq, Hkv, G, D = w.batch, w.n_q_heads, w.n_kv_heads, w.group, w.head_dim
    assert len(lens) == B
    seqs = list(range(B)) if seqs is None else list(seqs)
    say(f"[block parity] {w.name} B={B} Hq={Hq} Hkv={Hkv} lens={lens[:6]}{'...' if B > 6 else ''} "
        f"steps={n_steps} fused={fused} seqs={seqs if len(seqs) <= 8 else len(seqs)}")
    off = np.concatenate([[0], np.cumsum(lens)])
    if device_inputs:
        from kv_cache_eviction_h2o_amd import _lib as L
        pk, pv = S.device_prompt_kv(w.recipe, layer, lens, Hkv)
        cfg = L.config_from_workload(w, max_len=max(lens) + n_steps + 1)
        cfg.max_pages = L.pages_needed(lens, n_steps, cfg)
        cache = L.H2OCache(cfg, lens, pk, pv)
        K = _Rows(off, {b: _host_bits(pk[off[b]:off[b + 1]]) for b in seqs})
        V = _Rows(off, {b: _host_bits(pv[off[b]:off[b + 1]]) for b in seqs})
        del pk, pv
    else:
        cache, K, V = make_cache(w, lens, n_steps, layer, init_scores)
    units = [(b, h) for b in seqs for h in range(Hkv)]
    ocfg = O.cfg_from_workload(w)
    orc = {}
    for (b, h) in units:
        isc = None if init_scores is None else init_scores[off[b]:off[b + 1], h]
        orc[(b, h)] = O.Unit(ocfg, b, h, oracle_rows(w, K[off[b]:off[b + 1], h]),
                             oracle_rows(w, V[off[b]:off[b + 1], h]),
                             lens[b] + n_steps + 1, init_scores=isc)
    rep = ParityReport(units=len(units))
    # reads sized by the host mirror of the counts (the library rejects a short cap)
    mirror = [M.retained_counts(w, P, n_steps) for P in lens]
    cap = int(max(c["count"].max() for c in mirror))
    cap_pre = int(max(c["n_att"].max() for c in mirror))
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    win = 256
    gen_k, gen_v = [], []
    for s0 in range(0, n_steps, win):
        ns = min(win, n_steps - s0)
        t0 = [p + s0 for p in lens]
        if device_inputs:
            qd, kd, vd = S.device_step_window(w.recipe, layer, t0, ns, Hq, Hkv)
            q, k, v = qd.cpu().numpy(), _host_bits(kd), _host_bits(vd)
        else:
            q, k, v = S.step_window(w.recipe, layer, t0, ns, Hq, Hkv)
            qd = torch.from_numpy(q).cuda()
            kd, vd = to_dev(k, w.recipe.kv_dtype), to_dev(v, w.recipe.kv_dtype)
        gen_k.append(k)
        gen_v.append(v)
        for i in range(ns):
            s = s0 + i
            check = (s % read_every == 0) or s == n_steps - 1
            pre = None
            if fused:
                cache.step_compact(qd[i], kd[i], vd[i], out)
            else:
                cache.step(qd[i], kd[i], vd[i], out)
                if check:
                    pre = cache.read_indices(cap_pre)
                cache.compact()
            if not check:
                for (b, h) in units:
                    orc[(b, h)].attend(q[i, b, h * G:(h + 1) * G], oracle_rows(w, k[i, b, h]),
                                       oracle_rows(w, v[i, b, h]))
                for b in seqs:
                    us = [orc[(b, h)] for h in range(Hkv)]
                    vic = O.block_select(us, page=16)
                    for u in us:
                        u.evict(vic)
                continue
            o_gpu = out.cpu().numpy()
            pos, cnt, sc, em = cache.read_indices(cap)
            for (b, h) in units:
                u = orc[(b, h)]
                o_ref = u.attend(q[i, b, h * G:(h + 1) * G], oracle_rows(w, k[i, b, h]),
                                 oracle_rows(w, v[i, b, h]))
                og = o_gpu[b, h * G:(h + 1) * G].astype(np.float64)
                err = np.max(np.abs(og - o_ref), axis=1) / np.maximum(np.max(np.abs(o_ref), axis=1), 1e-30)
                rep.max_out_err = max(rep.max_out_err, float(err.max()))
                assert np.all(err <= OUT_TOL), f"step {s} unit {(b, h)}: output rel err {err.max():.3g}"
            for b in seqs:
                us = [orc[(b, h)] for h in range(Hkv)]
                length = lens[b] + s + 1
                pre_pos = us[0].state()[0]
                if pre is not None:  # the pending state: the append done, no page gone yet
                    ppos, pcnt, psc, _ = pre
                    npre = int(pcnt[b])
                    for h, u in enumerate(us):
                        o_pos, o_sc, _ = u.state()
                        assert np.array_equal(ppos[b, h, :npre], o_pos), f"step {s} seq {b} head {h}: pending set"
                        if check_scores:
                            serr = np.abs(psc[b, h, :npre] - o_sc)
                            assert np.all(serr <= SCORE_TOL * np.abs(o_sc) + 1e-9), \
                                f"step {s} seq {b} head {h}: pending score err"
                n = int(cnt[b])
                gpos = pos[b, 0, :n]
                for h in range(1, Hkv):
                    assert np.array_equal(pos[b, h, :n], gpos), f"step {s} seq {b}: heads retain different sets"
                assert set(gpos.tolist()) <= set(pre_pos.tolist()), f"step {s} seq {b}: unknown positions"
                gvic = sorted(set(pre_pos.tolist()) - set(gpos.tolist()))
                ovic = O.block_select(us, page=16)
                if list(ovic) != gvic:
                    assert pre is not None, (
                        f"step {s} seq {b}: victim pages differ (fused run; oracle "
                        f"{sorted(set(np.asarray(ovic) // 16))[:8]} gpu {sorted(set(np.asarray(gvic) // 16))[:8]})")
                    ppos, pcnt, psc, _ = pre
                    npre = int(pcnt[b])
                    live = np.zeros(length, dtype=np.uint8)
                    live[ppos[b, 0, :npre]] = 1
                    gsc = np.zeros((Hkv, length))
                    for h in range(Hkv):
                        gsc[h, ppos[b, h, :npre]] = psc[b, h, :npre]
                    replay = O.block_rank(ocfg, length, live, gsc, page=16)
                    assert list(replay) == gvic, (f"step {s} seq {b}: GPU pages are not the rule's choice "
                                                  f"on its own scores")
                    vic = np.array(gvic, dtype=np.int32)
                    rep.adopted += 1
                else:
                    vic = ovic
                for h, u in enumerate(us):
                    u.evict(vic)
                    u.check()
                    o_pos, o_sc, o_em = u.state()
                    assert np.array_equal(o_pos, pos[b, h, :n]), f"step {s} seq {b} head {h}: retained sets differ"
                    if check_scores:
                        serr = np.abs(sc[b, h, :n] - o_sc)
                        assert np.all(serr <= SCORE_TOL * np.abs(o_sc) + 1e-9), \
                            f"step {s} seq {b} head {h}: score err {np.max(serr / (np.abs(o_sc) + 1e-9)):.3g}"
                        rep.max_score_err = max(rep.max_score_err,
                                                float(np.max(serr / np.maximum(np.abs(o_sc), 1e-30))))
                        assert abs(em[b, h] - o_em) <= SCORE_TOL * max(1.0, o_em), \
                            f"step {s} seq {b} head {h}: evicted mass {em[b, h]} vs {o_em}"
                rep.evictions += len(gvic) * Hkv
            rep.steps += 1
    if stored_rows:
        check_stored_rows(w, cache, units, lens, K, V, gen_k, gen_v, cap=cap)
    rep.cache = cache
    say(f"[block parity] ok: checked {rep.steps} steps x {len(seqs)} sequences, max out err "
        f"{rep.max_out_err:.2e}, max score err {rep.max_score_err:.2e}, evicted tokens x heads "
        f"{rep.evictions}, near-ties adopted {rep.adopted}")
    return rep


class _Rows:
    """Packed prompt rows [sum P_b][Hkv][D] of a few sequences (the rest absent),
    indexed like the full array."""

    def __init__(self, off, parts):
        self.off, self.parts = off, parts

    def __getitem__(self, idx):
        r, h = idx
        if isinstance(r, slice):
            b = int(np.searchsorted(self.off, r.start, side="right") - 1)
            assert r.stop == self.off[b + 1]
            return self.parts[b][:, h]
        b = int(np.searchsorted(self.off, r, side="right") - 1)
        return self.parts[b][r - self.off[b], h]


def _host_bits(t):
    """A bf16 / fp32 device tensor as host cache-dtype values (bf16 as uint16 bits)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def h2o_properties(w: WL.Workload, cache, lens, steps_done: int, cap=None):
    """What holds for every (sequence, KV head) unit after steps_done steps of
    token-level H2O with no initial scores, at any size: the count is the host
    mirror's min(n_att, K_t) at every step; positions are ascending, distinct
    and before the sequence's length; the sinks and the recent window are all
    retained; and retained scores plus evicted mass equal G x steps_done (each
    query head's softmax adds a total weight of 1 per step)."""
    from kv_cache_eviction_h2o_amd import metrics as M
    assert w.selector == "h2o"
    pos, cnt, sc, em = cache.read_indices(cap)
    ocfg = O.cfg_from_workload(w)
    for b in range(w.batch):
        length = lens[b] + steps_done
        n = int(cnt[b])
        assert n == int(M.retained_counts(w, lens[b], steps_done)["count"][-1]), f"seq {b}: count {n}"
        _, _, W = O.schedule(ocfg, length)
        p = pos[b, :, :n].astype(np.int64)  # [Hkv][n]
        assert np.all(np.diff(p, axis=1) > 0), f"seq {b}: positions not ascending"
        assert p.min() >= 0 and p.max() < length, f"seq {b}: position out of range"
        ns = min(w.n_sink, length)
        assert np.all(p[:, :ns] == np.arange(ns)), f"seq {b}: a sink is missing"
        nw = min(W, length)
        assert nw == 0 or np.all(p[:, n - nw:] == np.arange(length - nw, length)), f"seq {b}: window incomplete"
        mass = sc[b, :, :n].sum(axis=1) + em[b]
        want = float(w.group * steps_done)
        assert np.all(np.abs(mass - want) <= 1e-4 * want), f"seq {b}: mass {mass.min()}..{mass.max()}, want {want}"
    say(f"[parity] properties ok for {w.batch} x {w.n_kv_heads} units after {steps_done} steps")


def block_properties(w: WL.Workload, cache, lens, steps_done: int, cap=None):
    """What holds for every sequence after any step of block eviction, at any
    size: every head retains the same positions; they are whole 16-position
    pages (the last may be partial); the sinks and the recent window are all
    retained; and the count is <= K_t unless no candidate page is left."""
    pos, cnt, _, _ = cache.read_indices(cap)
    ocfg = O.cfg_from_workload(w)
    for b in range(w.batch):
        n = int(cnt[b])
        length = lens[b] + steps_done
        p = pos[b, 0, :n]
        assert all(np.array_equal(pos[b, h, :n], p) for h in range(w.n_kv_heads)), f"seq {b}: head sets differ"
        K, HH, W = O.schedule(ocfg, length)
        pages = p // 16
        up, c = np.unique(pages, return_counts=True)
        last = p[n - c[-1]:]
        assert np.all(c[:-1] == 16) and np.array_equal(last, up[-1] * 16 + np.arange(c[-1])), \
            f"seq {b}: a page is not whole"
        assert set(range(min(w.n_sink, length))) <= set(p.tolist()), f"seq {b}: a sink is gone"
        assert set(range(max(0, length - W), length)) <= set(p.tolist()), f"seq {b}: the window is not whole"
        cands = [k for k in up if k * 16 >= w.n_sink and k * 16 + 15 < length - W]
        assert n <= K or not cands, f"seq {b}: {n} > K = {K} with {len(cands)} candidate pages"
