#!/usr/bin/env python3
"""Benchmark of the H2O decode step (attention + evict + compact) on one MI355X.

Default workload: the paged mixed-length batch -- 64 sequences with prompts
uniform on [4096, 65536] tokens, 32 heads x 128, bf16 K/V in 16-token pages
with a block table, fp32 cumulative scores, 4 sinks and a budget of 20 % of the
current length split between heavy hitters and the recent window (the largest
single-GPU workload: ~2.2 M prompt tokens, ~36 GB of prompt K/V).  Its first
decode step bulk-evicts every sequence from its prompt to the budget and frees
~80 % of the pages; it runs untimed, then the warm-up steps, then the timed
window of steady steps (one eviction per sequence and head on four of every
five steps).  Other workloads (--workload): the OPT-6.7B layer stepped through
32 layer instances, the LLaMA-2-70B GQA layer through 80, Random Attention, the
tiny correctness workload, int8 rows and block eviction; the steps before each
one's window are run untimed to reach its state.

Metric: retained KV tokens processed per second (a retained token counts once
per sequence per layer-step), with the step's algorithmic bytes as a fraction
of the 8 TB/s HBM peak.  `roofline` reports the step kernel alone: algorithmic
bytes per launch over its mean duration, timed with HIP events recorded on the
launch stream around every decode step of the timed region (each step is the
layers' launches back to back, so this per-launch time includes the short
dispatch gap between launches).  `cpu_baseline` times
the fp64 CPU oracle on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from kv_cache_eviction_h2o_amd import metrics as M  # noqa: E402
from kv_cache_eviction_h2o_amd import synth as S  # noqa: E402
from kv_cache_eviction_h2o_amd import workloads as WL  # noqa: E402

METRIC = "retained KV tokens processed/sec per decode step (attn+evict+compact); % HBM peak"
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "kv_cache_eviction_h2o_amd", "csrc")
# device sources of the decode-step kernels, and of the prompt calls' kernels
STEP_SRCS = ("h2o_internal.h", "h2o_device.h", "h2o_step.h", "h2o_step_f32.hip", "h2o_step_f64.hip",
             "h2o_step_f16.hip", "h2o_kernels.hip", "h2o_mfma.hip", "h2o_block.hip")
PROMPT_SRCS = ("h2o_internal.h", "h2o_device.h", "h2o_prefill.hip")
PROMPT_KERNELS = ("colsum_", "snapkv_")
PROFILES = os.path.join(ROOT, "profiles")


def summarize(args) -> None:
    """Summary of rocprofv3 CSV output for one kernel (default: the step kernel; see --help)."""
    import csv
    line = None
    if args.summarize_bench_line:  # the JSON line the profiled run printed: its window and bytes
        with open(args.summarize_bench_line) as f:
            line = json.loads([x for x in f.read().splitlines() if x.startswith("{")][-1])
        n_last = line["steps"] * line["config"].get("layers", 1)
    else:
        if args.steps is None:
            raise SystemExit("--summarize-* needs --steps (and --layers) or --summarize-bench-line")
        n_last = args.steps * (args.layers or 1)
    kname = args.summarize_kernel
    out = [f"kernel_source_sha256_16: {kernel_hash(prompt=kname.startswith(PROMPT_KERNELS))}"]
    if args.summarize_trace:
        rows = [r for r in csv.DictReader(open(args.summarize_trace)) if kname in r["Kernel_Name"]]
        d = np.array([int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows], dtype=np.float64)
        s0 = np.array([int(r["Start_Timestamp"]) for r in rows], dtype=np.int64)
        e0 = np.array([int(r["End_Timestamp"]) for r in rows], dtype=np.int64)
        w = d[-n_last:]
        gaps = (s0[-n_last + 1:] - e0[-n_last:-1]) / 1e3
        out += [f"{kname} launches in trace: {len(d)}",
                f"all launches: mean {d.mean() / 1e3:.3f} us",
                f"timed window (last {n_last} launches): mean {w.mean() / 1e3:.3f} us, "
                f"median {np.median(w) / 1e3:.3f} us, p10 {np.percentile(w, 10) / 1e3:.3f} us, "
                f"p90 {np.percentile(w, 90) / 1e3:.3f} us",
                f"timed window gap between consecutive launches: mean {gaps.mean():.3f} us"]
    if args.summarize_counters:
        fetch_csv, write_csv = args.summarize_counters
        res = {}
        for name, f in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
            rows = list(csv.DictReader(open(f)))
            st = [float(r["Counter_Value"]) for r in rows if kname in r["Kernel_Name"]
                  and r["Counter_Name"] == name]
            cal = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]
                      and r["Counter_Name"] == name)
            factor = (1 << 20) / cal  # KiB that a 1 GiB device-to-device copy moves, per side
            res[name] = (np.mean(st[-n_last:]), factor, cal)
            out.append(f"{name}: timed-window mean {res[name][0]:.1f} KiB per launch; the 1 GiB "
                       f"copy reads {cal:.1f} KiB on this counter -> scale x{factor:.4f}")
        hbm = sum(v * f * 1024 for v, f, _ in res.values())
        out.append(f"hbm_bytes_per_launch: {hbm:.6e}")
        if line is not None and line.get("algorithmic_bytes_per_launch"):
            alg = line["algorithmic_bytes_per_launch"]
            out += [f"workload: {line['config']['workload']}",
                    f"window_steps: {json.dumps(line['config']['window_steps'])}",
                    f"algorithmic_bytes_per_launch: {alg:.6e}",
                    f"measured / algorithmic: {hbm / alg:.4f}"]
    if args.summarize_pmc:
        by = {}
        for r in csv.DictReader(open(args.summarize_pmc)):
            if kname in r["Kernel_Name"]:
                by.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        mean = {k: float(np.mean(v[-n_last:])) for k, v in by.items()}
        for k in sorted(mean):
            out.append(f"{k}: timed-window mean {mean[k]:.6g} per launch ({len(by[k])} launches)")
        wc = mean.get("SQ_WAVE_CYCLES")
        for k in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VMEM",
                  "SQ_ACTIVE_INST_VALU"):
            if wc and k in mean:
                out.append(f"{k} / SQ_WAVE_CYCLES: {mean[k] / wc:.3f}")
    print("\n".join(out))


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="print a summary of a rocprofv3 kernel trace of this benchmark and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="with FETCH_SIZE / WRITE_SIZE counter CSVs: HBM bytes per launch")
    ap.add_argument("--summarize-pmc", metavar="COUNTER_CSV",
                    help="with a rocprofv3 --pmc counter CSV: each counter's mean per launch")
    ap.add_argument("--summarize-bench-line", metavar="JSON_LINE_FILE",
                    help="the output of the profiled bench run: its timed window (steps x layers "
                         "launches at the end of the trace) and algorithmic bytes per launch")
    ap.add_argument("--summarize-kernel", default="step_kernel", metavar="NAME",
                    help="kernel the summaries cover (a substring of its name; the timed window is "
                         "the last steps x layers of its launches)")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: per workload)")
    ap.add_argument("--warmup", type=int, default=None, help="warm-up steps (default: per workload)")
    ap.add_argument("--workload", default=WL.PAGED_MIXED.name,
                    choices=[w.name for w in WL.ALL + WL.VARIANTS])
    ap.add_argument("--layers", type=int, default=0, help="layer instances (0 = workload default)")
    ap.add_argument("--window-start", type=int, default=None,
                    help="decode step at which the timed window starts (default: per workload; the "
                         "paged workloads start right after the bulk first step and the warm-up)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--events", choices=["step", "launch", "none"], default="step",
                    help="HIP events around every decode step (default: its layer launches run "
                         "back to back, so the per-launch time is the step time over the layers, "
                         "dispatch gaps included), around every launch (markers between kernels "
                         "slow the step), or none")
    ap.add_argument("--prefill", action="store_true",
                    help="time h2o_prefill_scores (prefill-scored initial scores) over the "
                         "workload's prompts instead of the decode step")
    ap.add_argument("--snapkv", action="store_true",
                    help="time h2o_snapkv_select (window 32, pooling 7, 20%% of each prompt kept per "
                         "query head) over the workload's prompts instead of the decode step")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    return ap.parse_args()


class HipEvents:
    """Timing events straight from the HIP runtime, created without the
    system-scope fence so a marker between two kernels does not write back L2."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.lib = C.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        self.lib.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.lib.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self):
        e = C.c_void_p()
        if self.lib.hipEventCreateWithFlags(C.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e

    def record(self, e, stream):
        if self.lib.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_s(self, e0, e1) -> float:
        ms = C.c_float()
        if self.lib.hipEventElapsedTime(C.byref(ms), e0, e1) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value * 1e-3

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


def kernel_hash(prompt: bool = False) -> str:
    """Hash of the device sources the decode-step kernels (or, with prompt, the
    prompt calls' kernels) are built from: a summary is valid for this value only."""
    h = hashlib.sha256()
    for name in PROMPT_SRCS if prompt else STEP_SRCS:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# Timed window of each workload when the command line names none: (steps,
# warm-up steps, first timed step or None = the bulk first step, then the
# warm-up).  OPT layer: steps 512-767 of its 1024-step trace; GQA layer: its
# steady state (every step attends 1029 slots and evicts one from step 4 on);
# Random Attention: a window holding two eviction events (steps 2303, 2431).
WINDOWS = {
    WL.TINY_H2O.name: (64, 16, 128),
    WL.OPT_LAYER.name: (256, 16, 512),
    WL.OPT_LAYER_I8.name: (256, 16, 512),
    WL.OPT_LAYER_F16.name: (256, 16, 512),
    WL.LLAMA_GQA.name: (256, 16, 16),
    WL.RANDOM_ATTN.name: (256, 16, 2176),
    WL.PAGED_MIXED.name: (60, 4, None),
    WL.PAGED_BLOCK.name: (60, 4, None),
}


def bench_window(w, steps=None, warmup=None, start=None):
    """(timed steps K, warm-up W, first timed step s0) for a workload: the
    command line's values where given, else the workload's defaults.  The steps
    before s0 run untimed (the last W of them are the warm-up); contiguous
    workloads keep the window inside their trace, the paged ones may run past
    their 65 nominal steps (the budget rule goes on)."""
    K0, W0, S0 = WINDOWS[w.name]
    K = K0 if steps is None else steps
    W = W0 if warmup is None else warmup
    s0 = start if start is not None else (S0 if S0 is not None else 1 + W)
    if not w.page_size:
        s0 = min(s0, w.decode_steps - K)
    if s0 < W or K < 1 or W < 0:
        raise SystemExit("window does not fit the trace: lower --steps or --warmup")
    return K, W, s0


def step_kernel_name(w) -> str:
    """The step kernel the library launches for a workload: GQA groups of 4 or 8
    over bf16 rows of 128 in contiguous slots run on the matrix cores."""
    if w.kv_dtype == "bf16" and w.head_dim == 128 and not w.page_size and w.group in (4, 8):
        return "mfma_step_kernel"
    return "step_kernel"


def retained_schedule(w, P: int, n_steps: int):
    """n_att (slots attended) at each decode step for one sequence with prompt P
    (the host mirror of the budget rule in metrics.retained_counts)."""
    return M.retained_counts(w, P, n_steps)["n_att"]


def traffic_from_profiles(w, alg_bytes: float):
    """Measured HBM bytes per launch for this line, from a committed counter
    summary taken on the current kernel source (else None).  The summary holds
    the counters' bytes per launch and the algorithmic bytes per launch of the
    window it was taken over; the line's own window gets the same ratio of
    measured to algorithmic bytes, applied to its algorithmic bytes."""
    path = os.path.join(PROFILES, f"h2o_{step_kernel_name(w)}_{w.name}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    a = re.search(r"algorithmic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    win = re.search(r"window_steps:\s*(\[[0-9, ]+\])", text)
    if not m or not t or m.group(1) != kernel_hash():
        return None
    hbm = float(t.group(1))
    if not a:
        return {"bytes": hbm, "ratio": None, "window": None}
    ratio = hbm / float(a.group(1))
    return {"bytes": ratio * alg_bytes, "ratio": ratio, "window": json.loads(win.group(1)) if win else None}


def cpu_baseline(w, n_att: int, seconds: float, max_slots: int = 600_000):
    """The fp64 oracle (as it stands) on a bounded sample of one layer of the
    workload at the window's retained length: as many whole sequences (every KV
    head) as keep the sample within max_slots retained slots, all host cores
    for about `seconds`, then one core for a third of that."""
    import oracle as O
    B, Hkv, Hq, G, D = w.batch, w.n_kv_heads, w.n_q_heads, w.group, w.head_dim
    K = n_att - 1  # fixed budget: every step attends n_att slots and evicts one
    ws = w.scaled(budget_fixed=K, hh_fixed=(K - w.n_sink) // 2)
    nseq = max(1, min(B, max_slots // max(1, Hkv * n_att)))
    lens = [K] * nseq
    Kp, Vp = S.prompt_kv(w.recipe, 0, lens, Hkv)
    cfg = O.cfg_from_workload(ws)
    max_steps = 4096  # positions the oracle units hold: 3072 for the all-core run, the rest for one core
    units = []
    for b in range(nseq):
        for h in range(Hkv):
            units.append(O.Unit(cfg, b, h, S.cache_to_f64(w.recipe, Kp[b * K:(b + 1) * K, h]),
                                S.cache_to_f64(w.recipe, Vp[b * K:(b + 1) * K, h]), K + max_steps + 1))
    del Kp, Vp
    threads = min(os.cpu_count() or 1, len(units))
    block = w.selector == "block"
    done = 0
    win = 32

    def run(nthreads, budget, last_step):
        nonlocal done
        t_used, tokens = 0.0, 0
        while t_used < budget and done < last_step:
            q, k, v = S.step_window(w.recipe, 0, [K + done] * nseq, win, Hq, Hkv)
            for i in range(win):
                qs = [np.ascontiguousarray(q[i, b, h * G:(h + 1) * G], np.float64)
                      for b in range(nseq) for h in range(Hkv)]
                ks = [S.cache_to_f64(w.recipe, k[i, b, h]) for b in range(nseq) for h in range(Hkv)]
                vs = [S.cache_to_f64(w.recipe, v[i, b, h]) for b in range(nseq) for h in range(Hkv)]
                tokens += nseq * n_att
                t0 = time.perf_counter()
                O.step_many(units, qs, ks, vs, nthreads)
                if block:  # whole pages go per sequence, chosen over its heads
                    for b in range(nseq):
                        us = units[b * Hkv:(b + 1) * Hkv]
                        vic = O.block_select(us)
                        for u in us:
                            u.evict(vic)
                t_used += time.perf_counter() - t0
                done += 1
                if t_used >= budget or done >= last_step:
                    break
        return (tokens / t_used if t_used > 0 else 0.0), t_used

    value, t_all = run(threads, seconds, 3 * max_steps // 4)
    steps_all = done
    value1, t_one = run(1, seconds / 3, max_steps)
    how = ("then the block selection of every sequence (one thread)" if block
           else "one token evicted per unit and step")
    return {"value": value, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host": host_cpu(),
            "one_core": {"value": value1, "cores": 1, "seconds": round(t_one, 1),
                         "steps": done - steps_all},
            "sample": (f"{nseq} of the layer's {B} sequences x {Hkv} KV heads ({nseq * Hkv} units) with a "
                       f"fixed budget at the window's retained length n_att={n_att}; {steps_all} decode steps "
                       f"of fp64 oracle steps on {threads} threads ({t_all:.1f} s of CPU step time), then "
                       f"{done - steps_all} on one thread ({t_one:.1f} s), {how}; input conversion excluded")}


def host_cpu() -> str:
    """The host's CPU model and logical core count (for the CPU baseline's record)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {os.cpu_count()} logical cores"


PEAK_BF16_TFLOPS = 2500.0
# Vector ALU: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3 T lane-operations/s
# of 32-bit VALU instructions (x2 for FMA and x2 for packed fp32 is the 157.3
# TFLOP/s fp32 vector peak); v_exp_f32 issues at a quarter of that rate, so an
# exponential costs 4 lane-operation equivalents.
PEAK_VALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
EXP_COST = 4.0
# Lane-operation equivalents per score (one causal (row, key, query head)
# logit) in the two column-sum passes, from the kernels' hot loops: the rows
# pass adds the hi and lo products, subtracts the running maximum, takes one
# exp2, compares, and updates sum and maximum by fma / add and two selects
# (7 VALU + 1 exp2); the columns pass adds hi and lo, subtracts the row maximum,
# takes one exp2, scales by 1 / L and accumulates, with a conversion and an
# fp64 add per two scores (4.75 VALU + 1 exp2).
ROWS_OPS_PER_SCORE = 7.0 + EXP_COST
COLS_OPS_PER_SCORE = 4.75 + EXP_COST
# SnapKV in one pass (prompts up to 1024 positions, windows up to 32 rows)
# scores each window row once: it adds the hi and lo
# products, takes the maximum (a three-way max per two scores), subtracts the
# row maximum, takes one exp2, adds to the row sum, multiplies by the row's
# factor and adds, and converts and adds in fp64 per two scores (the mask
# only on tiles that reach the window): 6 VALU + 1 exp2.
FUSED_SNAP_OPS_PER_SCORE = 6.0 + EXP_COST
FUSED_SNAP_MAX_P, FUSED_SNAP_MAX_W = 1024, 32


def call_roofline(nbytes: float, flops: float, per_call: float, note: str, alu_ops: float = 0.0) -> dict:
    """Roofline of one whole prompt call: the bound is whichever of HBM (the
    algorithmic bytes at 8 TB/s), the bf16 matrix peak (the algorithmic flops
    at 2.5 PFLOP/s) and the vector ALU (the passes' lane-operation equivalents
    at 39.3 T/s) takes longest; the others are reported beside it."""
    t_mem, t_mfma = nbytes / (HBM_PEAK_GBS * 1e9), flops / (PEAK_BF16_TFLOPS * 1e12)
    t_alu = alu_ops / (PEAK_VALU_TOPS * 1e12)
    cands = [("hbm", t_mem, nbytes / per_call / 1e9, HBM_PEAK_GBS, "GB/s"),
             ("mfma", t_mfma, flops / per_call / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s")]
    if alu_ops:
        cands.append(("alu", t_alu, alu_ops / per_call / 1e12, round(PEAK_VALU_TOPS, 2), "T lane-ops/s"))
    cands.sort(key=lambda c: -c[1])
    name, t, ach, peak, unit = cands[0]
    out = {"bound": name, "achieved": round(ach, 2 if name != "hbm" else 1), "peak": peak, "unit": unit,
           "frac": round(t / per_call, 4), "traffic": None, "mean_call_us": round(per_call * 1e6, 2),
           "algorithmic_bytes": nbytes, "algorithmic_flops": flops}
    if alu_ops:
        out["alu_lane_ops"] = alu_ops
    for oname, ot, oach, _, _ in cands[1:]:
        out[f"{oname}_frac"] = round(ot / per_call, 4)
        out[f"{oname}_achieved"] = round(oach, 2)
    out["note"] = note
    return out


def colsum_cpu_baseline(w, lens, seconds: float):
    """The oracle's column sums (orc_colsum, as it stands) on whole units of the
    workload's first sequence, all host cores, until about `seconds` have passed."""
    import oracle as O
    from concurrent.futures import ThreadPoolExecutor
    G, Hkv, P = w.group, w.n_kv_heads, lens[0]
    K, _ = S.prompt_kv(w.recipe, 0, [P], Hkv)
    Q = S.prompt_queries(w.recipe, 0, [P], w.n_q_heads)
    cfg = O.make_cfg(head_dim=w.head_dim, group=G)
    qs = [Q[:, h * G:(h + 1) * G].astype(np.float64) for h in range(Hkv)]
    ks = [S.cache_to_f64(w.recipe, K[:, h]) for h in range(Hkv)]
    threads = min(os.cpu_count() or 1, Hkv)
    done, t_used = 0, 0.0
    with ThreadPoolExecutor(threads) as ex:
        while t_used < seconds:
            t0 = time.perf_counter()
            list(ex.map(lambda h: O.colsum(cfg, qs[h], ks[h]), range(Hkv)))
            t_used += time.perf_counter() - t0
            done += 1
    return {"value": done * P / t_used, "unit": "prompt tokens/s", "cores": threads, "kind": "oracle",
            "host": host_cpu(),
            "sample": (f"sequence 0 ({P} prompt positions) x {Hkv} KV heads x {G} query heads, "
                       f"{done} repetitions, fp64 oracle column sums on {threads} threads; "
                       f"{t_used:.1f} s of CPU time")}


def snapkv_cpu_baseline(w, lens, window: int, pool: int, keep: int, seconds: float):
    """The oracle's SnapKV selection (orc_snapkv, as it stands: window votes,
    pooling, per-head top-k, union) on whole units of the workload's first
    sequence, all host cores, until about `seconds` have passed."""
    import oracle as O
    from concurrent.futures import ThreadPoolExecutor
    G, Hkv, P = w.group, w.n_kv_heads, lens[0]
    K, _ = S.prompt_kv(w.recipe, 0, [P], Hkv)
    Q = S.prompt_queries(w.recipe, 0, [P], w.n_q_heads)
    cfg = O.make_cfg(head_dim=w.head_dim, group=G)
    qs = [Q[:, h * G:(h + 1) * G].astype(np.float64) for h in range(Hkv)]
    ks = [S.cache_to_f64(w.recipe, K[:, h]) for h in range(Hkv)]
    threads = min(os.cpu_count() or 1, Hkv)
    done, t_used = 0, 0.0
    with ThreadPoolExecutor(threads) as ex:
        while t_used < seconds:
            t0 = time.perf_counter()
            list(ex.map(lambda h: O.snapkv(cfg, qs[h], ks[h], min(window, P), pool, keep), range(Hkv)))
            t_used += time.perf_counter() - t0
            done += 1
    return {"value": done * P / t_used, "unit": "prompt tokens/s", "cores": threads, "kind": "oracle",
            "host": host_cpu(),
            "sample": (f"sequence 0 ({P} prompt positions) x {Hkv} KV heads x {G} query heads, "
                       f"{done} repetitions, fp64 oracle SnapKV selection on {threads} threads; "
                       f"{t_used:.1f} s of CPU time")}


def prefill_main(args, w):
    """--prefill: h2o_prefill_scores over the workload's prompts (one layer)."""
    import torch
    from kv_cache_eviction_h2o_amd import _lib as L
    lens = WL.prompt_lengths(w)
    B, Hq, Hkv, D = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    dev = torch.device("cuda")
    L.load_library()
    pk, _ = S.device_prompt_kv(w.recipe, 0, lens, Hkv, dev)
    pq = S.device_prompt_queries(w.recipe, 0, lens, Hq, dev)
    cfg = L.config_from_workload(w, max_len=max(lens) + 1)
    out = torch.empty((sum(lens), Hkv), dtype=torch.float64, device=dev)
    stream = torch.cuda.current_stream()
    L.prefill_scores(cfg, lens, pq, pk, out)  # checked wrapper once
    # then the C entry point on the same buffers, so the loop measures the device work
    lib = L.load_library()
    lens_c = (C.c_int32 * B)(*lens)
    argv = (C.byref(cfg), lens_c, C.c_void_p(pq.data_ptr()), C.c_void_p(pk.data_ptr()),
            C.c_void_p(out.data_ptr()))
    sh = C.c_void_p(stream.cuda_stream)

    def call():
        rc = lib.h2o_prefill_scores(*argv, sh)
        if rc != 0:
            raise L.H2OError(rc, lib.h2o_last_error(None).decode())

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    hev = HipEvents()
    e0, e1 = hev.create(), hev.create()
    t0 = time.perf_counter()
    hev.record(e0, sh)
    for _ in range(args.steps):
        call()
    hev.record(e1, sh)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per_call = hev.elapsed_s(e0, e1) / args.steps
    hev.destroy(e0)
    hev.destroy(e1)
    total = float(out.sum().item())
    expect = float(sum(lens)) * Hq  # every row's weights sum to one
    if abs(total - expect) > 1e-4 * expect:
        raise SystemExit(f"column sums add up to {total}, expected {expect}")
    pairs = sum(P * (P + 1) // 2 for P in lens)
    flops = 2.0 * D * Hq * pairs  # the causal logits, once
    alu = Hq * pairs * (ROWS_OPS_PER_SCORE + COLS_OPS_PER_SCORE)  # both passes score every causal pair
    tokens = float(sum(lens))
    nbytes = tokens * (Hq * D * 4 + Hkv * D * 2 + Hkv * 8)  # q, K, the sums
    cpu = None if args.no_cpu_baseline else colsum_cpu_baseline(w, lens, args.cpu_seconds)
    line = {
        "metric": "prompt tokens scored/sec (prefill-scored initial scores, h2o_prefill_scores)",
        "value": round(tokens / per_call, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (q as hi+lo)",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D,
                   "prompt_lens": lens if len(set(lens)) > 1 else lens[0],
                   "entry_point": "h2o_prefill_scores", "parallelism": "single GPU"},
        "roofline": call_roofline(
            nbytes, flops, per_call,
            "whole call; algorithmic bytes = fp32 q, bf16 K and the fp64 sums once; algorithmic flops = "
            "the causal logits q.k once (the kernels compute them 4x: two passes, each on the bf16 hi "
            "and lo parts of q); ALU = every causal score in both passes at 11 (rows) + 8.75 (columns) "
            "lane-operation equivalents (an exp2 counts 4) against 39.3 T/s", alu_ops=alu),
        "cpu_baseline": cpu,
        "kernel_source_sha256_16": kernel_hash(prompt=True),
    }
    print(json.dumps(line), flush=True)


def copy_probe(args, dev) -> None:
    """--copy-probe-mib: one device-to-device copy of that many MiB, the
    calibration a counter run (FETCH_SIZE, WRITE_SIZE) scales its counts by."""
    import torch
    if not args.copy_probe_mib:
        return
    n = args.copy_probe_mib * (1 << 20) // 4
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    bcp = torch.empty_like(a)
    torch.cuda.synchronize()
    bcp.copy_(a)
    torch.cuda.synchronize()
    del a, bcp


def snapkv_traffic(wname: str):
    """Measured HBM bytes per h2o_snapkv_select call for this workload's
    prompts, from a committed counter summary taken on the current prompt
    kernel sources (else None)."""
    path = os.path.join(PROFILES, f"h2o_snapkv_kernels_{wname}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_call:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_hash(prompt=True):
        return None
    return float(t.group(1))


def snapkv_main(args, w):
    """--snapkv: h2o_snapkv_select over the workload's prompts (one layer)."""
    import torch
    from kv_cache_eviction_h2o_amd import _lib as L
    lens = WL.prompt_lengths(w)
    B, Hq, Hkv, D, G = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.group
    window, pool = 32, 7
    keep = max(1, min(lens) // 5)
    dev = torch.device("cuda")
    L.load_library()
    pk, _ = S.device_prompt_kv(w.recipe, 0, lens, Hkv, dev)
    pq = S.device_prompt_queries(w.recipe, 0, lens, Hq, dev)
    cfg = L.config_from_workload(w, max_len=max(lens) + 1)
    stream = torch.cuda.current_stream()
    kept, count, votes = L.snapkv_select(cfg, lens, pq, pk, window, pool, keep)  # checked wrapper once
    # then the C entry point on the same buffers, so the loop measures the device work
    lib = L.load_library()
    cap = kept.shape[2]
    lens_c = (C.c_int32 * B)(*lens)
    argv = (C.byref(cfg), lens_c, int(window), int(pool), int(keep), C.c_void_p(pq.data_ptr()),
            C.c_void_p(pk.data_ptr()), C.c_void_p(votes.data_ptr()), C.c_void_p(kept.data_ptr()),
            C.c_void_p(count.data_ptr()), int(cap))
    sh = C.c_void_p(stream.cuda_stream)

    def call():
        rc = lib.h2o_snapkv_select(*argv, sh)
        if rc != 0:
            raise L.H2OError(rc, lib.h2o_last_error(None).decode())

    copy_probe(args, dev)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    hev = HipEvents()
    e0, e1 = hev.create(), hev.create()
    t0 = time.perf_counter()
    hev.record(e0, sh)
    for _ in range(args.steps):
        call()
    hev.record(e1, sh)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per_call = hev.elapsed_s(e0, e1) / args.steps
    hev.destroy(e0)
    hev.destroy(e1)
    c = count.cpu().numpy()
    if not (np.all(c >= window + keep) and np.all(c <= window + G * keep)):
        raise SystemExit(f"kept counts out of range: {c.min()}..{c.max()}")
    tokens = float(sum(lens))
    rows = sum(sum(i + 1 for i in range(P - min(window, P), P)) for P in lens)
    flops = 2.0 * D * Hq * rows
    one_kernel = max(lens) <= FUSED_SNAP_MAX_P and all(min(window, P) <= FUSED_SNAP_MAX_W for P in lens)
    # the window rows' scores: once in the one-kernel path, else in both passes
    alu = Hq * rows * (FUSED_SNAP_OPS_PER_SCORE if one_kernel else ROWS_OPS_PER_SCORE + COLS_OPS_PER_SCORE)
    nbytes = (sum(min(window, P) for P in lens) * Hq * D * 4 + tokens * (Hkv * D * 2 + Hq * 8)
              + B * Hkv * cap * 4 + B * 4)  # window q, K, votes, kept positions and counts
    roof = call_roofline(
        nbytes, flops, per_call,
        "whole call; algorithmic bytes = the window rows' fp32 q, bf16 K, the fp64 votes and the kept "
        "positions once; algorithmic flops = the window rows' causal logits once; ALU = the window rows' "
        + ("scores once at 10 lane-operation equivalents (one pass)" if one_kernel else
           "scores in both passes at 11 + 8.75 lane-operation equivalents")
        + "; the call also pools and selects", alu_ops=alu)
    tr = snapkv_traffic(w.name)  # FETCH_SIZE + WRITE_SIZE of the call's kernels, from profiles/
    if tr is not None:
        roof["traffic"] = round(tr)
        roof["traffic_over_algorithmic"] = round(tr / nbytes, 4)
    line = {
        "metric": "prompt tokens selected/sec (SnapKV, h2o_snapkv_select)",
        "value": round(tokens / per_call, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (q as hi+lo)",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D,
                   "prompt_lens": lens if len(set(lens)) > 1 else lens[0], "window": window, "pool": pool,
                   "keep_per_head": keep, "mean_kept": round(float(c.mean()), 1),
                   "entry_point": "h2o_snapkv_select", "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": (None if args.no_cpu_baseline
                         else snapkv_cpu_baseline(w, lens, window, pool, keep, args.cpu_seconds)),
        "kernel_source_sha256_16": kernel_hash(prompt=True),
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.summarize_trace or args.summarize_counters or args.summarize_pmc:
        summarize(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the library runs the decode step on a single MI355X "
              f"and has no multi-GPU path (asked for --gpus {args.gpus}, WORLD_SIZE={world}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from kv_cache_eviction_h2o_amd import _lib as L

    w = next(x for x in WL.ALL + WL.VARIANTS if x.name == args.workload)
    if args.prefill or args.snapkv:
        if args.workload == WL.PAGED_MIXED.name and "--workload" not in sys.argv:
            w = WL.OPT_LAYER  # the prompt calls' default: one OPT-6.7B layer's prompts
        args.steps = 256 if args.steps is None else args.steps
        args.warmup = 16 if args.warmup is None else args.warmup
        (prefill_main if args.prefill else snapkv_main)(args, w)
        return
    layers = args.layers or w.layers
    K_steps, W_steps, s0 = bench_window(w, args.steps, args.warmup, args.window_start)
    total_steps = s0 + K_steps
    lens = WL.prompt_lengths(w)
    B, Hq, Hkv, D, G = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.group
    dev = torch.device("cuda")
    lib = L.load_library()
    stream = torch.cuda.current_stream()
    sh = C.c_void_p(stream.cuda_stream)

    # ---- set-up (untimed): layer instances, inputs of every step in HBM
    t_setup = time.perf_counter()
    caches, qs, ks, vs, outs = [], [], [], [], []
    n_trace = max(w.decode_steps, total_steps)
    max_len = max(lens) + n_trace + 1
    for l in range(layers):
        pk, pv = S.device_prompt_kv(w.recipe, l, lens, Hkv, dev)
        cfg = L.config_from_workload(w, max_len=max_len)
        if w.page_size:
            cfg.max_pages = L.pages_needed(lens, n_trace, cfg)
        caches.append(L.H2OCache(cfg, lens, pk, pv))
        q, k, v = S.device_step_window(w.recipe, l, lens, total_steps, Hq, Hkv, dev)
        qs.append(q)
        ks.append(k)
        vs.append(v)
        outs.append(torch.empty((B, Hq, D), dtype=torch.float32, device=dev))
        del pk, pv
    torch.cuda.synchronize()
    q_stride, kv_stride = B * Hq * D * 4, B * Hkv * D * (2 if w.recipe.kv_dtype == "bf16" else 4)
    ctxs = [c.ctx for c in caches]
    qb = [q.data_ptr() for q in qs]
    kb = [k.data_ptr() for k in ks]
    vb = [v.data_ptr() for v in vs]
    ob = [o.data_ptr() for o in outs]
    step_fn = lib.h2o_step_compact

    hev = HipEvents()

    def run_step(s, evs=None):
        for l in range(layers):
            if evs is not None and (events == "launch" or l == 0):
                hev.record(evs[l][0], sh)
            rc = step_fn(ctxs[l], C.c_void_p(qb[l] + s * q_stride), C.c_void_p(kb[l] + s * kv_stride),
                         C.c_void_p(vb[l] + s * kv_stride), C.c_void_p(ob[l]), sh)
            if evs is not None and (events == "launch" or l == layers - 1):
                hev.record(evs[l][1], sh)
            if rc != 0:
                raise L.H2OError(rc, lib.h2o_last_error(ctxs[l]).decode())

    for s in range(0, s0):  # reach the window (the last W of these are the warm-up)
        run_step(s)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    copy_probe(args, dev)

    # ---- timed region
    events = args.events
    use_ev = events != "none"
    evs = [[(hev.create(), hev.create()) for _ in range(layers)]
           for _ in range(K_steps)] if use_ev else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K_steps):
        run_step(s0 + i, evs[i] if use_ev else None)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # ---- accounting
    counts = [M.retained_counts(w, P, total_steps) for P in lens]
    sched = np.stack([c["n_att"] for c in counts])  # [B][steps]
    win = sched[:, s0:s0 + K_steps]  # n_att per sequence per timed step
    tokens = float(win.sum()) * layers
    value = tokens / elapsed
    sbytes = {"f64": 8, "f16": 2}.get(w.score_dtype, 4)
    if w.selector == "random":
        sbytes = 0
    kv_elem = 2 if w.recipe.kv_dtype == "bf16" else 4
    launch_b = np.array([M.launch_bytes(win[:, i], n_kv_heads=Hkv, head_dim=D, kv_elem=kv_elem,
                                        group=G, score_bytes=sbytes, int8_rows=w.kv_dtype == "i8")
                        for i in range(K_steps)])
    if w.selector == "block":  # the page-eviction launches that follow a step
        for i in range(K_steps):
            s = s0 + i
            hit = [c for c in counts if c["pages"][s] > 0]
            launch_b[i] += M.block_launch_bytes([c["cand"][s] for c in hit], [c["pages"][s] for c in hit],
                                                [c["n_att"][s] for c in hit], n_kv_heads=Hkv,
                                                score_bytes=sbytes)
    step_bytes = float(launch_b.sum()) * layers
    roof = None
    if use_ev:
        if events == "launch":
            dur = np.array([[hev.elapsed_s(e0, e1) for (e0, e1) in evs[i]] for i in range(K_steps)])
        else:  # one bracket per decode step: launches back to back, gaps included
            dur = np.array([[hev.elapsed_s(evs[i][0][0], evs[i][layers - 1][1]) / layers] * layers
                            for i in range(K_steps)])
        for row in evs:
            for (e0, e1) in row:
                hev.destroy(e0)
                hev.destroy(e1)
        achieved = float((launch_b[:, None] * np.ones((1, layers))).sum() / dur.sum()) / 1e9
        tr = traffic_from_profiles(w, float(launch_b.mean()))
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None if tr is None else round(tr["bytes"]),
                "kernel": step_kernel_name(w), "timing": events,
                "mean_launch_us": round(float(dur.mean()) * 1e6, 3),
                "algorithmic_bytes_per_launch": int(launch_b.mean())}
        if tr is not None and tr["ratio"] is not None:
            roof["traffic_over_algorithmic"] = round(tr["ratio"], 4)
            roof["traffic_note"] = (f"FETCH_SIZE + WRITE_SIZE per launch over the counter profile's window "
                                    f"(steps {tr['window']}), as a ratio to that window's algorithmic bytes, "
                                    f"applied to this window's")

    # sanity: the library's counts equal the schedule used for the accounting
    expect = np.array([c["count"][-1] for c in counts])
    _, cnt, _, _ = caches[0].read_indices(int(expect.max()))
    if not np.array_equal(cnt, expect):
        raise SystemExit(f"retained counts {cnt[:4]} differ from the schedule {expect[:4]}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, int(np.round(win.mean())), args.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K_steps, "warmup": W_steps, "ms_per_step": round(elapsed / K_steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "head_dim": D, "kv_dtype": w.kv_dtype, "score_dtype": w.score_dtype if sbytes else None,
                   "score_decay": w.score_decay if sbytes else None,
                   "layers": layers, "prompt_len": lens[0] if len(set(lens)) == 1 else "mixed",
                   "window_steps": [s0, s0 + K_steps], "mean_n_att": round(float(win.mean()), 1),
                   "entry_point": "h2o_step_compact", "parallelism": "single GPU"},
        "token_heads_per_s": round(value * Hkv, 1),
        "algorithmic_bytes_per_launch": int(launch_b.mean()),
        "hbm_frac_step": round(step_bytes / elapsed / (HBM_PEAK_GBS * 1e9), 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
        "kernel_source_sha256_16": kernel_hash(),
    }
    for c in caches:
        c.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
