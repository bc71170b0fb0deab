"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Every case runs the same seeded inputs through both, step by step; see
parity.py for the acceptance rule.  Shapes: the five workloads, reduced where
the oracle would take too long over the whole trace, plus full-shape runs
checked on sampled units, plus the degenerate cases of the method.
"""
import numpy as np
import pytest

from kv_cache_eviction_h2o_amd import workloads as WL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_eviction_h2o_amd import _lib
    _lib.load_library()


def P():
    import parity
    return parity


# ------------------------------------------------------------ the workloads
@pytest.mark.parametrize("fused", [True, False], ids=["step_compact", "step+compact"])
def test_tiny_h2o_full_trace(fused):
    rep = P().run_parity(WL.TINY_H2O, WL.TINY_H2O.decode_steps, fused=fused)
    assert rep.steps == 256 and rep.evictions > 0


def test_opt_layer_reduced_full_trace():
    w = WL.OPT_LAYER.scaled(batch=2, n_q_heads=8, n_kv_heads=8)
    rep = P().run_parity(w, w.decode_steps)
    assert rep.evictions > 0


def test_opt_layer_full_shape_sampled_units():
    w = WL.OPT_LAYER
    units = [(0, 0), (3, 17), (7, 31), (5, 4)]
    P().run_parity(w, 160, units=units)


def test_llama_gqa_reduced():
    # prompt above the 1028 budget so the first step bulk-evicts, then one per step
    w = WL.LLAMA_GQA.scaled(batch=1, prompt_len=1100)
    rep = P().run_parity(w, 96)
    assert rep.evictions >= 73 * 8


def test_llama_gqa_full_context_trace():
    """The GQA layer's whole trace at batch 1: prompt 1024, then 31,744 decode
    steps until the context reaches 32,768 tokens, every step against the oracle
    (fp64 scores; one eviction per unit and step from t = 1028 on).  Long enough
    for score rounding to drift if it did: the heavy hitters' scores reach
    thousands while the eviction boundary sits at scores of order one."""
    w = WL.LLAMA_GQA.scaled(batch=1)
    n = w.decode_steps
    assert w.prompt_len + n == 32768
    rep = P().run_parity(w, n, stored_rows=True)
    assert rep.steps == n and rep.evictions == 8 * (n - 4)  # K = 1028: the first eviction at step 4


def test_random_attention_long_trace():
    w = WL.RANDOM_ATTN.scaled(batch=2, n_q_heads=8, n_kv_heads=2, rand_k=256, rand_r=32, prompt_len=300)
    rep = P().run_parity(w, 2000)
    assert rep.evictions == 4 * 54 * 32  # 4 units x 54 events x r


def test_paged_mixed_long_trace():
    # 2000 steps at the 20 % budget: four evictions every five steps, pages
    # returned and reused throughout
    w = WL.PAGED_MIXED.scaled(batch=3, n_q_heads=4, n_kv_heads=4)
    rep = P().run_parity(w, 2000, lens=[700, 1500, 3000])
    assert rep.evictions > 0


def test_llama_gqa_full_shape_sampled_units():
    w = WL.LLAMA_GQA.scaled(prompt_len=1040)
    P().run_parity(w, 24, units=[(0, 0), (9, 5), (15, 7)])


def test_random_attention_reduced():
    w = WL.RANDOM_ATTN.scaled(batch=2, n_q_heads=8, n_kv_heads=2, rand_k=64, rand_r=16,
                              prompt_len=40)
    rep = P().run_parity(w, 200)
    assert rep.evictions == 4 * 8 * 16  # 4 units x 8 events x r


@pytest.mark.parametrize("fused", [True, False], ids=["step_compact", "step+compact"])
def test_random_attention_paged(fused):
    # events drop r tokens at once: holes filled from the tail, whole pages released
    w = WL.RANDOM_ATTN.scaled(batch=3, n_q_heads=8, n_kv_heads=2, rand_k=64, rand_r=16, prompt_len=40,
                              page_size=16)
    rep = P().run_parity(w, 200, lens=[40, 23, 57], fused=fused)
    assert rep.evictions == 3 * 2 * 8 * 16  # 6 units x 8 events x r


def test_random_attention_full_shape_sampled_units():
    w = WL.RANDOM_ATTN.scaled(rand_k=256)
    rep = P().run_parity(w, 400, units=[(0, 0), (31, 7), (12, 3)])
    assert rep.evictions == 3 * 128  # the event at 384 generated tokens


def test_random_attention_stated_config_two_events():
    """Random Attention exactly as stated: 32 sequences, 32 query / 8 KV heads,
    a 2048-token prompt kept, K = 2048 generated tokens kept, buffer r = 128.
    The first event fires at step 2175 (2176 generated tokens after the append),
    the second 128 steps later; four sampled units are checked every 128 steps
    and around both events, their victim sets identical to the oracle's."""
    w = WL.RANDOM_ATTN
    assert (w.batch, w.n_q_heads, w.n_kv_heads, w.prompt_len, w.rand_k, w.rand_r) == (32, 32, 8, 2048, 2048, 128)
    units = [(0, 0), (31, 7), (12, 3), (5, 5)]
    rep = P().run_parity(w, 2304, units=units, read_every=128, check_steps={2174, 2175, 2176, 2302, 2303})
    assert rep.evictions == len(units) * 2 * 128


def test_paged_mixed_reduced():
    w = WL.PAGED_MIXED.scaled(batch=4, n_q_heads=4, n_kv_heads=4)
    P().run_parity(w, 40, lens=[300, 517, 1024, 2000])


def test_paged_first_step_window_relink():
    # the first fused step keeps the recent window's pages and relinks them
    # (window W >= 32, e >= 2W); prompts around W = 31 / 32 / 33 and around
    # page boundaries of the window's first slot and of n2, checked every step
    w = WL.PAGED_MIXED.scaled(batch=8, n_q_heads=2, n_kv_heads=2)
    rep = P().run_parity(w, 24, lens=[330, 334, 335, 343, 350, 1023, 1024, 1025], properties=True)
    assert rep.evictions > 0
    # a fixed budget (window 100) and prefill-style initial scores
    wf = WL.PAGED_MIXED.scaled(batch=2, n_q_heads=2, n_kv_heads=2, budget_fixed=200, hh_fixed=96)
    lens = [700, 1201]
    init = np.random.default_rng(11).random((sum(lens), wf.n_kv_heads)) * 0.25
    rep = P().run_parity(wf, 16, lens=lens, init_scores=init)
    assert rep.evictions >= 2 * (501 + 1001)


def test_paged_mixed_reduced_unfused():
    w = WL.PAGED_MIXED.scaled(batch=3, n_q_heads=2, n_kv_heads=2)
    P().run_parity(w, 40, lens=[64, 255, 1500], fused=False)


# ------------------------------------------------------------- edge cases
def test_budget_above_length_is_full_attention():
    w = WL.TINY_H2O.scaled(budget_fixed=4096, hh_fixed=2000)
    rep = P().run_parity(w, 64)
    assert rep.evictions == 0


@pytest.mark.parametrize("wname", ["tiny_fma", "gqa_matrix_core"])
def test_exactly_tied_scores(wname):
    """Zero queries: every step weighs its slots equally, so every prompt token
    reaches the bulk first step with exactly the same score and the tie rule
    alone (equal scores: the lower position is kept) decides which of them
    stay; later steps keep ties among tokens present over the same steps.
    Every step is checked against the oracle, and no near-tie may be adopted:
    the victim sets must be the oracle's exactly."""
    if wname == "tiny_fma":
        w = WL.TINY_H2O.scaled(batch=2)
    else:
        w = WL.LLAMA_GQA.scaled(batch=2, n_q_heads=16, n_kv_heads=2, budget_fixed=96, hh_fixed=40)
    rep = P().run_parity(w, 40, lens=[300, 257], zero_q=True)
    assert rep.evictions > 0 and rep.adopted == 0


def test_ragged_prompts_fixed_budget():
    w = WL.TINY_H2O.scaled(batch=4)
    rep = P().run_parity(w, 80, lens=[20, 63, 64, 150])
    assert rep.evictions > 0


def test_sliding_window_and_zero_recent_window():
    # no sinks, no heavy hitters: the last W positions only
    P().run_parity(WL.TINY_H2O.scaled(n_sink=0, budget_fixed=40, hh_fixed=0), 50)
    # W = 0: the new token is itself a candidate and may go at once
    P().run_parity(WL.TINY_H2O.scaled(budget_fixed=24, hh_fixed=20), 50)


def test_gqa_group_of_two_bf16():
    w = WL.OPT_LAYER.scaled(batch=2, n_q_heads=4, n_kv_heads=2)
    P().run_parity(w, 60, lens=[200, 333])


def test_unfused_bulk_and_random():
    w = WL.OPT_LAYER.scaled(batch=1, n_q_heads=4, n_kv_heads=4)
    P().run_parity(w, 30, lens=[700], fused=False)
    wr = WL.RANDOM_ATTN.scaled(batch=2, n_q_heads=4, n_kv_heads=2, rand_k=20, rand_r=5,
                               prompt_len=16)
    P().run_parity(wr, 60, fused=False)


def test_initial_scores():
    w = WL.TINY_H2O.scaled(batch=2)
    lens = [100, 90]
    rng = np.random.default_rng(5)
    init = rng.random((sum(lens), w.n_kv_heads)) * 0.01
    P().run_parity(w, 40, lens=lens, init_scores=init)


# -------------------------------------- more sequences than the kernel arguments hold
# Above 128 sequences the step kernels read each sequence's prompt length and
# retained count from device memory instead of their arguments, and take the
# units in plain order.  Prompts from 1 token on (below the sinks and budget).
def _many_lens(n, seed):
    r = np.random.default_rng(seed)
    lens = [int(x) for x in r.integers(1, 90, size=n)]
    lens[0], lens[1] = 1, 2
    return lens


@pytest.mark.parametrize("fused", [True, False], ids=["step_compact", "step+compact"])
def test_batch_above_argument_limit_fma_path(fused):
    w = WL.OPT_LAYER.scaled(batch=131, n_q_heads=2, n_kv_heads=2, budget_fixed=40, hh_fixed=16)
    rep = P().run_parity(w, 30, lens=_many_lens(131, 1), fused=fused)
    assert rep.evictions > 0


def test_batch_above_argument_limit_matrix_core_path():
    w = WL.LLAMA_GQA.scaled(batch=130, n_q_heads=8, n_kv_heads=2, budget_fixed=40, hh_fixed=16)
    rep = P().run_parity(w, 30, lens=_many_lens(130, 2))
    assert rep.evictions > 0


def test_batch_above_argument_limit_random_attention():
    w = WL.RANDOM_ATTN.scaled(batch=129, n_q_heads=8, n_kv_heads=2, rand_k=12, rand_r=4)
    rep = P().run_parity(w, 40, lens=_many_lens(129, 3))
    assert rep.evictions > 0


# ----------------------------------- FMA path with logits in global scratch
# G x n_att x 4 bytes above 64 KB: the FMA step kernel keeps its logits in
# global scratch instead of LDS (contiguous and paged layouts).
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
@pytest.mark.parametrize("fused", [True, False], ids=["step_compact", "step+compact"])
def test_fma_logits_in_global_scratch(paged, fused):
    base = WL.PAGED_MIXED if paged else WL.OPT_LAYER
    w = base.scaled(batch=2, n_q_heads=2, n_kv_heads=1, budget_fixed=17000, hh_fixed=8000)
    rep = P().run_parity(w, 12, lens=[17100, 9000], fused=fused)
    assert rep.evictions > 0


# ------------------------------------------------ matrix-core path (G = 4, 8)
def test_gqa_ragged_units_cross_tile_edges():
    # units start at 5, 64 (a whole number of 32-slot tiles), 95 and 130 slots
    # and grow by one a step, so n passes multiples of 32 and partial tiles
    w = WL.LLAMA_GQA.scaled(batch=4, budget_fixed=100, hh_fixed=48)
    rep = P().run_parity(w, 60, lens=[5, 64, 95, 130])
    assert rep.evictions > 0


def test_gqa_unfused_tiles_compaction():
    # bulk hole fill and single moves in the operand-order layout
    w = WL.LLAMA_GQA.scaled(batch=2, budget_fixed=200, hh_fixed=96)
    rep = P().run_parity(w, 40, lens=[300, 150], fused=False)
    assert rep.evictions > 0


def test_gqa_logits_in_global_scratch():
    # 8 heads x 2624 slots of logits exceed the LDS budget: global scratch
    w = WL.LLAMA_GQA.scaled(batch=1, budget_fixed=2600, hh_fixed=1300)
    rep = P().run_parity(w, 12, lens=[2700])
    assert rep.evictions >= 8 * 100


def test_gqa_group_of_four_h2o_fp32_scores():
    w = WL.OPT_LAYER.scaled(batch=2, n_q_heads=8, n_kv_heads=2)
    rep = P().run_parity(w, 40, lens=[400, 257])
    assert rep.evictions > 0


# ------------------------------------------------ FMA path with G >= 4
def test_paged_group_of_four():
    w = WL.PAGED_MIXED.scaled(batch=2, n_q_heads=8, n_kv_heads=2)
    P().run_parity(w, 30, lens=[300, 700])


def test_fp32_rows_group_of_eight():
    w = WL.TINY_H2O.scaled(batch=2, n_q_heads=16, n_kv_heads=2)
    rep = P().run_parity(w, 60, lens=[90, 200])
    assert rep.evictions > 0


# ------------------------------------------------ compressed state (int8 rows)
@pytest.mark.parametrize("fused", [True, False], ids=["step_compact", "step+compact"])
def test_int8_opt_layer_reduced_full_trace(fused):
    w = WL.OPT_LAYER_I8.scaled(batch=2, n_q_heads=8, n_kv_heads=8)
    rep = P().run_parity(w, w.decode_steps if fused else 200, fused=fused)
    assert rep.evictions > 0


def test_int8_opt_layer_full_shape_sampled_units():
    # the benchmarked shape and launch configuration of the int8 variant
    w = WL.OPT_LAYER_I8
    P().run_parity(w, 160, units=[(0, 0), (3, 17), (7, 31), (5, 4)])


def test_int8_paged_mixed():
    w = WL.PAGED_MIXED.scaled(kv_dtype="i8", batch=3, n_q_heads=4, n_kv_heads=4)
    P().run_parity(w, 30, lens=[300, 517, 1500])


def test_int8_gqa_group_of_four_and_random():
    w = WL.LLAMA_GQA.scaled(kv_dtype="i8", batch=1, n_q_heads=16, n_kv_heads=4, prompt_len=1100)
    P().run_parity(w, 40)
    wr = WL.RANDOM_ATTN.scaled(kv_dtype="i8", batch=2, n_q_heads=8, n_kv_heads=2, rand_k=64, rand_r=16,
                               prompt_len=40)
    rep = P().run_parity(wr, 120)
    assert rep.evictions == 4 * 3 * 16  # events after steps 79, 95, 111 (K + r = 80 generated)


# ------------------------------------------- paged workload at its full shape
def test_paged_mixed_full_shape_sampled_units():
    """The paged workload's shape and launch configuration (64 sequences of
    4k-64k prompts, 32 KV heads, fused entry point, device-drawn inputs): three
    heads of each of the two shortest and the two longest sequences against the
    oracle at every step -- the first step bulk-evicts the longest units from
    ~65K slots to ~13K through the radix select and the hole fill -- then every
    unit for the properties that hold at any size.  After the first step the
    scores are single softmax weights (~1e-5), all within the near-tie rule's
    absolute gap of each other, so the number of victims a unit-step may swap
    under that rule is also capped."""
    w = WL.PAGED_MIXED
    lens = WL.prompt_lengths(w)
    order = np.argsort(lens)
    seqs = [int(x) for x in order[:2]] + [int(x) for x in order[-2:]]
    assert max(lens[b] for b in seqs) > 60000
    units = [(b, h) for b in seqs for h in (0, 13, w.n_kv_heads - 1)]
    rep = P().run_parity(w, 16, lens=lens, units=units, device_inputs=True, stored_rows=False,
                         read_every=1, properties=True, max_swapped=8)
    # the bulk first step alone evicts len + 1 - floor((len + 1) / 5) tokens per unit
    bulk = sum(3 * (lens[b] + 1 - (lens[b] + 1) // 5) for b in seqs)
    assert rep.evictions > bulk


# ------------------------------------- compressed score state (moving sum, binary16)
# "Attention Sinks and KV cache eviction", section 6.2: the per-token score state
# is quantised to FP16, or the exact sum replaced by a moving average.  Binary16
# runs are checked in lockstep at every step (parity.py).
@pytest.mark.parametrize("fused", [True, False], ids=["step_compact", "step+compact"])
def test_f16_moving_sum_opt_layer_reduced_full_trace(fused):
    w = WL.OPT_LAYER_F16.scaled(batch=2, n_q_heads=8, n_kv_heads=8)
    assert w.score_dtype == "f16" and 0 < w.score_decay < 1
    rep = P().run_parity(w, w.decode_steps if fused else 200, fused=fused)
    assert rep.evictions > 0


def test_f16_moving_sum_opt_layer_full_shape_sampled_units():
    # the benchmarked shape and launch configuration of the binary16 variant
    w = WL.OPT_LAYER_F16
    rep = P().run_parity(w, 160, units=[(0, 0), (3, 17), (7, 31), (5, 4)])
    assert rep.evictions > 0


def test_f16_exact_sum_paged_bulk_first_step():
    # decay 1 (the exact sum, rounded to binary16 each step), paged, bulk first step
    w = WL.PAGED_MIXED.scaled(batch=3, n_q_heads=4, n_kv_heads=4, score_dtype="f16")
    rep = P().run_parity(w, 40, lens=[300, 517, 1500])
    assert rep.evictions > 0


def test_f16_gqa_matrix_core_path():
    # the matrix-core kernel (G = 8) with binary16 scores: bulk eviction at the
    # first step through the radix select on widened binary16 keys, then one a step
    w = WL.LLAMA_GQA.scaled(batch=2, prompt_len=1100, score_dtype="f16", score_decay=0.998)
    rep = P().run_parity(w, 96)
    assert rep.evictions >= 2 * 8 * (73 + 95)


def test_f16_int8_rows_and_initial_scores():
    w = WL.OPT_LAYER_I8.scaled(batch=2, n_q_heads=4, n_kv_heads=4, score_dtype="f16", score_decay=0.99)
    P().run_parity(w, 60, lens=[400, 257])
    wt = WL.TINY_H2O.scaled(batch=2, score_dtype="f16", score_decay=0.995)
    lens = [100, 90]
    init = np.random.default_rng(7).random((sum(lens), wt.n_kv_heads)) * 0.5
    P().run_parity(wt, 40, lens=lens, init_scores=init)


@pytest.mark.parametrize("score_dtype", ["f32", "f64"])
def test_moving_sum_fp32_fp64_scores(score_dtype):
    w = WL.OPT_LAYER.scaled(batch=2, n_q_heads=8, n_kv_heads=4, score_dtype=score_dtype, score_decay=0.99)
    rep = P().run_parity(w, 300, lens=[700, 333])
    assert rep.evictions > 0
    wg = WL.LLAMA_GQA.scaled(batch=1, prompt_len=1100, score_dtype=score_dtype, score_decay=0.995)
    P().run_parity(wg, 60)
