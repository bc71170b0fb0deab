"""The five synthetic workloads the H2O decode step is built and measured on.

Shapes follow the pages: an OPT-6.7B layer (32 heads x 128) at a 20 % budget
("H2O: Heavy-Hitter Oracle", results summary), a LLaMA-2-70B GQA layer
(64 query / 8 KV heads x 128, "Attention Sinks and KV cache eviction", section
1.1) with a 4 sink + 512 heavy-hitter + 512 recent budget (the StreamingLLM vs
H2O article, cache-manager listing), Random Attention's kept prompt with a
period K and buffer r ("Random Attention", method and experiments), and 16-token
KV pages ("Attention Sinks and KV cache eviction", section 5).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

from .synth import Recipe


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    kv_dtype: str                 # storage: "f32" | "bf16" | "i8" (inputs in recipe.kv_dtype)
    score_dtype: str              # "f32" | "f64" | "f16" (unused by the Random selector)
    selector: str                 # "h2o" | "random" | "block" (paged only)
    n_sink: int = 4
    budget_fixed: int = 0         # > 0: fixed budget K
    hh_fixed: int = 0             #        with this many heavy hitters
    budget_num: int = 1           # else K_t = floor(len * num / den)
    budget_den: int = 5
    score_decay: float = 1.0      # 1 = exact cumulative sum; < 1 = moving sum (decay per step)
    rand_k: int = 0
    rand_r: int = 0
    prompt_len: int = 0           # > 0: every sequence has this prompt
    len_lo: int = 0               # else prompt lengths uniform on [len_lo, len_hi]
    len_hi: int = 0
    decode_steps: int = 0
    page_size: int = 0            # 0 = contiguous slots, 16 = paged
    layers: int = 1               # independent layer instances stepped in turn
    recipe: Recipe = field(default_factory=lambda: Recipe(seed=0, head_dim=128))

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY_H2O = Workload(
    name="tiny_h2o", batch=1, n_q_heads=4, n_kv_heads=4, head_dim=64, kv_dtype="f32",
    score_dtype="f32", selector="h2o", budget_fixed=64, hh_fixed=28, prompt_len=256,
    decode_steps=256, recipe=Recipe(seed=0xC1, head_dim=64, kv_dtype="f32", boost_frac=0.02))

OPT_LAYER = Workload(
    name="opt6.7b_layer_20pct", batch=8, n_q_heads=32, n_kv_heads=32, head_dim=128,
    kv_dtype="bf16", score_dtype="f32", selector="h2o", budget_num=1, budget_den=5,
    prompt_len=1024, decode_steps=1024, layers=32,
    recipe=Recipe(seed=0xC2, head_dim=128, kv_dtype="bf16", boost_frac=0.03))

LLAMA_GQA = Workload(
    name="llama2_70b_gqa_4+512+512", batch=16, n_q_heads=64, n_kv_heads=8, head_dim=128,
    kv_dtype="bf16", score_dtype="f64", selector="h2o", budget_fixed=1028, hh_fixed=512,
    prompt_len=1024, decode_steps=31744, layers=80,
    recipe=Recipe(seed=0xC3, head_dim=128, kv_dtype="bf16", boost_frac=0.01, zipf_s=1.1,
                  zipf_n=16))

RANDOM_ATTN = Workload(
    name="random_attention_k2048_r128", batch=32, n_q_heads=32, n_kv_heads=8, head_dim=128,
    kv_dtype="bf16", score_dtype="f32", selector="random", rand_k=2048, rand_r=128,
    prompt_len=2048, decode_steps=30720,
    recipe=Recipe(seed=0xC4, head_dim=128, kv_dtype="bf16", boost_frac=0.02))

PAGED_MIXED = Workload(
    name="paged_mixed_4k-64k_20pct", batch=64, n_q_heads=32, n_kv_heads=32, head_dim=128,
    kv_dtype="bf16", score_dtype="f32", selector="h2o", budget_num=1, budget_den=5,
    len_lo=4096, len_hi=65536, decode_steps=65, page_size=16,
    recipe=Recipe(seed=0xC5, head_dim=128, kv_dtype="bf16", boost_frac=0.03))

ALL = (TINY_H2O, OPT_LAYER, LLAMA_GQA, RANDOM_ATTN, PAGED_MIXED)

# Compressed state: the OPT layer with its K/V stored as int8 rows of 128 plus
# one fp32 scale per row (inputs stay bf16; see oracle.quantize_rows for the
# quantisation), the INT8 K/V storage the pages list beside eviction.
OPT_LAYER_I8 = OPT_LAYER.scaled(name="opt6.7b_layer_20pct_int8", kv_dtype="i8")

# Block-granular eviction: the paged workload with whole 16-token pages evicted,
# those with the fewest heavy-hitter tokens over the sequence's KV heads first
# ("Attention Sinks and KV cache eviction", section 5).
PAGED_BLOCK = PAGED_MIXED.scaled(name="paged_mixed_4k-64k_20pct_block", selector="block")
# Compressed score state ("Attention Sinks and KV cache eviction", section 6.2):
# the OPT layer with its cumulative scores stored as IEEE binary16 and the exact
# sum replaced by a moving sum that decays by 1 - 2^-8 per step (an effective
# memory of ~256 steps, a quarter of the trace; binary16 and this decay keep the
# largest score below G / (1 - decay) = 256).
OPT_LAYER_F16 = OPT_LAYER.scaled(name="opt6.7b_layer_20pct_f16", score_dtype="f16", score_decay=1.0 - 2.0 ** -8)
VARIANTS = (OPT_LAYER_I8, PAGED_BLOCK, OPT_LAYER_F16)


def prompt_lengths(w: Workload):
    """Per-sequence prompt lengths of a workload (list of int)."""
    if w.prompt_len > 0:
        return [w.prompt_len] * w.batch
    from .synth import uniform_lengths
    return [int(x) for x in uniform_lengths(w.recipe.seed, w.batch, w.len_lo, w.len_hi)]
