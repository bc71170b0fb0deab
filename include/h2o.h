/*
 * h2o.h -- C ABI of the MI355X (gfx950) H2O decode-step library (libh2o.so).
 *
 * One decode step for a batch of sequences, per (sequence b, KV head h):
 *   a1 append   the new token's key/value becomes a retained slot;
 *   a2-a4       its G query heads attend over the retained keys/values
 *               (q.K, softmax, P.V);
 *   a5 (H2O)    every softmax weight is added to its token's cumulative score,
 *               the G weights of a GQA group summed into the shared KV head;
 *   a6 select   H2O: the lowest-score tokens outside the sink tokens and the
 *               recent window are evicted down to the budget K_t;
 *               Random Attention: when the retained generated tokens reach
 *               K + r, r of them are evicted uniformly at random per head
 *               (the prompt is never evicted);
 *   a7 compact  the retained slots are made contiguous again in place
 *               (paged layout: whole 16-token pages are released).
 *   Block eviction (H2O_SEL_BLOCK, paged layout only): a5 as for H2O, no
 *               token goes in a6; after the step whole 16-token pages go
 *               instead (see H2O_SEL_BLOCK below) and a7 only rewrites the
 *               block table -- nothing in the cache moves.
 *
 * Where the operation is defined (titles of the pages describing the method):
 *   "H2O: Heavy-Hitter Oracle for Efficient Generative Inference of LLMs",
 *       summary -- budget K, the greedy eviction over S_{i-1} + {i} by
 *       cumulative attention (Algorithm 1 as summarised there).
 *   "Attention Sinks and KV cache eviction: why a sliding window is not
 *       enough" -- sec. 3.1 (softmax weights of one query sum to one),
 *       sec. 4.1 (four sink tokens kept for good), sec. 4.2 (scores summed
 *       over decode steps; sinks + top-k heavy hitters + recent window kept),
 *       sec. 5 (16-token KV blocks), sec. 6.2 (per-token fp32 score state).
 *   "KV Cache compression and selective retention: StreamingLLM vs H2O" --
 *       cache-manager listing: evict(key_cache, value_cache, scores) with
 *       4 sinks + heavy hitters + recent rows, [B, H, S, D] layout.
 *   "Random Attention: rethinking KV cache eviction" -- method modules 1-3
 *       and the integration notes (keep the prompt; per-head uniform random
 *       eviction; eviction period K and buffer r).
 *
 * Conventions
 *   - The decode calls (h2o_step, h2o_compact, h2o_step_compact) and the
 *     prompt calls are asynchronous on `stream` (a hipStream_t; NULL = the
 *     device's null stream): they only enqueue work.  h2o_init enqueues the
 *     prompt load on `stream` but first uploads its small host tables (prompt
 *     lengths and offsets, the block table) with blocking copies, so it
 *     returns once those are on the device.  h2o_read_indices and h2o_read_kv
 *     wait for `stream`; h2o_destroy waits for the device.  Pointers named
 *     "device" must stay valid until the stream has run the work and be
 *     16-byte aligned (the kernels use 16-byte vector accesses; a misaligned
 *     one is rejected with H2O_EINVAL before anything runs).
 *   - Inputs must be finite: q, K and V values that are NaN or infinite give
 *     unspecified outputs, scores and selections (the prompt calls are built
 *     on the assumption that no NaN occurs).  Nothing checks this.
 *   - Kernel self-checks: the step kernels record inconsistencies they detect
 *     (a selection that found a different number of victims than scheduled,
 *     no evictable candidate, a compaction whose holes and live tail slots
 *     do not pair up, a block-eviction range that does not match the stored
 *     positions) in an error word of the context.  Nothing in the decode loop
 *     reads it back: the next h2o_read_indices reports it as H2O_EDEVICE
 *     ("kernel consistency check failed"), so a loop that never reads does
 *     not see it.
 *   - Layouts (row-major): q and out [B][Hq][D] fp32; k_new, v_new
 *     [B][Hkv][D] in kv_dtype (bf16 = raw bf16 bits); query head j belongs to
 *     KV head j / G, G = Hq / Hkv.
 *   - Positions: sequence b's prompt holds positions 0..P_b-1; its s-th
 *     decode step (s = 0, 1, ...) appends position t = P_b + s.  All sequences
 *     step together.
 *   - Supported shapes: (kv_dtype, head_dim) = (H2O_BF16, 128), (H2O_I8, 128)
 *     or (H2O_F32, 64); G in {1, 2, 4, 8}.
 *   - H2O_I8 (compressed state; "KV cache eviction policies", section on
 *     alternatives used with eviction: INT8 K/V storage is orthogonal to
 *     eviction; "Attention Sinks and KV cache eviction", sec. 1.2): prompts
 *     and new tokens arrive as bf16 and are stored as int8 rows of 128 with
 *     one fp32 scale per (token, KV head) row: scale = max |x| / 127,
 *     code = rint(x / scale) in [-127, 127], all in fp32 (a zero row has
 *     scale 0).  Attention, also over the new token, uses code * scale.
 *   - Compressed score state ("Attention Sinks and KV cache eviction",
 *     sec. 6.2: the fp32 per-token score state costs 4 MB per 1M tokens, and
 *     deployments quantise it to FP16/INT8 or replace the exact sum by a
 *     moving average).  score_decay lam in (0, 1) turns the cumulative sum
 *     into a moving sum: at every step each retained score becomes
 *     lam * score + (the step's weights summed over the group), evaluated as
 *     one fused multiply-add in the score's precision (fp32 for H2O_F16), the
 *     new token starting from zero; lam = 1 is the exact sum.  The moving sum
 *     stays below G / (1 - lam).  score_dtype H2O_F16 stores each score as
 *     IEEE binary16, rounded to nearest (ties to even) after every update and
 *     on entry (initial scores), so a score past 65504 becomes infinite and is
 *     never evicted; with lam <= 1 - G / 65504 that cannot happen.  The
 *     selection ranks the stored values (equal values: the lower position is
 *     kept), and evicted_mass sums them in fp64.
 *   - Errors: every call returns an h2o_status.  Arguments are validated
 *     before anything is enqueued; on error nothing is enqueued and the
 *     context is unchanged (H2O_EDEVICE aside).  h2o_last_error() gives the
 *     message.  One context must not be used from two threads at once;
 *     different contexts are independent and may be driven from different
 *     threads at the same time (the library's shared host records -- kernel
 *     launch limits, the prompt calls' scratch, the last context-free error
 *     -- are guarded).
 *   - Ownership: the library owns the context and its device state,
 *     allocated with hipMalloc on the device current at h2o_init and freed
 *     by h2o_destroy -- unless h2o_config::workspace is given, in which case
 *     the state is carved from that caller-owned memory and nothing is
 *     allocated.  The prompt calls (h2o_prefill_scores, h2o_snapkv_select)
 *     keep one scratch buffer per device for the life of the process.  The
 *     caller owns every pointer it passes.
 */
#ifndef H2O_H
#define H2O_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct h2o_ctx h2o_ctx;

typedef enum {
    H2O_OK = 0,
    H2O_EINVAL = -1,   /* bad argument or unsupported configuration */
    H2O_ENOMEM = -2,   /* device memory or KV page pool exhausted */
    H2O_EDEVICE = -3,  /* a HIP call failed (message kept) */
    H2O_ESTATE = -4    /* call out of order (e.g. h2o_step while a compaction is pending) */
} h2o_status;

/* Selectors.  H2O_SEL_BLOCK: block-granular eviction ("Attention Sinks and KV
 * cache eviction", sec. 5: the cache is managed in blocks, so eviction frees
 * whole blocks, those with the lowest share of important tokens first).  With
 * the paged layout, at length len = t + 1 and the H2O schedule (K, HH, W):
 * when the retained count n exceeds K, the candidates are the sequence's
 * whole retained pages holding no sink position (< n_sink) and ending before
 * the recent window (positions < len - W); a token is important for a KV head
 * when it is among that head's HH highest-scored candidate tokens (equal
 * scores: the older token); a page's importance is its count of important
 * (token, head) pairs over the sequence's KV heads; the
 * min(#candidates, ceil((n - K) / 16)) pages of lowest importance go (equal
 * importance: the older page first).  Pages hold 16 consecutive positions and
 * never move, so after a step a sequence holds either <= K tokens or no
 * candidate page.  Slot capacity: max(P, K_max + 16 * ceil(n_sink / 16) + 15) + 1
 * tokens, at most 5120 pages per sequence; at most 1024 KV heads. */
enum { H2O_SEL_H2O = 0, H2O_SEL_RANDOM = 1, H2O_SEL_BLOCK = 2 };
enum { H2O_F32 = 0, H2O_BF16 = 1, H2O_F64 = 2, H2O_I8 = 3, H2O_F16 = 4 };

typedef struct {
    int32_t batch;         /* B sequences */
    int32_t n_q_heads;     /* Hq */
    int32_t n_kv_heads;    /* Hkv; Hq must be a multiple */
    int32_t head_dim;      /* D */
    int32_t kv_dtype;      /* H2O_BF16, H2O_F32, or H2O_I8 (bf16 inputs stored as int8 rows) */
    int32_t score_dtype;   /* H2O, block: H2O_F32 or H2O_F64 cumulative scores; H2O also
                              H2O_F16 (compressed state, see score_decay) */
    float scale;           /* logit scale; 0 -> 1/sqrt(D) */
    int32_t selector;      /* H2O_SEL_H2O, H2O_SEL_RANDOM or H2O_SEL_BLOCK (needs page_size 16) */
    int32_t n_sink;        /* H2O: positions 0..n_sink-1 are never evicted (4 on the pages) */
    int32_t budget_fixed;  /* H2O: > 0 -> fixed budget K ...                          */
    int32_t hh_fixed;      /*        ... of which hh_fixed heavy hitters; recent window
                                     W = K - n_sink - hh_fixed                         */
    int32_t budget_num;    /* H2O: else K_t = floor(len * num / den) with len = t + 1, */
    int32_t budget_den;    /*      HH_t = floor((K_t - n_sink) / 2), W_t = the rest    */
    int32_t rand_k;        /* Random: generated tokens kept after an eviction (K) */
    int32_t rand_r;        /* Random: buffer r; r tokens are evicted at K + r */
    uint64_t seed;         /* Random: Philox4x64-10 key word 0 */
    int32_t page_size;     /* 0 = contiguous slots per (b, h); 16 = paged */
    int32_t max_pages;     /* paged: size of the page pool (pages of Hkv x 16 tokens) */
    int32_t max_len;       /* most positions any sequence will reach (prompt + steps) */
    void *workspace;       /* device memory for the context's state, or NULL (the library
                              allocates it).  Non-NULL: 256-byte aligned and at least
                              h2o_workspace_size() bytes; the caller owns it, keeps it
                              until h2o_destroy has returned, and h2o_destroy leaves it
                              alone.  Lets an allocator that owns device memory (a
                              framework's caching allocator) hold the cache. */
    uint64_t workspace_bytes;  /* size of workspace (ignored when it is NULL) */
    float score_decay;     /* H2O, block: 0 or 1 = the exact cumulative sum; else in (0, 1):
                              a moving sum, see the compressed-state note above */
} h2o_config;

/* Device bytes the context of (cfg, prompt_len) keeps for its state: the K/V
 * cache, scores, positions, counts, page tables and scratch -- the size a
 * caller-provided h2o_config::workspace must have.  Validates as h2o_init does
 * and touches no device.  Errors: H2O_EINVAL (config/shape), H2O_ENOMEM (paged:
 * the prompts need more pages than max_pages). */
int h2o_workspace_size(const h2o_config *cfg, const int32_t *prompt_len, uint64_t *bytes);

/* Page pool size for the paged layout: the pages (of Hkv x 16 tokens) that
 * cover the prompts and `steps` decode steps of every sequence under the
 * configured selector and budget ("Attention Sinks and KV cache eviction",
 * sec. 5: the cache is managed in fixed-size blocks).  It is the sum over the
 * sequences of the most pages each holds at any point: ceil(P_b / 16) after
 * the prompt load, and ceil(n_att / 16) while a step runs (the appended
 * token's page is taken before anything is evicted).  A pool of this size
 * (h2o_config::max_pages) never runs out in those steps.  cfg->max_pages is
 * ignored; host arithmetic only, no device is touched.
 * Errors: H2O_EINVAL (config/shape, page_size != 16, steps < 0, or a prompt
 * plus `steps` past max_len). */
int h2o_pool_pages(const h2o_config *cfg, const int32_t *prompt_len, int32_t steps, int32_t *pages);

/* Create a context and load the prompts.
 *   prompt_len  host [B]: P_b >= 1.
 *   prompt_k/v  device, packed [sum_b P_b][Hkv][D] in kv_dtype, sequences in order.
 *   init_scores device [sum_b P_b][Hkv] fp64 initial cumulative scores, or NULL = 0.
 * The prompts are copied; the caller may reuse its buffers once the stream has
 * run the copy.  On success *out receives the context.
 * With cfg->workspace the state is carved from it and nothing is allocated.
 * Errors: H2O_EINVAL (config/shape; a workspace below h2o_workspace_size),
 * H2O_ENOMEM (device memory or page pool), H2O_EDEVICE. */
int h2o_init(h2o_ctx **out, const h2o_config *cfg, const int32_t *prompt_len,
             const void *prompt_k, const void *prompt_v, const double *init_scores,
             void *stream);

/* One decode step, steps a1-a6: append, attend, accumulate (H2O), select.
 *   q    device [B][Hq][D] fp32       k_new, v_new device [B][Hkv][D] kv_dtype
 *   out  device [B][Hq][D] fp32 attention output over the pre-eviction set.
 * The victims are recorded; h2o_compact must follow before the next step or read.
 * Errors: H2O_EINVAL (a sequence would pass max_len), H2O_ENOMEM (no free page
 * for the append), H2O_ESTATE (a compaction is pending), H2O_EDEVICE. */
int h2o_step(h2o_ctx *ctx, const float *q, const void *k_new, const void *v_new, float *out,
             void *stream);

/* Step a7 for the pending step: move retained slots into the victims' holes,
 * set the retained counts, release pages no longer used (block eviction:
 * choose and release the step's pages, see H2O_SEL_BLOCK).
 * Errors: H2O_ESTATE (no step pending), H2O_EDEVICE. */
int h2o_compact(h2o_ctx *ctx, void *stream);

/* Steps a1-a7 in one launch where the selection allows it: the same result as
 * h2o_step followed by h2o_compact.  Leaves nothing pending. */
int h2o_step_compact(h2o_ctx *ctx, const float *q, const void *k_new, const void *v_new,
                     float *out, void *stream);

/* Read the retained state back to the host; waits for `stream`.
 *   pos           host [B][Hkv][cap]: retained positions of each (b, h), ascending
 *                 (entries past the count are set to -1).
 *   count         host [B]: retained tokens per sequence (equal for all its heads).
 *   scores        host [B][Hkv][cap] fp64, aligned with pos; NULL to skip.
 *   evicted_mass  host [B][Hkv] fp64 summed scores of evicted tokens; NULL to skip.
 *   cap           entries per (b, h) in pos/scores; must be >= every count.
 * With block eviction a pending step may be read: the state after the append,
 * before any page goes (the scores the page ranking will use).  A read is not
 * a hot-path call: it allocates device staging of 12 bytes per entry
 * (B x Hkv x cap) for its duration, also for a context in a caller workspace.
 * Errors: H2O_EINVAL (cap too small), H2O_ESTATE (a compaction is pending,
 * block eviction aside), H2O_EDEVICE. */
int h2o_read_indices(h2o_ctx *ctx, int32_t *pos, int32_t *count, double *scores,
                     double *evicted_mass, size_t cap, void *stream);

/* Read the stored K/V rows of the retained tokens back to the host, in the
 * order h2o_read_indices gives positions (ascending); waits for `stream`.
 *   k_rows, v_rows    host [B][Hkv][cap][row bytes]: rows as stored, in natural
 *                     element order -- bf16 bits or fp32 (256 bytes), or int8
 *                     codes (128 bytes); entries past the count are zeroed.
 *   k_scale, v_scale  host [B][Hkv][cap] fp32 row scales (H2O_I8; ignored and
 *                     may be NULL otherwise).
 *   cap               entries per (b, h); must be >= every count.
 * A pending block-eviction step reads as in h2o_read_indices.  Allocates
 * device staging for the rows (and positions) for its duration.
 * Errors: H2O_EINVAL, H2O_ESTATE (a compaction is pending, block eviction
 * aside), H2O_EDEVICE. */
int h2o_read_kv(h2o_ctx *ctx, void *k_rows, void *v_rows, float *k_scale, float *v_scale, size_t cap,
                void *stream);

/* Slot capacity per (b, h) unit and the current step index s (host-side, no sync). */
int h2o_info(const h2o_ctx *ctx, int32_t *slot_capacity, int32_t *steps_done,
             int32_t *pages_in_use);

/* Free the context and its device memory (waits for the device). NULL is a no-op. */
void h2o_destroy(h2o_ctx *ctx);

/* Prefill-scored initial scores: the cumulative attention score each prompt
 * token would hold had every prompt position's query been scored like a decode
 * step ("Attention Sinks and KV cache eviction", sec. 4.2: the score sums a
 * token's attention weights over the queries that saw it; sec. 4.3: scores
 * gathered only during decode start from nothing).  For sequence b, KV head h
 * and prompt position j, with off_b = P_0 + ... + P_{b-1}:
 *   out[(off_b + j) * Hkv + h] = sum over positions i in [j, P_b) and the G
 *       query heads g of h of the causal softmax weight of key j in row i,
 *       softmax over j' <= i of scale * q[off_b + i][h G + g] . k[off_b + j'][h].
 * The result is h2o_init's init_scores.
 *   cfg         batch, n_q_heads, n_kv_heads, head_dim, kv_dtype and scale are used.
 *   prompt_len  host [B]: P_b >= 1; 1 <= batch <= 128.
 *   prompt_q    device [sum P_b][Hq][D] fp32.
 *   prompt_k    device [sum P_b][Hkv][D] kv_dtype: the packed prompt h2o_init takes.
 *   out         device [sum P_b][Hkv] fp64; every element is written.
 * Supported: kv_dtype H2O_BF16 with head_dim 128, G in {1, 2, 4, 8}.
 * Scratch: the library keeps one device buffer per device for this call and
 * h2o_snapkv_select (about the size of prompt_q; SnapKV adds up to 16 bytes
 * per prompt position and query head, and with G > 1 one bit per position of
 * the longest prompt for each sequence and query head), grown with
 * hipMallocAsync on `stream` when a call needs more and held until the
 * process ends.  Calls on one device are ordered through it: a call on
 * another stream than the previous call makes its stream wait for the
 * previous call's work.  A SnapKV call that runs in one pass (every P_b <=
 * 1024, w_b <= 32) with G = 1 and the caller's votes uses no scratch and
 * takes no part in this ordering.  Errors: H2O_EINVAL,
 * H2O_ENOMEM, H2O_EDEVICE; the message is h2o_last_error(NULL). */
int h2o_prefill_scores(const h2o_config *cfg, const int32_t *prompt_len, const float *prompt_q,
                       const void *prompt_k, double *out, void *stream);

/* SnapKV's prompt selection ("Attention Sinks and KV cache eviction",
 * sec. 4.3), per sequence b and KV head h, with w_b = min(window, P_b) and the
 * prefix [0, P_b - w_b):
 *   votes     for each query head g of h and prompt position j, the sum over
 *             the window rows i in [P_b - w_b, P_b) of row i's causal softmax
 *             weight on key j (rows as in h2o_prefill_scores, one sum per head);
 *   pooling   each prefix vote replaced by the largest vote of the prefix
 *             positions within pool / 2 of it;
 *   keep      each query head keeps its `keep` prefix positions of highest
 *             pooled vote (equal votes: the lower position);
 *   kept set  the union over the G query heads of h, plus the window.
 *   prompt_q, prompt_k  as h2o_prefill_scores.
 *   votes       device [sum P_b][Hq] fp64 (query head h G + g in column h G + g;
 *               entries of window positions are the window rows' weights on
 *               them), or NULL to use scratch.
 *   kept        device [B][Hkv][cap] int32: kept positions ascending, -1 after.
 *   kept_count  device [B][Hkv] int32.
 *   cap         >= min(P_b, w_b + G min(keep, P_b - w_b)) for every b.
 *   window >= 1, pool odd >= 1, keep >= 0; P_b <= 524288.
 * Supported shapes and errors as h2o_prefill_scores. */
int h2o_snapkv_select(const h2o_config *cfg, const int32_t *prompt_len, int32_t window, int32_t pool,
                      int32_t keep, const float *prompt_q, const void *prompt_k, double *votes,
                      int32_t *kept, int32_t *kept_count, int32_t cap, void *stream);

/* h2o_snapkv_select without any allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops that must not
 * call hipMalloc, harnesses that forbid it.  Arguments, result and errors as
 * h2o_snapkv_select.  Its scratch is a fixed array of 64 MiB (67108864 bytes)
 * in the library, one copy per device, held until the process ends; a call
 * whose scratch need is larger returns H2O_EINVAL with the size in the message
 * before anything is enqueued.  The need is, in bytes, rounded up to 256 each:
 * (votes == NULL ? 8 sum P_b Hq : 0) + (G > 1 ? 4 B Hq ceil(max P_b / 128) * 4
 * : 0) (per-head kept bitmaps), and unless the call runs in one pass (every
 * P_b <= 1024 and w_b <= 32) + 8 sum P_b Hq (pooled votes) + 4160 B Hkv G T
 * (window q tiles and row statistics, T = the most 8-row tiles a window
 * spans, ceil(w_b / 8) + 1 at most).  Calls on one
 * device share that array: two calls whose work overlaps on the device (on
 * different streams, with nothing ordering them) race and give undefined
 * results.  Nothing is cleared between calls (no part of the scratch needs to
 * start at zero).  Errors: H2O_EINVAL, H2O_EDEVICE; the message is
 * h2o_last_error(NULL). */
int h2o_snapkv_select_noalloc(const h2o_config *cfg, const int32_t *prompt_len, int32_t window, int32_t pool,
                              int32_t keep, const float *prompt_q, const void *prompt_k, double *votes,
                              int32_t *kept, int32_t *kept_count, int32_t cap, void *stream);

/* Message of the last error on ctx, or, when ctx is NULL, of the last failed call
 * made without a context (h2o_init, h2o_prefill_scores, h2o_snapkv_select). */
const char *h2o_last_error(const h2o_ctx *ctx);

#ifdef __cplusplus
}
#endif
#endif /* H2O_H */
