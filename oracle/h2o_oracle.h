/*
 * CPU oracle of the H2O decode step -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 reference of what one decode step computes for one
 * (sequence, KV head) unit: append the new token, attend with every query
 * head of the unit's group, add each softmax weight to the token's cumulative
 * score, then evict down to the budget outside the sinks and the recent
 * window (H2O) or, for Random Attention, evict generated tokens at random.
 * Only the tests, the package's smoke check and the benchmark's CPU baseline
 * may load it.  It shares no code with the GPU library.
 *
 * Sources (titles of the pages the method is described on):
 *   "H2O: Heavy-Hitter Oracle for Efficient Generative Inference of LLMs"
 *       (summary page) -- the greedy step over S_{i-1} + {i} with budget K.
 *   "Attention Sinks and KV cache eviction: why a sliding window is not
 *       enough" -- sec. 4.1 (4 sink tokens + recent window), sec. 4.2
 *       (cumulative score over decode steps, top-k of the middle region,
 *       sinks + heavy hitters + recent kept).
 *   "KV Cache compression and selective retention: StreamingLLM vs H2O"
 *       -- the cache-manager listing (4 sinks, heavy hitters by top-k of the
 *       middle scores, recent rows kept).
 *   "Random Attention: rethinking KV cache eviction" -- method (prompt kept,
 *       per-head uniform random eviction of generated tokens) and the
 *       integration notes (period K, buffer r).
 */
#ifndef H2O_ORACLE_H
#define H2O_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_H2O = 0, ORC_RANDOM = 1, ORC_BLOCK = 2 };
enum { ORC_OK = 0, ORC_EARG = -1, ORC_ECHECK = -2, ORC_ENOMEM = -3 };

typedef struct {
    int head_dim;      /* D */
    int group;         /* G: query heads per KV head */
    double scale;      /* logit scale; 0 -> 1/sqrt(D) */
    int selector;      /* ORC_H2O, ORC_RANDOM or ORC_BLOCK (see orc_block_select) */
    int n_sink;        /* H2O: positions 0..n_sink-1 are never evicted */
    int budget_fixed;  /* H2O: > 0 -> budget K fixed ...            */
    int hh_fixed;      /*        ... with this many heavy hitters   */
    int budget_num;    /* H2O: else K_t = floor(len*num/den),       */
    int budget_den;    /*      HH_t = floor((K_t - n_sink)/2)       */
    int rand_k;        /* Random: generated tokens kept after an event (K) */
    int rand_r;        /* Random: buffer r; an event fires at K + r generated */
    uint64_t seed;     /* Random: Philox key word 0 */
    /* Compressed score state (attention-sinks page sec. 6.2: fp32 score state
     * costs 4 MB per 1M tokens; deployments quantise it to FP16/INT8 or replace
     * the exact sum by a moving average): */
    double decay;      /* 0 or 1: exact cumulative sum; else in (0, 1): every retained
                          score is multiplied by decay once per step before that
                          step's weights are added (a moving sum) */
    int score_f16;     /* 1: every score is rounded to IEEE binary16 (nearest, ties to
                          even) after each update, and initial scores on entry */
} orc_cfg;

typedef struct orc_unit orc_unit;

/* Budget K_t, heavy hitters HH_t and recent window W_t at current length len. */
void orc_schedule(const orc_cfg *c, int len, int *K, int *HH, int *W);

/* New unit: sequence b, KV head h, prompt rows pk/pv [prompt_len][D] (fp64),
 * optional initial scores [prompt_len]; cap = most positions it will ever see. */
orc_unit *orc_new(const orc_cfg *c, int b, int h, int prompt_len, int cap,
                  const double *pk, const double *pv, const double *init_scores);
void orc_free(orc_unit *u);

/* Append position t = current length, attend with q [G][D] over the retained
 * set, write out [G][D] and (optionally) probs [G][n_att] in ascending
 * position order, and (H2O) add the weights to the scores.  Returns n_att. */
int orc_attend(orc_unit *u, const double *q, const double *k, const double *v,
               double *out, double *probs);

/* The victims the method picks after orc_attend, in eviction order.
 * Returns e >= 0; *tau = score of the e-th victim (H2O; 0 if e == 0). */
int orc_select(orc_unit *u, int32_t *victims, double *tau);

/* Evict exactly these positions (the oracle's own pick, or an accepted
 * near-tie alternative).  Each must be retained and evictable. */
int orc_evict(orc_unit *u, const int32_t *victims, int e);

/* Post-step invariants: budget, sinks, recent window / prompt, score mass. */
int orc_check(const orc_unit *u);

/* attend + select + evict + check with the oracle's own choice. */
int orc_step(orc_unit *u, const double *q, const double *k, const double *v, double *out);

/* Retained positions ascending (pos), their scores, evicted mass.  Returns count. */
int orc_state(const orc_unit *u, int32_t *pos, double *scores, double *evicted_mass);

/* Score of any position ever seen (frozen once evicted). */
double orc_score_of(const orc_unit *u, int pos);
int orc_length(const orc_unit *u);

/* orc_step on n units, spread over nthreads POSIX threads; returns first error. */
int orc_step_many(orc_unit **u, int n, const double *const *q, const double *const *k,
                  const double *const *v, double *const *out, int nthreads);

/* Block-granular eviction of one sequence ("Attention Sinks and KV cache
 * eviction", sec. 5.1: KV lives in fixed-size blocks, so eviction frees whole
 * blocks; blocks with the lowest share of important tokens go first).  The n
 * units are the KV heads of one sequence (selector ORC_BLOCK, all with the same
 * positions appended and retained; orc_step / orc_select of such a unit never
 * evict).  Block k holds positions [k page, (k + 1) page).  At current length
 * len with budget K, heavy hitters HH and window W (orc_schedule):
 *   - nothing goes while the retained count n <= K;
 *   - candidates: blocks with all `page` positions retained, none of them a
 *     sink (< n_sink) or in the recent window (>= len - W);
 *   - a (token, head) pair is important when the token is among that head's
 *     HH highest-scored candidate tokens (equal scores: the lower position
 *     first), i.e. the heavy hitters token-level eviction would keep;
 *   - a block's importance is its count of important pairs; the
 *     m = min(#candidates, ceil((n - K) / page)) candidates of lowest
 *     importance go (equal importance: the older block first).
 * victims receives the evicted positions in ascending order (at most n);
 * returns their count, or ORC_EARG. */
int orc_block_select(orc_unit *const *u, int n, int page, int32_t *victims);

/* The same rule on given data: n_units score rows of len positions (row i =
 * the scores of head i by position) over the shared retained set live[len]
 * (nonzero = retained) under configuration c's schedule at length len. */
int orc_block_rank(const orc_cfg *c, int len, int page, int n_units, const unsigned char *live,
                   const double *scores, int32_t *victims);

/* Causal-attention column sums of one unit's prompt (P positions):
 * for every query row i in [row_lo, P), every query head g of the group and
 * every key j <= i, the weight softmax_{j' <= i}(scale * q[i][g] . k[j'])[j]
 * is added to out[j] (per_head = 0, summed over the group: out is [P]) or to
 * out[g * P + j] (per_head = 1: out is [G][P]).  out is overwritten.
 *   row_lo = 0, summed: the cumulative attention score each prompt token would
 *     hold had the prompt been scored like decode steps ("Attention Sinks and
 *     KV cache eviction", sec. 4.2 cumulative score, and sec. 4.3 on scores
 *     gathered only during decode);
 *   row_lo = P - w, per head: SnapKV's observation-window vote (sec. 4.3).
 * q: [P][G][D]; k: [P][D].  Returns ORC_OK, or ORC_EARG / ORC_ECHECK (a row's
 * weights not summing to one within 1e-12). */
int orc_colsum(const orc_cfg *c, int P, int row_lo, const double *q, const double *k,
               int per_head, double *out);

/* SnapKV's prompt selection for one unit ("Attention Sinks and KV cache
 * eviction", sec. 4.3): the prompt's last w positions form the observation
 * window; each query head g votes for the prefix positions j < P - w with
 * votes[g][j] (its window rows' attention weights on j, orc_colsum with
 * row_lo = P - w, per head); the votes are max-pooled over the positions
 * within pool / 2 of j (pool odd, clipped at the prefix ends); each head keeps
 * its `keep` prefix positions of highest pooled vote (equal votes: the lower
 * position first); the unit keeps the union over its heads plus the window.
 * votes: [G][P] (entries j >= P - w unused).  kept: receives the kept
 * positions in ascending order (at most P).  Returns the count, or ORC_EARG. */
int orc_snapkv_select(int G, int P, int w, int pool, int keep, const double *votes, int32_t *kept);

/* orc_colsum (row_lo = P - w, per head) followed by orc_snapkv_select; votes
 * receives the [G][P] votes when not NULL.  Returns the count or an error. */
int orc_snapkv(const orc_cfg *c, int P, int w, int pool, int keep, const double *q, const double *k,
               double *votes, int32_t *kept);

/* Philox4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw, SC'11). */
void orc_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]);

/* x rounded to the nearest IEEE binary16 value (ties to even), returned as a
 * double; magnitudes from 65520 on become infinite, as in IEEE rounding to
 * nearest.  out[i] = that of in[i] for i < n. */
double orc_round_f16(double x);
void orc_round_f16_many(const double *in, double *out, int n);

/* Replace the scores of retained positions pos[0..n) by scores[0..n) (the
 * test's lockstep adoption of another implementation's stored, rounded
 * scores, so that its next step starts from the same state).  Each position
 * must be retained.  Returns ORC_OK or ORC_EARG. */
int orc_set_scores(orc_unit *u, const int32_t *pos, const double *scores, int n);

#ifdef __cplusplus
}
#endif
#endif
