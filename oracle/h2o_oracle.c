/*
 * CPU oracle of the H2O decode step -- TEST INFRASTRUCTURE ONLY (see
 * h2o_oracle.h).  fp64 throughout, one (sequence, KV head) unit at a time,
 * no blocking, fusion or reordering beyond what the method states.
 */
#include "h2o_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

struct orc_unit {
    orc_cfg c;
    int b, h, prompt_len, cap;
    double *K, *V;        /* [cap][D]: every position ever appended */
    double *score;        /* [cap]: cumulative attention (frozen once evicted) */
    unsigned char *live;  /* [cap]: 1 = retained */
    int len;              /* positions appended so far (next position = len) */
    int steps;            /* decode steps taken */
    double init_mass;     /* sum of initial scores */
    double evicted_mass;  /* sum of scores of evicted tokens */
    double kept_expect;   /* retained score mass the update rule implies (decay < 1) */
    int *R;               /* scratch: retained positions */
    double *w;            /* scratch: one softmax row */
};

/* ---- budget schedule -----------------------------------------------------
 * H2O summary page: the cache is bounded by a budget K (e.g. 20 % of the
 * sequence).  Sinks/heavy-hitters/recent split: attention-sinks page sec. 4.2
 * and the StreamingLLM-vs-H2O cache manager (4 + HH + recent).  For the
 * proportional budget the pages give no split; K_t = floor(len*num/den) and
 * half of what is left after the sinks goes to heavy hitters (rounded down),
 * the rest to the recent window. */
void orc_schedule(const orc_cfg *c, int len, int *K, int *HH, int *W)
{
    int k, hh;
    if (c->budget_fixed > 0) {
        k = c->budget_fixed;
        hh = c->hh_fixed;
    } else {
        k = (int)(((int64_t)len * c->budget_num) / c->budget_den);
        hh = (k - c->n_sink) / 2;
    }
    *K = k;
    *HH = hh;
    *W = k - c->n_sink - hh;
}

orc_unit *orc_new(const orc_cfg *c, int b, int h, int prompt_len, int cap,
                  const double *pk, const double *pv, const double *init_scores)
{
    if (c->head_dim <= 0 || c->group <= 0 || prompt_len < 0 || cap < prompt_len)
        return NULL;
    if (c->selector == ORC_H2O || c->selector == ORC_BLOCK) {
        if (c->n_sink < 0) return NULL;
        if (c->budget_fixed > 0 &&
            (c->hh_fixed < 0 || c->budget_fixed - c->n_sink - c->hh_fixed < 0))
            return NULL;
        if (c->budget_fixed <= 0 && (c->budget_den <= 0 || c->budget_num < 0)) return NULL;
    } else if (c->selector == ORC_RANDOM) {
        if (c->rand_k < 0 || c->rand_r <= 0) return NULL;
    } else {
        return NULL;
    }
    if (!(c->decay == 0.0 || (c->decay > 0.0 && c->decay <= 1.0))) return NULL;
    if (c->score_f16 != 0 && c->score_f16 != 1) return NULL;
    orc_unit *u = (orc_unit *)calloc(1, sizeof(*u));
    if (!u) return NULL;
    const size_t D = (size_t)c->head_dim;
    u->c = *c;
    if (u->c.scale == 0.0) u->c.scale = 1.0 / sqrt((double)c->head_dim);
    if (u->c.decay == 0.0) u->c.decay = 1.0;
    u->b = b;
    u->h = h;
    u->prompt_len = prompt_len;
    u->cap = cap;
    u->K = (double *)malloc(sizeof(double) * D * (size_t)(cap > 0 ? cap : 1));
    u->V = (double *)malloc(sizeof(double) * D * (size_t)(cap > 0 ? cap : 1));
    u->score = (double *)calloc((size_t)cap + 1, sizeof(double));
    u->live = (unsigned char *)calloc((size_t)cap + 1, 1);
    u->R = (int *)malloc(sizeof(int) * ((size_t)cap + 1));
    u->w = (double *)malloc(sizeof(double) * ((size_t)cap + 1));
    if (!u->K || !u->V || !u->score || !u->live || !u->R || !u->w) {
        orc_free(u);
        return NULL;
    }
    if (prompt_len > 0) {
        memcpy(u->K, pk, sizeof(double) * D * (size_t)prompt_len);
        memcpy(u->V, pv, sizeof(double) * D * (size_t)prompt_len);
    }
    for (int p = 0; p < prompt_len; ++p) {
        u->live[p] = 1;
        u->score[p] = init_scores ? init_scores[p] : 0.0;
        if (u->c.score_f16) u->score[p] = orc_round_f16(u->score[p]);
        u->init_mass += u->score[p];
    }
    u->kept_expect = u->init_mass;
    u->len = prompt_len;
    return u;
}

void orc_free(orc_unit *u)
{
    if (!u) return;
    free(u->K);
    free(u->V);
    free(u->score);
    free(u->live);
    free(u->R);
    free(u->w);
    free(u);
}

static int retained(const orc_unit *u, int *R)
{
    int n = 0;
    for (int p = 0; p < u->len; ++p)
        if (u->live[p]) R[n++] = p;
    return n;
}

/* ---- attention and score accumulation --------------------------------------
 * One new query attends over the retained keys: s_j = scale * q.k_j, softmax
 * over j, output = sum_j p_j v_j (attention-sinks page sec. 3.1: the weights
 * of one query sum to one).  H2O: each weight is added to key j's cumulative
 * score every decode step (attention-sinks page sec. 4.2, step 1); for GQA the
 * weights of the group's query heads are all added to the shared KV head. */
int orc_attend(orc_unit *u, const double *q, const double *k, const double *v,
               double *out, double *probs)
{
    const int D = u->c.head_dim, G = u->c.group;
    if (u->len >= u->cap) return ORC_EARG;
    const int t = u->len;
    memcpy(u->K + (size_t)t * D, k, sizeof(double) * D);
    memcpy(u->V + (size_t)t * D, v, sizeof(double) * D);
    u->score[t] = 0.0;
    u->live[t] = 1;
    u->len = t + 1;

    const int n = retained(u, u->R);
    const int scored = u->c.selector != ORC_RANDOM;  /* H2O and block eviction rank by scores */
    /* moving sum: the retained scores decay once per step, before the step's
     * weights are added (the new token starts from zero) */
    const double lam = u->c.decay;
    if (scored)
        for (int i = 0; i < n; ++i) u->score[u->R[i]] *= lam;
    for (int g = 0; g < G; ++g) {
        const double *qg = q + (size_t)g * D;
        double m = -INFINITY;
        for (int i = 0; i < n; ++i) {
            const double *kj = u->K + (size_t)u->R[i] * D;
            double s = 0.0;
            for (int d = 0; d < D; ++d) s += qg[d] * kj[d];
            s *= u->c.scale;
            u->w[i] = s;
            if (s > m) m = s;
        }
        double z = 0.0;
        for (int i = 0; i < n; ++i) {
            u->w[i] = exp(u->w[i] - m);
            z += u->w[i];
        }
        double total = 0.0;
        for (int i = 0; i < n; ++i) {
            u->w[i] /= z;
            total += u->w[i];
        }
        if (fabs(total - 1.0) > 1e-12) return ORC_ECHECK;
        double *og = out + (size_t)g * D;
        for (int d = 0; d < D; ++d) og[d] = 0.0;
        for (int i = 0; i < n; ++i) {
            const double *vj = u->V + (size_t)u->R[i] * D;
            for (int d = 0; d < D; ++d) og[d] += u->w[i] * vj[d];
        }
        if (probs)
            for (int i = 0; i < n; ++i) probs[(size_t)g * n + i] = u->w[i];
        if (scored)
            for (int i = 0; i < n; ++i) u->score[u->R[i]] += u->w[i];
    }
    /* binary16 storage: each updated score is rounded once */
    if (scored && u->c.score_f16)
        for (int i = 0; i < n; ++i) u->score[u->R[i]] = orc_round_f16(u->score[u->R[i]]);
    u->kept_expect = lam * u->kept_expect + (double)G;  /* each query head's weights sum to one */
    u->steps += 1;
    return n;
}

/* ---- selection ---------------------------------------------------------- */
typedef struct {
    double score;   /* H2O: cumulative score */
    uint64_t key;   /* Random: Philox word */
    int pos;
} cand;

/* Eviction order: smallest first; on equal values the higher position goes
 * first, so the lower position is the one retained. */
static int cmp_score(const void *a, const void *b)
{
    const cand *x = (const cand *)a, *y = (const cand *)b;
    if (x->score < y->score) return -1;
    if (x->score > y->score) return 1;
    return (x->pos > y->pos) ? -1 : (x->pos < y->pos) ? 1 : 0;
}

static int cmp_key(const void *a, const void *b)
{
    const cand *x = (const cand *)a, *y = (const cand *)b;
    if (x->key < y->key) return -1;
    if (x->key > y->key) return 1;
    return (x->pos > y->pos) ? -1 : (x->pos < y->pos) ? 1 : 0;
}

/* Philox4x64-10, SC'11 "Parallel random numbers: as easy as 1, 2, 3":
 * each round multiplies counter words 0 and 2 by the round multipliers, the
 * high halves are xored with the other words and the key, the key is bumped
 * by the Weyl constants between rounds. */
void orc_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4])
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
    const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
    uint64_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint64_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += W0;
            k1 += W1;
        }
        unsigned __int128 p0 = (unsigned __int128)M0 * x0;
        unsigned __int128 p1 = (unsigned __int128)M1 * x2;
        uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        uint64_t y0 = hi1 ^ x1 ^ k0, y1 = lo1, y2 = hi0 ^ x3 ^ k1, y3 = lo0;
        x0 = y0;
        x1 = y1;
        x2 = y2;
        x3 = y3;
    }
    out[0] = x0;
    out[1] = x1;
    out[2] = x2;
    out[3] = x3;
}

/* H2O (H2O summary page, greedy step; attention-sinks page sec. 4.2): with
 * the new token appended, if more than K_t tokens are retained, evict the
 * e = n - K_t retained candidates of lowest cumulative score.  Candidates are
 * retained positions outside the sinks [0, n_sink) and the recent window
 * [len - W_t, len).  Because the retained-set score is a sum, evicting the
 * lowest scores is the greedy choice that maximises what is left.
 *
 * Random Attention (method, modules 1-3; integration notes): the prompt is
 * never evicted; once the retained generated tokens reach K + r, r of them
 * are evicted uniformly at random, per head.  The uniform r-subset is the r
 * smallest of i.i.d. 64-bit Philox words drawn per (sequence, head, step,
 * position). */
int orc_select(orc_unit *u, int32_t *victims, double *tau)
{
    *tau = 0.0;
    const int n = retained(u, u->R);
    const int len = u->len, t = u->len - 1;
    cand *cs = (cand *)malloc(sizeof(cand) * ((size_t)n + 1));
    if (!cs) return ORC_ENOMEM;
    int nc = 0, e = 0;
    if (u->c.selector == ORC_BLOCK) {  /* chosen per sequence: orc_block_select */
        free(cs);
        return 0;
    }
    if (u->c.selector == ORC_H2O) {
        int K, HH, W;
        orc_schedule(&u->c, len, &K, &HH, &W);
        e = n - K;
        if (e > 0) {
            for (int i = 0; i < n; ++i) {
                const int p = u->R[i];
                if (p >= u->c.n_sink && p < len - W) {
                    cs[nc].score = u->score[p];
                    cs[nc].key = 0;
                    cs[nc].pos = p;
                    ++nc;
                }
            }
            if (nc < e) {
                free(cs);
                return ORC_ECHECK;
            }
            qsort(cs, (size_t)nc, sizeof(cand), cmp_score);
            *tau = cs[e - 1].score;
        }
    } else {
        for (int i = 0; i < n; ++i)
            if (u->R[i] >= u->prompt_len) {
                cs[nc].pos = u->R[i];
                cs[nc].score = 0.0;
                ++nc;
            }
        if (nc == u->c.rand_k + u->c.rand_r) {
            const uint64_t key[2] = {u->c.seed, 0};
            for (int i = 0; i < nc; ++i) {
                const uint64_t ctr[4] = {(uint64_t)u->b, (uint64_t)u->h, (uint64_t)t,
                                         (uint64_t)cs[i].pos};
                uint64_t o[4];
                orc_philox4x64_10(ctr, key, o);
                cs[i].key = o[0];
            }
            qsort(cs, (size_t)nc, sizeof(cand), cmp_key);
            e = u->c.rand_r;
        }
    }
    if (e < 0) e = 0;
    for (int i = 0; i < e; ++i) victims[i] = cs[i].pos;
    free(cs);
    return e;
}

static int evictable(const orc_unit *u, int p)
{
    if (p < 0 || p >= u->len || !u->live[p]) return 0;
    if (u->c.selector == ORC_RANDOM) return p >= u->prompt_len;
    int K, HH, W;
    orc_schedule(&u->c, u->len, &K, &HH, &W);
    return p >= u->c.n_sink && p < u->len - W;
}

int orc_evict(orc_unit *u, const int32_t *victims, int e)
{
    for (int i = 0; i < e; ++i)
        if (!evictable(u, victims[i])) return ORC_EARG;
    for (int i = 0; i < e; ++i) {
        u->live[victims[i]] = 0;
        u->evicted_mass += u->score[victims[i]];
        u->kept_expect -= u->score[victims[i]];
    }
    for (int i = 0; i < e; ++i)   /* a repeated victim shows up here */
        if (u->live[victims[i]]) return ORC_EARG;
    return ORC_OK;
}

int orc_check(const orc_unit *u)
{
    int n = 0;
    for (int p = 0; p < u->len; ++p) n += u->live[p];
    if (u->c.selector == ORC_H2O || u->c.selector == ORC_BLOCK) {
        int K, HH, W;
        orc_schedule(&u->c, u->len, &K, &HH, &W);
        /* block eviction bounds the count per sequence (orc_block_select) */
        if (u->c.selector == ORC_H2O && u->steps > 0 && n > K) return ORC_ECHECK;
        for (int p = 0; p < u->c.n_sink && p < u->len; ++p)
            if (!u->live[p]) return ORC_ECHECK;
        for (int p = u->len - W; p < u->len; ++p)
            if (p >= 0 && !u->live[p]) return ORC_ECHECK;
        double kept = 0.0;
        for (int p = 0; p < u->len; ++p)
            if (u->live[p]) kept += u->score[p];
        if (u->c.decay == 1.0 && !u->c.score_f16) {
            /* exact sums: retained + evicted mass = initial mass + G per step */
            const double expect = u->init_mass + (double)u->c.group * u->steps;
            if (fabs(kept + u->evicted_mass - expect) > 1e-9 * (expect > 1.0 ? expect : 1.0))
                return ORC_ECHECK;
        } else if (!u->c.score_f16) {
            /* moving sum: retained mass = decay x previous retained mass + G, less the victims */
            const double ex = u->kept_expect;
            if (fabs(kept - ex) > 1e-9 * (ex > 1.0 ? ex : 1.0)) return ORC_ECHECK;
        }
    } else {
        for (int p = 0; p < u->prompt_len; ++p)
            if (!u->live[p]) return ORC_ECHECK;
        if (n - u->prompt_len >= u->c.rand_k + u->c.rand_r) return ORC_ECHECK;
    }
    return ORC_OK;
}

int orc_step(orc_unit *u, const double *q, const double *k, const double *v, double *out)
{
    int n = orc_attend(u, q, k, v, out, NULL);
    if (n < 0) return n;
    int32_t *vic = (int32_t *)malloc(sizeof(int32_t) * ((size_t)n + 1));
    if (!vic) return ORC_ENOMEM;
    double tau;
    int e = orc_select(u, vic, &tau);
    int rc = e < 0 ? e : orc_evict(u, vic, e);
    free(vic);
    if (rc != ORC_OK) return rc;
    return orc_check(u);
}

int orc_state(const orc_unit *u, int32_t *pos, double *scores, double *evicted_mass)
{
    int n = 0;
    for (int p = 0; p < u->len; ++p)
        if (u->live[p]) {
            if (pos) pos[n] = p;
            if (scores) scores[n] = u->score[p];
            ++n;
        }
    if (evicted_mass) *evicted_mass = u->evicted_mass;
    return n;
}

/* binary16 (IEEE 754): 1 sign bit, 5 exponent bits, 10 fraction bits; normal
 * values 2^-14 .. 65504, subnormals multiples of 2^-24.  A finite value whose
 * leading bit is 2^e is a multiple of the quantum 2^(max(e, -14) - 10), so the
 * nearest value is the quantum times x / quantum rounded to an integer (ties
 * to even: rint in the default rounding mode).  65520, half a quantum above
 * the largest value, and anything larger round to infinity. */
double orc_round_f16(double x)
{
    if (x != x) return x;
    const double a = fabs(x);
    if (a >= 65520.0) return copysign(INFINITY, x);
    if (a == 0.0) return x;
    int E;
    (void)frexp(a, &E);  /* a = m 2^E with m in [0.5, 1): the leading bit is 2^(E - 1) */
    int e = E - 1;
    if (e < -14) e = -14;
    const double q = ldexp(1.0, e - 10);
    return copysign(rint(a / q) * q, x);
}

void orc_round_f16_many(const double *in, double *out, int n)
{
    for (int i = 0; i < n; ++i) out[i] = orc_round_f16(in[i]);
}

int orc_set_scores(orc_unit *u, const int32_t *pos, const double *scores, int n)
{
    for (int i = 0; i < n; ++i)
        if (pos[i] < 0 || pos[i] >= u->len || !u->live[pos[i]]) return ORC_EARG;
    for (int i = 0; i < n; ++i) {
        u->kept_expect += scores[i] - u->score[pos[i]];
        u->score[pos[i]] = scores[i];
    }
    return ORC_OK;
}

double orc_score_of(const orc_unit *u, int pos)
{
    return (pos >= 0 && pos < u->len) ? u->score[pos] : 0.0;
}

int orc_length(const orc_unit *u) { return u->len; }

/* ---- many units in parallel (independent work, no shared state) ---------- */
typedef struct {
    orc_unit **u;
    const double *const *q, *const *k, *const *v;
    double *const *out;
    int n, stride, first, rc;
} job;

static void *run_job(void *arg)
{
    job *j = (job *)arg;
    j->rc = ORC_OK;
    for (int i = j->first; i < j->n; i += j->stride) {
        int rc = orc_step(j->u[i], j->q[i], j->k[i], j->v[i], j->out[i]);
        if (rc < 0 && j->rc == ORC_OK) j->rc = rc;
    }
    return NULL;
}

int orc_step_many(orc_unit **u, int n, const double *const *q, const double *const *k,
                  const double *const *v, double *const *out, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > n) nthreads = n > 0 ? n : 1;
    job *jobs = (job *)calloc((size_t)nthreads, sizeof(job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return ORC_ENOMEM;
    }
    /* started[i]: job i runs on its own thread; a job whose thread could not be
     * created runs here instead, so every unit is stepped exactly once */
    unsigned char *started = (unsigned char *)calloc((size_t)nthreads, 1);
    if (!started) {
        free(jobs);
        free(th);
        return ORC_ENOMEM;
    }
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (job){u, q, k, v, out, n, nthreads, i, ORC_OK};
        if (i > 0) started[i] = pthread_create(&th[i], NULL, run_job, &jobs[i]) == 0;
    }
    run_job(&jobs[0]);
    for (int i = 1; i < nthreads; ++i)
        if (!started[i]) run_job(&jobs[i]);
    int rc = jobs[0].rc;
    for (int i = 1; i < nthreads; ++i) {
        if (started[i]) pthread_join(th[i], NULL);
        if (rc == ORC_OK) rc = jobs[i].rc;
    }
    free(started);
    free(jobs);
    free(th);
    return rc;
}

/* ---- prompt column sums -------------------------------------------------- */
/* Plain definition, one query row at a time: the row's logits over the keys
 * it may see (j <= i), the softmax of that row, then each weight added to its
 * key's column. */
int orc_colsum(const orc_cfg *c, int P, int row_lo, const double *q, const double *k,
               int per_head, double *out)
{
    if (!c || P < 0 || row_lo < 0 || row_lo > P || !q || !k || !out) return ORC_EARG;
    const int D = c->head_dim, G = c->group;
    if (D <= 0 || G <= 0) return ORC_EARG;
    const double scale = c->scale == 0.0 ? 1.0 / sqrt((double)D) : c->scale;
    const size_t n_out = per_head ? (size_t)G * P : (size_t)P;
    for (size_t x = 0; x < n_out; ++x) out[x] = 0.0;
    double *w = (double *)malloc(sizeof(double) * (P > 0 ? (size_t)P : 1));
    if (!w) return ORC_ENOMEM;
    int rc = ORC_OK;
    for (int i = row_lo; i < P && rc == ORC_OK; ++i) {
        for (int g = 0; g < G; ++g) {
            const double *qi = q + ((size_t)i * G + g) * D;
            double m = -INFINITY;
            for (int j = 0; j <= i; ++j) {
                const double *kj = k + (size_t)j * D;
                double s = 0.0;
                for (int d = 0; d < D; ++d) s += qi[d] * kj[d];
                w[j] = scale * s;
                if (w[j] > m) m = w[j];
            }
            double z = 0.0;
            for (int j = 0; j <= i; ++j) {
                w[j] = exp(w[j] - m);
                z += w[j];
            }
            double total = 0.0;
            double *o = per_head ? out + (size_t)g * P : out;
            for (int j = 0; j <= i; ++j) {
                const double p = w[j] / z;
                total += p;
                o[j] += p;
            }
            if (fabs(total - 1.0) > 1e-12) {
                rc = ORC_ECHECK;
                break;
            }
        }
    }
    free(w);
    return rc;
}

/* ---- SnapKV selection ----------------------------------------------------- */
typedef struct {
    double v;
    int pos;
} vote_pos;

/* Keep order: higher vote first; on equal votes the lower position first. */
static int cmp_vote_keep(const void *a, const void *b)
{
    const vote_pos *x = (const vote_pos *)a, *y = (const vote_pos *)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->pos < y->pos) ? -1 : (x->pos > y->pos) ? 1 : 0;
}

int orc_snapkv_select(int G, int P, int w, int pool, int keep, const double *votes, int32_t *kept)
{
    if (G < 1 || P < 1 || w < 1 || w > P || pool < 1 || pool % 2 == 0 || keep < 0 || !votes || !kept)
        return ORC_EARG;
    const int Pp = P - w, r = pool / 2;
    char *mark = (char *)calloc((size_t)P, 1);
    vote_pos *cand = (vote_pos *)malloc(sizeof(vote_pos) * (Pp > 0 ? (size_t)Pp : 1));
    if (!mark || !cand) {
        free(mark);
        free(cand);
        return ORC_ENOMEM;
    }
    for (int g = 0; g < G; ++g) {
        const double *vg = votes + (size_t)g * P;
        for (int j = 0; j < Pp; ++j) {
            double m = -INFINITY;
            for (int x = j - r; x <= j + r; ++x)
                if (x >= 0 && x < Pp && vg[x] > m) m = vg[x];
            cand[j].v = m;
            cand[j].pos = j;
        }
        qsort(cand, (size_t)Pp, sizeof(vote_pos), cmp_vote_keep);
        const int kk = keep < Pp ? keep : Pp;
        for (int i = 0; i < kk; ++i) mark[cand[i].pos] = 1;
    }
    for (int j = Pp; j < P; ++j) mark[j] = 1;
    int n = 0;
    for (int j = 0; j < P; ++j)
        if (mark[j]) kept[n++] = j;
    free(mark);
    free(cand);
    return n;
}

int orc_snapkv(const orc_cfg *c, int P, int w, int pool, int keep, const double *q, const double *k,
               double *votes, int32_t *kept)
{
    if (!c || P < 1 || w < 1 || w > P) return ORC_EARG;
    double *v = votes ? votes : (double *)malloc(sizeof(double) * (size_t)c->group * P);
    if (!v) return ORC_ENOMEM;
    int rc = orc_colsum(c, P, P - w, q, k, 1, v);
    if (rc == ORC_OK) rc = orc_snapkv_select(c->group, P, w, pool, keep, v, kept);
    if (!votes) free(v);
    return rc;
}

/* ---- block-granular eviction ------------------------------------------------ */
typedef struct {
    int imp, block;
} block_rank;

/* Eviction order of candidate blocks: lower importance first, then the older block. */
static int cmp_block(const void *a, const void *b)
{
    const block_rank *x = (const block_rank *)a, *y = (const block_rank *)b;
    if (x->imp != y->imp) return x->imp < y->imp ? -1 : 1;
    return (x->block < y->block) ? -1 : (x->block > y->block) ? 1 : 0;
}

int orc_block_rank(const orc_cfg *c, int len, int page, int n_units, const unsigned char *live,
                   const double *scores, int32_t *victims)
{
    if (!c || len < 0 || page < 1 || n_units < 1 || !live || !scores || !victims) return ORC_EARG;
    int K, HH, W;
    orc_schedule(c, len, &K, &HH, &W);
    int n = 0;
    for (int p = 0; p < len; ++p) n += live[p] != 0;
    if (n <= K) return 0;
    const int nb = (len + page - 1) / page;
    char *cand = (char *)calloc((size_t)nb + 1, 1);
    int *imp = (int *)calloc((size_t)nb + 1, sizeof(int));
    vote_pos *tok = (vote_pos *)malloc(sizeof(vote_pos) * ((size_t)len + 1));
    block_rank *br = (block_rank *)malloc(sizeof(block_rank) * ((size_t)nb + 1));
    if (!cand || !imp || !tok || !br) {
        free(cand);
        free(imp);
        free(tok);
        free(br);
        return ORC_ENOMEM;
    }
    /* candidates: whole retained blocks outside the sinks and the recent window */
    int ncand = 0;
    for (int k = 0; k < nb; ++k) {
        const int lo = k * page, hi = lo + page - 1;
        int full = hi < len;
        for (int p = lo; full && p <= hi && p < len; ++p) full = live[p] != 0;
        cand[k] = full && lo >= c->n_sink && hi < len - W;
        ncand += cand[k];
    }
    /* importance: per head, its HH best candidate tokens count once each */
    for (int i = 0; i < n_units; ++i) {
        const double *sc = scores + (size_t)i * len;
        int nt = 0;
        for (int p = 0; p < len; ++p)
            if (cand[p / page]) {
                tok[nt].v = sc[p];
                tok[nt].pos = p;
                ++nt;
            }
        qsort(tok, (size_t)nt, sizeof(vote_pos), cmp_vote_keep);
        const int hh = HH < nt ? HH : nt;
        for (int x = 0; x < hh; ++x) imp[tok[x].pos / page] += 1;
    }
    /* the least important candidate blocks go, older first on equal importance */
    int nr = 0;
    for (int k = 0; k < nb; ++k)
        if (cand[k]) {
            br[nr].imp = imp[k];
            br[nr].block = k;
            ++nr;
        }
    qsort(br, (size_t)nr, sizeof(block_rank), cmp_block);
    const int need = (n - K + page - 1) / page;
    const int m = need < ncand ? need : ncand;
    for (int k = 0; k < nb; ++k) cand[k] = 0; /* reused: the evicted blocks */
    for (int x = 0; x < m; ++x) cand[br[x].block] = 1;
    int e = 0;
    for (int p = 0; p < len; ++p)
        if (cand[p / page]) victims[e++] = p;
    free(cand);
    free(imp);
    free(tok);
    free(br);
    return e;
}

int orc_block_select(orc_unit *const *u, int n_units, int page, int32_t *victims)
{
    if (!u || n_units < 1 || page < 1 || !victims) return ORC_EARG;
    const orc_unit *u0 = u[0];
    const int len = u0->len;
    for (int i = 1; i < n_units; ++i) {
        if (u[i]->len != len) return ORC_EARG;
        for (int p = 0; p < len; ++p)
            if (u[i]->live[p] != u0->live[p]) return ORC_EARG;
    }
    double *sc = (double *)malloc(sizeof(double) * ((size_t)n_units * len + 1));
    if (!sc) return ORC_ENOMEM;
    for (int i = 0; i < n_units; ++i)
        memcpy(sc + (size_t)i * len, u[i]->score, sizeof(double) * (size_t)len);
    const int e = orc_block_rank(&u0->c, len, page, n_units, u0->live, sc, victims);
    free(sc);
    return e;
}
