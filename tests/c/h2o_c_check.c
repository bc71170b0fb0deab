/* A C client of libh2o.so: only include/h2o.h and the HIP runtime, no Python.
 *
 * Runs H2O decode steps on seeded inputs and checks, after every step, what
 * the method fixes whatever the numbers ("Attention Sinks and KV cache
 * eviction", sec. 4.2; "H2O: Heavy-Hitter Oracle"):
 *   - the retained count is min(n_att, K_t) (the budget at the new length);
 *   - positions are ascending, distinct and no later than the newest token;
 *   - the n_sink first positions and the recent window are all retained;
 *   - retained scores plus evicted mass equal G x (steps done) for every
 *     (sequence, KV head): each query head's softmax adds a total weight of 1;
 *   - every output element is finite.
 * Exit status 0 and "c check ok" on success.  Needs a GPU. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "h2o.h"

#define D 128

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static float uniform01(void)
{
    /* xorshift64*: a seeded generator for test inputs only */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (float)((rng_state * 0x2545F4914F6CDD1Dull) >> 40) / 16777216.0f;
}

static float normalish(void) { return (uniform01() + uniform01() + uniform01() - 1.5f) * 2.0f; }

static uint16_t bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

#define HIP_OK(x)                                                                \
    do {                                                                         \
        hipError_t e_ = (x);                                                     \
        if (e_ != hipSuccess) {                                                  \
            fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__);     \
            exit(2);                                                             \
        }                                                                        \
    } while (0)

static int fails = 0;
#define CHECK(cond, ...)                          \
    do {                                          \
        if (!(cond)) {                            \
            fprintf(stderr, __VA_ARGS__);         \
            fputc('\n', stderr);                  \
            if (++fails > 20) exit(1);            \
        }                                         \
    } while (0)

/* budget K, heavy hitters HH and window W at length len (as documented in h2o.h) */
static void schedule(const h2o_config* c, int len, int* K, int* W)
{
    int k, hh;
    if (c->budget_fixed > 0) {
        k = c->budget_fixed;
        hh = c->hh_fixed;
    } else {
        k = (int)(((long long)len * c->budget_num) / c->budget_den);
        hh = (k - c->n_sink) / 2;
    }
    *K = k;
    *W = k - c->n_sink - hh;
}

static void run(const char* name, h2o_config cfg, const int32_t* plen, int steps, int fused)
{
    const int B = cfg.batch, Hq = cfg.n_q_heads, Hkv = cfg.n_kv_heads, G = Hq / Hkv;
    long long total = 0;
    for (int b = 0; b < B; ++b) total += plen[b];
    size_t pk_n = (size_t)total * Hkv * D;
    uint16_t* hk = malloc(pk_n * 2);
    uint16_t* hv = malloc(pk_n * 2);
    for (size_t i = 0; i < pk_n; ++i) {
        hk[i] = bf16(normalish());
        hv[i] = bf16(normalish());
    }
    void *dk, *dv, *dq, *dkn, *dvn, *dout;
    HIP_OK(hipMalloc(&dk, pk_n * 2));
    HIP_OK(hipMalloc(&dv, pk_n * 2));
    HIP_OK(hipMemcpy(dk, hk, pk_n * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dv, hv, pk_n * 2, hipMemcpyHostToDevice));
    h2o_ctx* ctx = NULL;
    int rc = h2o_init(&ctx, &cfg, plen, dk, dv, NULL, NULL);
    if (rc != H2O_OK) {
        fprintf(stderr, "%s: h2o_init: %d %s\n", name, rc, h2o_last_error(NULL));
        exit(1);
    }
    int32_t cap = 0, done = 0, pages = 0;
    h2o_info(ctx, &cap, &done, &pages);
    const size_t nq = (size_t)B * Hq * D, nkv = (size_t)B * Hkv * D;
    float* hq = malloc(nq * 4);
    float* hout = malloc(nq * 4);
    uint16_t* hkn = malloc(nkv * 2);
    uint16_t* hvn = malloc(nkv * 2);
    HIP_OK(hipMalloc(&dq, nq * 4));
    HIP_OK(hipMalloc(&dout, nq * 4));
    HIP_OK(hipMalloc(&dkn, nkv * 2));
    HIP_OK(hipMalloc(&dvn, nkv * 2));
    int32_t* pos = malloc((size_t)B * Hkv * cap * 4);
    int32_t* cnt = malloc((size_t)B * 4);
    double* sc = malloc((size_t)B * Hkv * cap * 8);
    double* em = malloc((size_t)B * Hkv * 8);
    int32_t* count = malloc((size_t)B * 4);
    for (int b = 0; b < B; ++b) count[b] = plen[b];

    for (int s = 0; s < steps; ++s) {
        for (size_t i = 0; i < nq; ++i) hq[i] = normalish();
        for (size_t i = 0; i < nkv; ++i) {
            hkn[i] = bf16(normalish());
            hvn[i] = bf16(normalish());
        }
        HIP_OK(hipMemcpy(dq, hq, nq * 4, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(dkn, hkn, nkv * 2, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(dvn, hvn, nkv * 2, hipMemcpyHostToDevice));
        if (fused) {
            rc = h2o_step_compact(ctx, dq, dkn, dvn, dout, NULL);
        } else {
            rc = h2o_step(ctx, dq, dkn, dvn, dout, NULL);
            if (rc == H2O_OK) rc = h2o_compact(ctx, NULL);
        }
        if (rc != H2O_OK) {
            fprintf(stderr, "%s: step %d: %d %s\n", name, s, rc, h2o_last_error(ctx));
            exit(1);
        }
        rc = h2o_read_indices(ctx, pos, cnt, sc, em, (size_t)cap, NULL);
        if (rc != H2O_OK) {
            fprintf(stderr, "%s: read: %d %s\n", name, rc, h2o_last_error(ctx));
            exit(1);
        }
        HIP_OK(hipMemcpy(hout, dout, nq * 4, hipMemcpyDeviceToHost));
        for (size_t i = 0; i < nq; ++i) CHECK(isfinite(hout[i]), "%s: step %d: output %zu not finite", name, s, i);
        for (int b = 0; b < B; ++b) {
            const int t = plen[b] + s, len = t + 1;
            int K, W;
            schedule(&cfg, len, &K, &W);
            const int n_att = count[b] + 1;
            const int want = n_att < K ? n_att : K;
            CHECK(cnt[b] == want, "%s: step %d seq %d: count %d, want %d", name, s, b, cnt[b], want);
            count[b] = cnt[b];
            for (int h = 0; h < Hkv; ++h) {
                const int32_t* p = pos + ((size_t)b * Hkv + h) * cap;
                const double* q = sc + ((size_t)b * Hkv + h) * cap;
                double mass = em[b * Hkv + h];
                int sinks = 0, window = 0;
                for (int i = 0; i < cnt[b]; ++i) {
                    CHECK(p[i] >= 0 && p[i] <= t, "%s: step %d (%d,%d): position %d out of range", name, s, b, h, p[i]);
                    if (i > 0) CHECK(p[i] > p[i - 1], "%s: step %d (%d,%d): positions not ascending", name, s, b, h);
                    if (p[i] < cfg.n_sink) ++sinks;
                    if (p[i] >= len - W) ++window;
                    mass += q[i];
                }
                const int want_sinks = cfg.n_sink < len ? cfg.n_sink : len;
                const int want_window = W < len ? W : len;
                CHECK(sinks == want_sinks, "%s: step %d (%d,%d): %d sinks kept, want %d", name, s, b, h, sinks, want_sinks);
                CHECK(window >= want_window, "%s: step %d (%d,%d): %d of the %d window positions kept", name, s, b,
                      h, window, want_window);
                const double want_mass = (double)G * (s + 1);
                CHECK(fabs(mass - want_mass) <= 1e-4 * want_mass, "%s: step %d (%d,%d): mass %.9f, want %.1f", name,
                      s, b, h, mass, want_mass);
            }
        }
    }
    h2o_destroy(ctx);
    HIP_OK(hipFree(dk));
    HIP_OK(hipFree(dv));
    HIP_OK(hipFree(dq));
    HIP_OK(hipFree(dout));
    HIP_OK(hipFree(dkn));
    HIP_OK(hipFree(dvn));
    free(hk), free(hv), free(hq), free(hout), free(hkn), free(hvn), free(pos), free(cnt), free(sc), free(em), free(count);
    printf("%s: %d steps checked\n", name, steps);
}

int main(void)
{
    h2o_config c;
    memset(&c, 0, sizeof c);
    c.head_dim = D;
    c.kv_dtype = H2O_BF16;
    c.selector = H2O_SEL_H2O;
    c.n_sink = 4;

    /* GQA group of 4 (matrix-core path), fixed budget 64 = 4 + 28 + 32, fp64 scores */
    h2o_config g = c;
    g.batch = 3;
    g.n_q_heads = 8;
    g.n_kv_heads = 2;
    g.score_dtype = H2O_F64;
    g.budget_fixed = 64;
    g.hh_fixed = 28;
    g.max_len = 400;
    const int32_t gl[3] = {100, 40, 64};
    run("gqa4_fixed", g, gl, 90, 1);

    /* one query head per KV head (FMA path), budget 20 % of the length, fp32 scores */
    h2o_config m = c;
    m.batch = 2;
    m.n_q_heads = 4;
    m.n_kv_heads = 4;
    m.score_dtype = H2O_F32;
    m.budget_num = 1;
    m.budget_den = 5;
    m.max_len = 600;
    const int32_t ml[2] = {300, 130};
    run("mha_20pct_fused", m, ml, 60, 1);
    run("mha_20pct_step_then_compact", m, ml, 60, 0);

    if (fails) {
        fprintf(stderr, "%d check(s) failed\n", fails);
        return 1;
    }
    printf("c check ok\n");
    return 0;
}
