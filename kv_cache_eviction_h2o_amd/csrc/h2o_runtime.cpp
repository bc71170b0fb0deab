// Host runtime of libh2o.so: the C ABI declared in include/h2o.h.
//
// The host keeps a mirror of every sequence's position and retained count.
// Because the budget schedule depends only on (position, configuration), the
// host knows each step's eviction count e_b -- and so the page demand of the
// paged layout -- without reading anything back from the device: a step is
// pure enqueue work.  Pages are handed out and taken back here; a new page id
// travels to the kernel in its arguments.  Under block eviction the device
// picks which pages go, so free pages live on a device stack; the host still
// knows how many pages each step takes and frees, and so the stack's depth.
#include "h2o.h"
#include "h2o_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

using namespace h2o;

struct h2o_ctx {
    h2o_config cfg{};
    Geometry g{};
    State s{};
    Sched sc{};
    int device = 0;
    float qscale = 0.f;
    std::vector<int> plen;    // P_b
    std::vector<int> count;   // retained slots per sequence (all its heads)
    int step = 0;             // decode steps completed
    bool pending = false;     // h2o_step done, h2o_compact not yet
    std::vector<int> pend_e;  // e_b of the pending step
    std::vector<std::vector<int>> pages;  // paged: page ids of each sequence, in slot order
    std::vector<int> free_pages;
    // block eviction: pages are tracked by count (the device stack holds the ids)
    bool block = false;
    int js = 0;                // block-table entries holding sink positions
    int ftop = 0;              // depth of the device free-page stack
    std::vector<int> evb;      // pages evicted so far per sequence
    BlockArgs pend_blk{};      // the pending step's block eviction (h2o_compact)
    std::vector<int> pend_n;   // block eviction, step pending: counts before the eviction
    std::vector<void*> allocs;   // hipMalloc'd state (none when the caller gave a workspace)
    // state placement: measure only (h2o_workspace_size), carve from the
    // caller's workspace, or hipMalloc each buffer
    bool measure = false;
    size_t need = 0;
    char* ws = nullptr;
    size_t ws_bytes = 0, ws_used = 0;
    std::string err;
};

namespace {

std::mutex g_err_mu;
std::string g_init_err;

int fail(h2o_ctx* c, int code, const std::string& msg)
{
    if (c) {
        c->err = msg;
    } else {
        std::lock_guard<std::mutex> lk(g_err_mu);
        g_init_err = msg;
    }
    return code;
}

// Device arguments are read and written with 16-byte vector accesses.
bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

int hip_fail(h2o_ctx* c, hipError_t e, const char* what)
{
    std::string m = std::string(what) + ": " + hipGetErrorString(e);
    return fail(c, e == hipErrorOutOfMemory ? H2O_ENOMEM : H2O_EDEVICE, m);
}

struct DeviceGuard {
    int prev = -1;
    explicit DeviceGuard(int dev)
    {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        if (prev != dev) (void)hipSetDevice(dev);
    }
    ~DeviceGuard()
    {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

Sched make_sched(const h2o_config& c)
{
    Sched s{};
    s.selector = c.selector;
    s.n_sink = c.n_sink;
    s.budget_fixed = c.budget_fixed;
    s.hh_fixed = c.hh_fixed;
    s.budget_num = c.budget_num;
    s.budget_den = c.budget_den;
    s.rand_k = c.rand_k;
    s.rand_r = c.rand_r;
    s.seed = (unsigned long long)c.seed;
    s.decay = c.score_decay > 0.f ? c.score_decay : 1.0f;
    return s;
}

// Block-table entries that hold sink positions (block eviction never takes them).
int sink_pages(int n_sink) { return (n_sink + kPageSize - 1) >> kPageShift; }

// Most slots a (b, h) unit can hold during the run (the pre-eviction set).
long long slot_capacity(const h2o_config& c, int maxP)
{
    long long cap;
    if (c.selector == H2O_SEL_H2O || c.selector == H2O_SEL_BLOCK) {
        long long kmax = c.budget_fixed > 0 ? c.budget_fixed
                                             : ((long long)c.max_len * c.budget_num) / c.budget_den;
        // block eviction: after a step either n <= K, or every candidate page is
        // gone and what is left is the sinks' pages plus the pages from the
        // window's first full page on (at most W + 15 positions), W <= K
        if (c.selector == H2O_SEL_BLOCK) kmax += (long long)sink_pages(c.n_sink) * kPageSize + kPageSize - 1;
        cap = std::max<long long>(maxP, kmax) + 1;
    } else {
        cap = (long long)maxP + c.rand_k + c.rand_r;
    }
    return std::min<long long>(cap, c.max_len);
}

int validate(const h2o_config* c, const int32_t* plen, std::string& why)
{
    auto bad = [&](const char* m) {
        why = m;
        return H2O_EINVAL;
    };
    if (!c || !plen) return bad("null config or prompt_len");
    if (c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1) return bad("batch and heads must be >= 1");
    if (c->n_q_heads % c->n_kv_heads) return bad("n_q_heads must be a multiple of n_kv_heads");
    const int G = c->n_q_heads / c->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return bad("query group size must be 1, 2, 4 or 8");
    const bool bf = c->kv_dtype == H2O_BF16, f32 = c->kv_dtype == H2O_F32, i8 = c->kv_dtype == H2O_I8;
    if (!((bf || i8) && c->head_dim == 128) && !(f32 && c->head_dim == 64))
        return bad("supported (kv_dtype, head_dim): (bf16, 128), (i8, 128) or (f32, 64)");
    if (!(c->scale >= 0.f) || !std::isfinite(c->scale)) return bad("scale must be finite and >= 0");
    if (c->max_len < 2) return bad("max_len must be >= 2");
    int maxP = 0;
    for (int b = 0; b < c->batch; ++b) {
        if (plen[b] < 1) return bad("every prompt length must be >= 1");
        if (plen[b] >= c->max_len) return bad("prompt length must be < max_len");
        maxP = std::max(maxP, (int)plen[b]);
    }
    if (c->selector == H2O_SEL_BLOCK && c->page_size != kPageSize)
        return bad("block eviction needs the paged layout (page_size 16)");
    if (c->selector == H2O_SEL_BLOCK && c->n_kv_heads > 1024)
        return bad("block eviction supports at most 1024 KV heads");
    if (c->selector == H2O_SEL_H2O || c->selector == H2O_SEL_BLOCK) {
        if (c->score_dtype == H2O_F16 && c->selector != H2O_SEL_H2O)
            return bad("binary16 scores (score_dtype f16) need the H2O selector");
        if (c->score_dtype != H2O_F32 && c->score_dtype != H2O_F64 && c->score_dtype != H2O_F16)
            return bad("score_dtype must be f32, f64 or f16");
        if (!(c->score_decay >= 0.f && c->score_decay <= 1.f))
            return bad("score_decay must be 0 (exact sum) or in (0, 1]");
        if (c->n_sink < 0) return bad("n_sink must be >= 0");
        if (c->budget_fixed > 0) {
            if (c->hh_fixed < 0 || c->budget_fixed - c->n_sink - c->hh_fixed < 0)
                return bad("fixed budget needs 0 <= hh_fixed <= budget_fixed - n_sink");
        } else {
            if (c->budget_den <= 0 || c->budget_num <= 0 || c->budget_num > c->budget_den)
                return bad("proportional budget needs 0 < budget_num <= budget_den");
            // K_t is non-decreasing; the first step of the shortest prompt is the smallest.
            int minP = maxP;
            for (int b = 0; b < c->batch; ++b) minP = std::min(minP, (int)plen[b]);
            const long long k0 = ((long long)(minP + 1) * c->budget_num) / c->budget_den;
            if (k0 < (long long)c->n_sink + 1) return bad("budget at the first step is below n_sink + 1");
        }
        if (c->budget_fixed > 0 && c->budget_fixed < 1) return bad("budget must be >= 1");
    } else if (c->selector == H2O_SEL_RANDOM) {
        if (c->rand_k < 0 || c->rand_r < 1) return bad("Random needs rand_k >= 0 and rand_r >= 1");
    } else {
        return bad("unknown selector");
    }
    if (c->page_size != 0 && c->page_size != kPageSize) return bad("page_size must be 0 or 16");
    if (c->workspace && (reinterpret_cast<uintptr_t>(c->workspace) & 255) != 0)
        return bad("workspace must be 256-byte aligned");
    if (c->page_size) {
        if (!bf && !i8) return bad("the paged layout needs bf16 or i8 rows");
        if (c->batch > kMaxArgBatch) return bad("paged layout supports at most 128 sequences");
        if (c->max_pages < 1) return bad("paged layout needs max_pages >= 1");
    }
    const long long cap = slot_capacity(*c, maxP);
    if (cap > (1LL << 30)) return bad("slot capacity too large");
    // contiguous units are read through raw buffer descriptors whose size and
    // offsets are 32-bit: a unit's rows must stay below 2^31 bytes
    if (!c->page_size && cap * (long long)(i8 ? kRowBytesI8 : kRowBytes) >= (1LL << 31))
        return bad("contiguous slot capacity too large: a unit's K (or V) rows must stay below 2^31 bytes "
                   "(use the paged layout)");
    if (c->selector == H2O_SEL_BLOCK && (cap + kPageSize - 1) / kPageSize > kMaxBlockPages)
        return bad("block eviction supports at most 5120 pages (81920 slots) per sequence");
    return H2O_OK;
}

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <typename T>
int dalloc(h2o_ctx* c, T** p, size_t bytes, const char* what)
{
    *p = nullptr;
    if (bytes == 0) return H2O_OK;
    if (c->measure) {  // buffers start on 256-byte boundaries, as carved below
        c->need = align256(c->need) + bytes;
        return H2O_OK;
    }
    if (c->ws) {
        const size_t off = align256(c->ws_used);
        if (off > c->ws_bytes || bytes > c->ws_bytes - off)
            return fail(c, H2O_EINVAL, std::string(what) + ": workspace too small");
        *p = (T*)(c->ws + off);
        c->ws_used = off + bytes;
        return H2O_OK;
    }
    void* v = nullptr;
    hipError_t e = hipMalloc(&v, bytes);
    if (e != hipSuccess) return hip_fail(c, e, what);
    c->allocs.push_back(v);
    *p = (T*)v;
    return H2O_OK;
}

void release_pages(h2o_ctx* c, int b)
{
    const size_t need = (size_t)((c->count[b] + kPageSize - 1) >> kPageShift);
    auto& pg = c->pages[b];
    while (pg.size() > need) {
        c->free_pages.push_back(pg.back());
        pg.pop_back();
    }
}

void free_all(h2o_ctx* c)
{
    for (void* p : c->allocs) (void)hipFree(p);
    c->allocs.clear();
}

// Retained slots of sequence b as the device holds them now: with a block
// eviction pending, the step's appended state before any page goes.
int visible_count(const h2o_ctx* c, int b)
{
    return (c->pending && c->block) ? c->pend_n[b] : c->count[b];
}

// Block eviction after the step that appends position t_b = P_b + step (see
// h2o_block.hip): per sequence, the candidate pages are the whole pages past
// the sinks' pages that end before the recent window, less those evicted so
// far (all of them lay before the window, whose start never moves back), and
// min(candidates, ceil((n - K) / 16)) of them go.  Updates the host's counts,
// evicted pages and free-stack depth; returns the launch arguments.
BlockArgs plan_blocks(h2o_ctx* c)
{
    BlockArgs ba{};
    ba.g = c->g;
    ba.s = c->s;
    ba.sc = c->sc;
    ba.js = c->js;
    int pushed = 0;
    for (int b = 0; b < c->g.B; ++b) {
        const int len = c->plen[b] + c->step + 1;
        const int n_att = c->count[b] + 1;
        int K, HH, W;
        schedule(c->sc, len, K, HH, W);
        int m = 0, nc = 0;
        if (n_att > K) {
            const int kb = len - W > 0 ? (len - W) >> kPageShift : 0;  // pages ending before the window
            nc = std::max(0, kb - c->js) - c->evb[b];
            m = std::min(nc, (n_att - K + kPageSize - 1) >> kPageShift);
        }
        c->count[b] = n_att - m * kPageSize;
        if (m <= 0) continue;
        const int i = ba.nseq++;
        ba.seq_b[i] = b;
        ba.seq_len[i] = len;
        ba.seq_n[i] = n_att;
        ba.seq_c[i] = nc;
        ba.seq_m[i] = m;
        ba.seq_push[i] = c->ftop + pushed;
        pushed += m;
        c->evb[b] += m;
    }
    c->ftop += pushed;
    return ba;
}

int do_step(h2o_ctx* c, const float* q, const void* kn, const void* vn, float* out, void* stream,
            bool fused)
{
    if (!c) return H2O_EINVAL;
    if (c->pending) return fail(c, H2O_ESTATE, "a compaction is pending: call h2o_compact first");
    if (!q || !kn || !vn || !out) return fail(c, H2O_EINVAL, "null q, k_new, v_new or out");
    if (misaligned(q) || misaligned(kn) || misaligned(vn) || misaligned(out))
        return fail(c, H2O_EINVAL, "q, k_new, v_new and out must be 16-byte aligned");
    const int B = c->g.B;
    std::vector<int> e(B);
    int max_n_att = 0;
    for (int b = 0; b < B; ++b) {
        const int t = c->plen[b] + c->step;
        if (t + 1 > c->cfg.max_len) return fail(c, H2O_EINVAL, "a sequence would pass max_len");
        const int n_att = c->count[b] + 1;
        if (n_att > c->g.cap) return fail(c, H2O_EINVAL, "slot capacity exceeded");
        e[b] = evict_count(c->sc, t, c->plen[b], n_att);
        max_n_att = std::max(max_n_att, n_att);
    }
    DeviceGuard dg(c->device);
    StepArgs a{};
    a.g = c->g;
    a.s = c->s;
    a.sc = c->sc;
    a.q = q;
    a.kn = kn;
    a.vn = vn;
    a.out = out;
    a.qscale = c->qscale;
    a.step = c->step;
    a.fused = fused ? 1 : 0;
    a.lds_n = (max_n_att + 3) & ~3;
    a.npg_lds = (max_n_att + kPageSize - 1) >> kPageShift;
    int32_t newpage[kMaxArgBatch];
    for (int i = 0; i < kMaxArgBatch; ++i) newpage[i] = -1;
    a.seq_in_args = B <= kMaxArgBatch ? 1 : 0;
    a.pop_stack = 0;
    // the first fused step of paged H2O keeps the recent window's pages where
    // they are (window_remap) and relinks them after the step
    a.remap = (c->g.paged && !c->block && fused && c->sc.selector == H2O_SEL_H2O && c->step == 0 &&
               B <= kMaxArgBatch)
                  ? 1
                  : 0;
    std::vector<char> relink(B, 0);
    std::vector<WindowRemap> rmap(B);
    for (int b = 0; b < B && a.remap; ++b) {
        relink[b] = window_remap(c->sc, c->plen[b] + c->step, c->count[b] + 1, e[b], rmap[b]) ? 1 : 0;
        // the window lies in the row (its pages, the appended one included, exist)
        const size_t rows = (size_t)((c->count[b] + 1 + kPageSize - 1) >> kPageShift);
        if (relink[b] && (size_t)((rmap[b].src + rmap[b].m + kPageSize - 1) >> kPageShift) > rows)
            return fail(c, H2O_EDEVICE, "page relink out of range");
    }
    std::vector<int> got;  // sequences given a page in this call (returned if the launch fails)
    if (c->block) {
        // every block-table entry but the last is full: a sequence needs a page
        // when its count is a multiple of 16; pages come off the device stack
        int demand = 0;
        for (int b = 0; b < B; ++b) demand += (c->count[b] & (kPageSize - 1)) == 0 ? 1 : 0;
        if (demand > c->ftop) return fail(c, H2O_ENOMEM, "KV page pool exhausted");
        a.pop_stack = 1;
        int k = 0;
        for (int b = 0; b < B; ++b)
            if ((c->count[b] & (kPageSize - 1)) == 0) newpage[b] = c->ftop - 1 - k++;
    } else if (c->g.paged) {
        int demand = 0;
        std::vector<char> need(B, 0);
        for (int b = 0; b < B; ++b) {
            const bool inplace = fused && c->sc.selector == H2O_SEL_H2O && e[b] == 1;
            const int n = c->count[b];
            if (!inplace && (n & (kPageSize - 1)) == 0 && (size_t)(n >> kPageShift) == c->pages[b].size()) {
                need[b] = 1;
                ++demand;
            }
        }
        if ((size_t)demand > c->free_pages.size())
            return fail(c, H2O_ENOMEM, "KV page pool exhausted");
        for (int b = 0; b < B; ++b)
            if (need[b]) {
                const int p = c->free_pages.back();
                c->free_pages.pop_back();
                c->pages[b].push_back(p);
                newpage[b] = p;
                got.push_back(b);
            }
    }
    if (a.seq_in_args) {
        // workgroups of the longest sequences first (a workgroup's time grows with its count)
        std::vector<int> ord(B);
        for (int b = 0; b < B; ++b) ord[b] = b;
        std::stable_sort(ord.begin(), ord.end(), [&](int x, int y) { return c->count[x] > c->count[y]; });
        for (int i = 0; i < B; ++i) {
            const int b = ord[i];
            a.seq[i] = SeqArg{b, c->count[b], c->plen[b], newpage[b]};
        }
    }
    hipError_t err = launch_step(a, max_n_att, (hipStream_t)stream);
    if (err != hipSuccess) {  // nothing ran: the pages go back as they came
        for (auto it = got.rbegin(); it != got.rend(); ++it) {
            c->free_pages.push_back(c->pages[*it].back());
            c->pages[*it].pop_back();
        }
        return hip_fail(c, err, "step kernel launch");
    }
    if (c->block) {
        for (int b = 0; b < B; ++b) c->ftop -= (c->count[b] & (kPageSize - 1)) == 0 ? 1 : 0;
        BlockArgs ba = plan_blocks(c);  // updates counts, evicted pages and the stack depth
        if (c->ftop > c->cfg.max_pages)  // the pool's pages are all accounted for: cannot happen
            return fail(c, H2O_EDEVICE, "free-page accounting out of range");
        if (fused) {
            if ((err = launch_block(ba, (hipStream_t)stream)) != hipSuccess)
                return hip_fail(c, err, "block eviction launch");
            c->step += 1;
        } else {
            c->pending = true;
            c->pend_blk = ba;
            c->pend_n.resize(B);
            for (int b = 0; b < B; ++b) c->pend_n[b] = c->count[b];
            for (int i = 0; i < ba.nseq; ++i) c->pend_n[ba.seq_b[i]] = ba.seq_n[i];
        }
        return H2O_OK;
    }
    if (fused) {
        RemapArgs ra{};
        ra.bt = c->s.bt;
        ra.maxp = c->g.maxp;
        for (int b = 0; b < B; ++b) {
            if (relink[b]) {
                // the mirror of the relinked row: the front pages, then the
                // window's; the pages in between and after go back to the pool
                const WindowRemap& r = rmap[b];
                auto& pg = c->pages[b];
                const int f = r.front >> kPageShift, src = r.src >> kPageShift;
                const int cnt = (r.m + kPageSize - 1) >> kPageShift;
                std::vector<int> kept(pg.begin(), pg.begin() + f);
                kept.insert(kept.end(), pg.begin() + src, pg.begin() + src + cnt);
                for (int k = (int)pg.size() - 1; k >= 0; --k)
                    if (k >= src + cnt || (k >= f && k < src)) c->free_pages.push_back(pg[k]);
                pg.swap(kept);
                ra.seq_b[ra.nseq] = b;
                ra.seq_front[ra.nseq] = f;
                ra.seq_src[ra.nseq] = src;
                ra.seq_cnt[ra.nseq] = cnt;
                ++ra.nseq;
            }
            c->count[b] = c->count[b] + 1 - e[b];
            if (c->g.paged) release_pages(c, b);
        }
        if (ra.nseq > 0 && (err = launch_remap(ra, (hipStream_t)stream)) != hipSuccess)
            return hip_fail(c, err, "page relink launch");
        c->step += 1;
    } else {
        c->pending = true;
        c->pend_e = e;
    }
    return H2O_OK;
}


// Scratch of the prompt calls (h2o_prefill_scores, h2o_snapkv_select): one
// grow-only device buffer per device, kept until the process ends, so a call
// allocates nothing once a call at least as large has run (a stream-ordered
// allocation and release per call cost more host time than the kernels take).
// The mutex orders the calls that use it.  Every call records an event on its
// stream once its kernels are enqueued; a call on another stream than the
// previous one first makes its stream wait for that event.
struct PromptScratch {
    std::mutex mu;
    char* base = nullptr;
    size_t bytes = 0;
    bool used = false;
    hipStream_t last = nullptr;
    hipEvent_t ev = nullptr;
};
PromptScratch g_prompt_scratch[kMaxDevices];


// With s.mu held: at least `need` bytes of s, usable by work enqueued on st next.
hipError_t scratch_take(PromptScratch& s, size_t need, hipStream_t st, char** out)
{
    hipError_t e;
    if (!s.ev && (e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming)) != hipSuccess) return e;
    if (s.used && s.last != st && (e = hipStreamWaitEvent(st, s.ev, 0)) != hipSuccess) return e;
    if (need > s.bytes) {
        const size_t grow = std::max(need, s.bytes + s.bytes / 2);
        if (s.base && (e = hipFreeAsync(s.base, st)) != hipSuccess) return e;
        s.base = nullptr;
        s.bytes = 0;
        if ((e = hipMallocAsync((void**)&s.base, grow, st)) != hipSuccess) return e;
        s.bytes = grow;
    }
    *out = s.base;
    return hipSuccess;
}

// With s.mu held, once everything of the call that uses s is enqueued on st
// (also after a failed launch): later calls on other streams wait for it.
hipError_t scratch_done(PromptScratch& s, hipStream_t st)
{
    s.last = st;
    s.used = true;
    return hipEventRecord(s.ev, st);
}

PromptScratch* prompt_scratch(std::string& why)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        why = "no HIP device (or device index above 63)";
        return nullptr;
    }
    return &g_prompt_scratch[dev];
}

// Causal-attention column sums of packed prompts: validate and fill the
// launch arguments (the caller checks and sets `out`); scratch_bytes = the
// scratch the two passes need.
int colsum_setup(const h2o_config* cfg, const int32_t* plen, const int32_t* row_lo, const float* q,
                 const void* k, int per_head, double* out, ColsumArgs& a, int& maxP, size_t& scratch_bytes)
{
    if (!cfg || !plen) return fail(nullptr, H2O_EINVAL, "null config or prompt lengths");
    const int B = cfg->batch, Hq = cfg->n_q_heads, Hkv = cfg->n_kv_heads;
    if (B < 1 || B > kMaxArgBatch)
        return fail(nullptr, H2O_EINVAL, "prompt column sums take 1 to 128 sequences");
    if (Hkv < 1 || Hq < Hkv || Hq % Hkv != 0)
        return fail(nullptr, H2O_EINVAL, "n_q_heads must be a positive multiple of n_kv_heads");
    const int G = Hq / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(nullptr, H2O_EINVAL, "group size must be 1, 2, 4 or 8");
    if (cfg->head_dim != 128 || cfg->kv_dtype != H2O_BF16)
        return fail(nullptr, H2O_EINVAL, "prompt column sums need bf16 K rows of head_dim 128");
    if (!(cfg->scale >= 0.f)) return fail(nullptr, H2O_EINVAL, "scale must be >= 0");
    a = ColsumArgs{};
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = G;
    a.per_head = per_head ? 1 : 0;
    maxP = 0;
    long long off = 0;
    for (int b = 0; b < B; ++b) {
        const int P = plen[b];
        const int lo = row_lo ? row_lo[b] : 0;
        if (P < 1) return fail(nullptr, H2O_EINVAL, "prompt lengths must be >= 1");
        if (lo < 0 || lo >= P) return fail(nullptr, H2O_EINVAL, "first row must lie in [0, P_b)");
        a.seq_p[b] = P;
        a.seq_lo[b] = lo;
        a.seq_off[b] = off;
        off += P;
        maxP = std::max(maxP, P);
    }
    if (off > (1LL << 31)) return fail(nullptr, H2O_EINVAL, "too many prompt positions");
    if (!q || !k) return fail(nullptr, H2O_EINVAL, "null prompt_q or prompt_k");
    if (misaligned(q) || misaligned(k) || misaligned(out))
        return fail(nullptr, H2O_EINVAL, "prompt_q, prompt_k and the output must be 16-byte aligned");
    const double scale = cfg->scale > 0.f ? (double)cfg->scale : 1.0 / std::sqrt((double)cfg->head_dim);
    a.qscale = (float)(scale * 1.4426950408889634);
    a.q = q;
    a.k = k;
    a.out = out;
    a.nt8 = 0;  // scratch tiles per unit: those from row lo_b's on
    for (int b = 0; b < B; ++b) a.nt8 = std::max(a.nt8, (a.seq_p[b] + 7) / 8 - a.seq_lo[b] / 8);
    const size_t units = (size_t)B * Hkv;
    scratch_bytes = align256(units * a.nt8 * G * 256 * sizeof(uint4)) + align256(units * a.nt8 * G * 8 * sizeof(float2));
    return H2O_OK;
}

// The two column-sum passes with their scratch at sp (colsum_setup's size).
hipError_t colsum_launch(ColsumArgs& a, int maxP, char* sp, hipStream_t st)
{
    const size_t units = (size_t)a.B * a.Hkv;
    a.qs = reinterpret_cast<uint4*>(sp);
    a.st = reinterpret_cast<float2*>(sp + align256(units * a.nt8 * a.G * 256 * sizeof(uint4)));
    return launch_colsum(a, maxP, st);
}

int colsum_run(const h2o_config* cfg, const int32_t* plen, const float* q, const void* k, double* out,
               void* stream)
{
    ColsumArgs a;
    int maxP = 0;
    size_t need = 0;
    int rc = colsum_setup(cfg, plen, nullptr, q, k, 0, out, a, maxP, need);
    if (rc != H2O_OK) return rc;
    if (!out) return fail(nullptr, H2O_EINVAL, "null out");
    std::string why;
    PromptScratch* ps = prompt_scratch(why);
    if (!ps) return fail(nullptr, H2O_EDEVICE, why);
    std::lock_guard<std::mutex> lk(ps->mu);
    hipStream_t st = (hipStream_t)stream;
    char* sp = nullptr;
    hipError_t e = scratch_take(*ps, need, st, &sp);
    if (e != hipSuccess) return hip_fail(nullptr, e, "prompt column sums: scratch");
    e = colsum_launch(a, maxP, sp, st);
    const hipError_t e2 = scratch_done(*ps, st);
    if (e != hipSuccess) return hip_fail(nullptr, e, "prompt column sums: launch");
    if (e2 != hipSuccess) return hip_fail(nullptr, e2, "prompt column sums: scratch event");
    return H2O_OK;
}

// SnapKV's selection, validated and sized: the launch arguments of both
// passes and the scratch they need, laid out as [votes (when the caller passes
// none)] [pooled votes] [column-sum passes] [per-head kept bitmaps (G > 1)].
struct SnapPlan {
    SnapArgs a{};
    ColsumArgs ca{};
    int maxP = 0, maxPc = 0;
    size_t vown = 0, vbytes = 0, cbytes = 0, hbytes = 0;
    size_t scratch_bytes() const { return vown + vbytes + cbytes + hbytes; }
};

int snapkv_plan(const h2o_config* cfg, const int32_t* plen, int window, int pool, int keep, const float* q,
                const void* k, double* votes, int32_t* kept, int32_t* count, int cap, SnapPlan& pl)
{
    if (!cfg || !plen) return fail(nullptr, H2O_EINVAL, "null config or prompt lengths");
    const int B = cfg->batch, Hq = cfg->n_q_heads, Hkv = cfg->n_kv_heads;
    if (B < 1 || B > kMaxArgBatch)
        return fail(nullptr, H2O_EINVAL, "prompt column sums take 1 to 128 sequences");
    if (Hkv < 1 || Hq < Hkv || Hq % Hkv != 0)
        return fail(nullptr, H2O_EINVAL, "n_q_heads must be a positive multiple of n_kv_heads");
    if (window < 1) return fail(nullptr, H2O_EINVAL, "observation window must be >= 1");
    if (pool < 1 || pool % 2 == 0) return fail(nullptr, H2O_EINVAL, "pooling kernel must be odd and >= 1");
    if (keep < 0) return fail(nullptr, H2O_EINVAL, "keep must be >= 0");
    const int G = Hq / Hkv;
    std::vector<int32_t> lo(B);
    SnapArgs& a = pl.a;
    a = SnapArgs{};
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = G;
    a.pool_r = pool / 2;
    a.keep = keep;
    a.cap = cap;
    long long off = 0;
    pl.maxP = 0;
    for (int b = 0; b < B; ++b) {
        const int P = plen[b];
        if (P < 1) return fail(nullptr, H2O_EINVAL, "prompt lengths must be >= 1");
        if (P > (1 << 19)) return fail(nullptr, H2O_EINVAL, "SnapKV selection takes prompts up to 524288");
        const int w = std::min(window, P);
        lo[b] = P - w;
        const long long most = std::min<long long>(P, (long long)w + (long long)G * std::min(keep, P - w));
        if (cap < most) return fail(nullptr, H2O_EINVAL, "cap is below the largest kept set");
        a.seq_p[b] = P;
        a.seq_w[b] = w;
        a.seq_off[b] = off;
        off += P;
        pl.maxP = std::max(pl.maxP, P);
    }
    const long long total = off;
    if (!kept || !count) return fail(nullptr, H2O_EINVAL, "null kept or kept_count");
    if (misaligned(kept) || misaligned(count))
        return fail(nullptr, H2O_EINVAL, "kept and kept_count must be 16-byte aligned");
    a.kept = kept;
    a.count = count;
    pl.vbytes = align256((size_t)total * Hq * sizeof(double));
    a.bits_words = ((pl.maxP + 31) / 32 + 3) & ~3;  // whole 16-byte groups, so staged votes stay aligned
    pl.hbytes = G > 1 ? align256((size_t)B * Hq * a.bits_words * sizeof(unsigned)) : 0;
    pl.vown = votes ? 0 : pl.vbytes;
    const int rc = colsum_setup(cfg, plen, lo.data(), q, k, 1, votes, pl.ca, pl.maxPc, pl.cbytes);
    if (rc == H2O_OK && snapkv_fused_fits(a)) pl.vbytes = pl.cbytes = 0;  // one pass: votes and head bitmaps only
    return rc;
}

// A planned selection on scratch sp of pl.scratch_bytes(): one kernel when it
// fits (snapkv_fused_fits), else both column-sum passes, then the selection.
hipError_t snapkv_enqueue(SnapPlan& pl, double* votes, char* sp, hipStream_t st)
{
    double* vb = votes ? votes : reinterpret_cast<double*>(sp);  // the caller's buffer, else the scratch's first part
    pl.a.votes = vb;
    pl.a.pooled = reinterpret_cast<double*>(sp + pl.vown);
    pl.a.hbits = pl.a.G > 1 ? reinterpret_cast<unsigned*>(sp + pl.vown + pl.vbytes + pl.cbytes) : nullptr;
    if (snapkv_fused_fits(pl.a)) return launch_snapkv_fused(pl.ca, pl.a, vb, st);
    pl.ca.out = vb;
    hipError_t e = colsum_launch(pl.ca, pl.maxPc, sp + pl.vown + pl.vbytes, st);
    if (e != hipSuccess) return e;
    return launch_snapkv(pl.a, pl.maxP, st);
}

// SnapKV's selection (h2o_snapkv_select): validate, per-head window votes by the
// column-sum passes, then pooling and the per-unit selection, on the grow-only
// per-device scratch.
int snapkv_run(const h2o_config* cfg, const int32_t* plen, int window, int pool, int keep, const float* q,
               const void* k, double* votes, int32_t* kept, int32_t* count, int cap, void* stream)
{
    SnapPlan pl;
    int rc = snapkv_plan(cfg, plen, window, pool, keep, q, k, votes, kept, count, cap, pl);
    if (rc != H2O_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    if (pl.scratch_bytes() == 0) {  // one pass into the caller's votes: no scratch, nothing to order
        const hipError_t e = snapkv_enqueue(pl, votes, nullptr, st);
        return e == hipSuccess ? H2O_OK : hip_fail(nullptr, e, "SnapKV: launch");
    }
    std::string why;
    PromptScratch* ps = prompt_scratch(why);
    if (!ps) return fail(nullptr, H2O_EDEVICE, why);
    std::lock_guard<std::mutex> lk(ps->mu);
    char* sp = nullptr;
    hipError_t e = scratch_take(*ps, pl.scratch_bytes(), st, &sp);
    if (e != hipSuccess) return hip_fail(nullptr, e, "SnapKV: scratch");
    e = snapkv_enqueue(pl, votes, sp, st);
    const hipError_t e2 = scratch_done(*ps, st);
    if (e != hipSuccess) return hip_fail(nullptr, e, "SnapKV: launch");
    if (e2 != hipSuccess) return hip_fail(nullptr, e2, "SnapKV: scratch event");
    return H2O_OK;
}

// The same selection on the library's fixed per-device scratch array: nothing
// is allocated, and no event orders it against other calls.
int snapkv_run_noalloc(const h2o_config* cfg, const int32_t* plen, int window, int pool, int keep,
                       const float* q, const void* k, double* votes, int32_t* kept, int32_t* count, int cap,
                       void* stream)
{
    SnapPlan pl;
    int rc = snapkv_plan(cfg, plen, window, pool, keep, q, k, votes, kept, count, cap, pl);
    if (rc != H2O_OK) return rc;
    if (pl.scratch_bytes() > kNoAllocScratchBytes) {
        char m[200];
        std::snprintf(m, sizeof m,
                      "SnapKV without allocation: the call needs %zu bytes of scratch, above the fixed %zu "
                      "(pass votes, or fewer or shorter prompts)",
                      pl.scratch_bytes(), (size_t)kNoAllocScratchBytes);
        return fail(nullptr, H2O_EINVAL, m);
    }
    char* sp = nullptr;
    hipError_t e = noalloc_scratch(&sp);
    if (e != hipSuccess) return hip_fail(nullptr, e, "SnapKV without allocation: scratch address");
    e = snapkv_enqueue(pl, votes, sp, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(nullptr, e, "SnapKV without allocation: launch");
    return H2O_OK;
}

}  // namespace

extern "C" {

// A context's host state and geometry from a validated configuration (no
// device work): slots_total = K/V slots of the cache, maxP = longest prompt.
int setup_ctx(h2o_ctx* c, const h2o_config* cfg, const int32_t* prompt_len, size_t& slots_total, int& maxP,
              std::string& why)
{
    c->cfg = *cfg;
    const int B = cfg->batch, Hkv = cfg->n_kv_heads;
    c->plen.assign(prompt_len, prompt_len + B);
    c->count = c->plen;
    maxP = *std::max_element(c->plen.begin(), c->plen.end());

    Geometry& g = c->g;
    g.B = B;
    g.Hq = cfg->n_q_heads;
    g.Hkv = Hkv;
    g.G = cfg->n_q_heads / Hkv;
    g.D = cfg->head_dim;
    g.cap = (int)slot_capacity(*cfg, maxP);
    g.paged = cfg->page_size ? 1 : 0;
    g.maxp = g.paged ? (g.cap + kPageSize - 1) / kPageSize : 0;
    g.kv_bf16 = cfg->kv_dtype == H2O_BF16;
    g.kv_i8 = cfg->kv_dtype == H2O_I8;
    g.score_f64 = scored(cfg->selector) && cfg->score_dtype == H2O_F64;
    g.score_f16 = scored(cfg->selector) && cfg->score_dtype == H2O_F16;
    // GQA groups of 4 or 8 over bf16 rows of 128 run on the matrix cores, with
    // K / V stored in operand order in whole 32-slot tiles
    g.kv_tiles = g.kv_bf16 && g.D == 128 && !g.paged && (g.G == 4 || g.G == 8);
    if (g.kv_tiles) g.cap = (g.cap + 31) & ~31;
    c->sc = make_sched(*cfg);
    c->block = cfg->selector == H2O_SEL_BLOCK;
    c->js = sink_pages(cfg->n_sink);
    c->evb.assign(B, 0);
    const double scale = cfg->scale > 0.f ? (double)cfg->scale : 1.0 / std::sqrt((double)cfg->head_dim);
    c->qscale = (float)(scale * 1.4426950408889634);  // log2(e)

    // paged: the prompts' pages, from the pool
    if (g.paged) {
        long long demand = 0;
        for (int p : c->plen) demand += (p + kPageSize - 1) / kPageSize;
        if (demand > cfg->max_pages) {
            why = "KV page pool too small for the prompts";
            return H2O_ENOMEM;
        }
        for (int p = cfg->max_pages - 1; p >= 0; --p) c->free_pages.push_back(p);
        c->pages.resize(B);
        for (int b = 0; b < B; ++b) {
            const int np = (c->plen[b] + kPageSize - 1) / kPageSize;
            for (int i = 0; i < np; ++i) {
                c->pages[b].push_back(c->free_pages.back());
                c->free_pages.pop_back();
            }
        }
        slots_total = (size_t)cfg->max_pages * Hkv * kPageSize;
    } else {
        slots_total = (size_t)B * Hkv * g.cap;
    }

    return H2O_OK;
}

// Every device buffer of a context, in one list: sized (c->measure), carved from
// the caller's workspace (c->ws) or allocated one by one.  t0 / poff receive the
// prompt lengths' and offsets' buffers.
int alloc_state(h2o_ctx* c, size_t slots_total, int32_t** t0, int64_t** poff)
{
    int rc = H2O_OK;
    State& s = c->s;
    const Geometry& g = c->g;
    const h2o_config* cfg = &c->cfg;
    const int B = g.B;
    const size_t units = (size_t)B * g.Hkv;
    const size_t sw = g.score_f64 ? 8 : (g.score_f16 ? 2 : 4);
    const size_t row_bytes = g.kv_i8 ? kRowBytesI8 : kRowBytes;
    if ((rc = dalloc(c, &s.kc, slots_total * row_bytes, "alloc K cache")) ||
        (rc = dalloc(c, &s.vc, slots_total * row_bytes, "alloc V cache")) ||
        (g.kv_i8 && (rc = dalloc(c, &s.kss, slots_total * 4, "alloc K row scales"))) ||
        (g.kv_i8 && (rc = dalloc(c, &s.vss, slots_total * 4, "alloc V row scales"))) ||
        (scored(cfg->selector) && (rc = dalloc(c, &s.sc, slots_total * sw, "alloc scores"))) ||
        (rc = dalloc(c, &s.ps, slots_total * 4, "alloc positions")) ||
        (rc = dalloc(c, &s.cnt, units * 4, "alloc counts")) ||
        (rc = dalloc(c, &s.emass, units * 8, "alloc evicted mass")) ||
        (rc = dalloc(c, &s.vinfo, units * 8, "alloc victim info")) ||
        (rc = dalloc(c, &s.err, 4, "alloc error word")) ||
        (rc = dalloc(c, t0, (size_t)B * 4, "alloc prompt lengths")) ||
        (rc = dalloc(c, poff, (size_t)(B + 1) * 8, "alloc prompt offsets")) ||
        (cfg->selector != H2O_SEL_BLOCK &&
         (rc = dalloc(c, &s.iscr, units * 2 * (size_t)g.cap * 4, "alloc compaction lists"))) ||
        (g.paged && (rc = dalloc(c, &s.bt, (size_t)B * g.maxp * 4, "alloc block table"))) ||
        (cfg->selector == H2O_SEL_BLOCK &&
         ((rc = dalloc(c, &s.fstack, (size_t)cfg->max_pages * 4, "alloc free-page stack")) ||
          (rc = dalloc(c, &s.bimp, units * (size_t)bimp_stride(g.maxp), "alloc page importance")))) ||
        ((size_t)g.G * g.cap * 4 > (size_t)kLogitLdsBytes &&
         (rc = dalloc(c, &s.lscr, units * g.G * (size_t)g.cap * 4, "alloc logit scratch")))) {
        return rc;
    }
    return H2O_OK;
}

int h2o_init(h2o_ctx** out, const h2o_config* cfg, const int32_t* prompt_len, const void* prompt_k,
             const void* prompt_v, const double* init_scores, void* stream)
{
    if (!out) return fail(nullptr, H2O_EINVAL, "null output pointer");
    *out = nullptr;
    std::string why;
    int rc = validate(cfg, prompt_len, why);
    if (rc != H2O_OK) return fail(nullptr, rc, why);
    if (!prompt_k || !prompt_v) return fail(nullptr, H2O_EINVAL, "null prompt_k or prompt_v");
    if (misaligned(prompt_k) || misaligned(prompt_v) || misaligned(init_scores))
        return fail(nullptr, H2O_EINVAL, "prompt_k, prompt_v and init_scores must be 16-byte aligned");

    h2o_ctx* c = new h2o_ctx();
    size_t slots_total = 0;
    int maxP = 0;
    if ((rc = setup_ctx(c, cfg, prompt_len, slots_total, maxP, why)) != H2O_OK) {
        delete c;
        return fail(nullptr, rc, why);
    }
    const Geometry& g = c->g;
    const int B = g.B;
    if (hipGetDevice(&c->device) != hipSuccess) {
        delete c;
        return fail(nullptr, H2O_EDEVICE, "no HIP device");
    }
    if (cfg->workspace) {  // the caller's memory: check its size first, then carve
        int32_t* t0m = nullptr;
        int64_t* poffm = nullptr;
        c->measure = true;
        (void)alloc_state(c, slots_total, &t0m, &poffm);
        c->measure = false;
        if (cfg->workspace_bytes < c->need) {
            const std::string m = "workspace_bytes " + std::to_string(cfg->workspace_bytes) +
                                  " is below h2o_workspace_size (" + std::to_string(c->need) + ")";
            delete c;
            return fail(nullptr, H2O_EINVAL, m);
        }
        c->ws = static_cast<char*>(cfg->workspace);
        c->ws_bytes = (size_t)cfg->workspace_bytes;
    }
    State& s = c->s;
    int32_t* t0 = nullptr;
    int64_t* poff = nullptr;
    if ((rc = alloc_state(c, slots_total, &t0, &poff)) != H2O_OK) {
        std::string why_alloc = c->err;
        free_all(c);
        delete c;
        return fail(nullptr, rc, why_alloc);
    }
    s.t0 = t0;
    s.poff = poff;

    std::vector<int64_t> off(B + 1, 0);
    for (int b = 0; b < B; ++b) off[b + 1] = off[b] + c->plen[b];
    hipError_t e;
    if ((e = hipMemcpy(t0, c->plen.data(), (size_t)B * 4, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(poff, off.data(), (size_t)(B + 1) * 8, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemset(s.err, 0, 4)) != hipSuccess) {
        int r = hip_fail(nullptr, e, "init upload");
        free_all(c);
        delete c;
        return r;
    }
    if (g.paged) {
        std::vector<int32_t> bt((size_t)B * g.maxp, -1);
        for (int b = 0; b < B; ++b)
            for (size_t i = 0; i < c->pages[b].size(); ++i) bt[(size_t)b * g.maxp + i] = c->pages[b][i];
        if ((e = hipMemcpy(s.bt, bt.data(), bt.size() * 4, hipMemcpyHostToDevice)) != hipSuccess ||
            (c->block && !c->free_pages.empty() &&
             (e = hipMemcpy(s.fstack, c->free_pages.data(), c->free_pages.size() * 4, hipMemcpyHostToDevice)) !=
                 hipSuccess)) {
            int r = hip_fail(nullptr, e, "block table upload");
            free_all(c);
            delete c;
            return r;
        }
        if (c->block) {  // from here on the device stack holds the free ids
            c->ftop = (int)c->free_pages.size();
            c->free_pages.clear();
            c->pages.clear();
        }
    }
    LoadArgs la{};
    la.g = g;
    la.s = s;
    la.pk = prompt_k;
    la.pv = prompt_v;
    la.init_scores = init_scores;
    if ((e = launch_load(la, maxP, (hipStream_t)stream)) != hipSuccess) {
        int r = hip_fail(nullptr, e, "prompt load launch");
        free_all(c);
        delete c;
        return r;
    }
    *out = c;
    return H2O_OK;
}

int h2o_workspace_size(const h2o_config* cfg, const int32_t* prompt_len, uint64_t* bytes)
{
    if (!bytes) return fail(nullptr, H2O_EINVAL, "null bytes");
    *bytes = 0;
    std::string why;
    int rc = validate(cfg, prompt_len, why);
    if (rc != H2O_OK) return fail(nullptr, rc, why);
    h2o_ctx c;
    size_t slots_total = 0;
    int maxP = 0;
    if ((rc = setup_ctx(&c, cfg, prompt_len, slots_total, maxP, why)) != H2O_OK) return fail(nullptr, rc, why);
    int32_t* t0 = nullptr;
    int64_t* poff = nullptr;
    c.measure = true;
    (void)alloc_state(&c, slots_total, &t0, &poff);
    *bytes = (uint64_t)c.need;
    return H2O_OK;
}

int h2o_pool_pages(const h2o_config* cfg, const int32_t* prompt_len, int32_t steps, int32_t* pages)
{
    if (!pages) return fail(nullptr, H2O_EINVAL, "null pages");
    *pages = 0;
    if (!cfg) return fail(nullptr, H2O_EINVAL, "null config or prompt_len");
    if (cfg->page_size != kPageSize) return fail(nullptr, H2O_EINVAL, "pool sizing needs the paged layout (page_size 16)");
    h2o_config c = *cfg;
    c.max_pages = 1;  // the size being computed: any valid value for the check
    c.workspace = nullptr;
    std::string why;
    const int rc = validate(&c, prompt_len, why);
    if (rc != H2O_OK) return fail(nullptr, rc, why);
    if (steps < 0) return fail(nullptr, H2O_EINVAL, "steps must be >= 0");
    const Sched sc = make_sched(c);
    const int js = sink_pages(c.n_sink);
    long long total = 0;
    for (int b = 0; b < c.batch; ++b) {
        const int P = prompt_len[b];
        if ((long long)P + steps > c.max_len) return fail(nullptr, H2O_EINVAL, "a sequence would pass max_len");
        // the host mirror of one sequence: a step holds ceil(n_att / 16) pages
        // while it runs (the append's page is taken before anything is evicted)
        long long most = (P + kPageSize - 1) >> kPageShift;
        int cnt = P, evb = 0;
        for (int s = 0; s < steps; ++s) {
            const int t = P + s, n_att = cnt + 1;
            most = std::max<long long>(most, (n_att + kPageSize - 1) >> kPageShift);
            if (c.selector == H2O_SEL_BLOCK) {
                int K, HH, W;
                schedule(sc, t + 1, K, HH, W);
                int m = 0;
                if (n_att > K) {
                    const int kb = t + 1 - W > 0 ? (t + 1 - W) >> kPageShift : 0;
                    const int nc = std::max(0, kb - js) - evb;
                    m = std::min(nc, (n_att - K + kPageSize - 1) >> kPageShift);
                }
                evb += std::max(m, 0);
                cnt = n_att - std::max(m, 0) * kPageSize;
            } else {
                cnt = n_att - evict_count(sc, t, P, n_att);
            }
        }
        total += most;
    }
    if (total > INT32_MAX) return fail(nullptr, H2O_EINVAL, "page pool larger than 2^31 pages");
    *pages = (int32_t)total;
    return H2O_OK;
}

int h2o_step(h2o_ctx* ctx, const float* q, const void* k_new, const void* v_new, float* out,
             void* stream)
{
    return do_step(ctx, q, k_new, v_new, out, stream, false);
}

int h2o_step_compact(h2o_ctx* ctx, const float* q, const void* k_new, const void* v_new, float* out,
                     void* stream)
{
    return do_step(ctx, q, k_new, v_new, out, stream, true);
}

int h2o_compact(h2o_ctx* c, void* stream)
{
    if (!c) return H2O_EINVAL;
    if (!c->pending) return fail(c, H2O_ESTATE, "no step is pending compaction");
    DeviceGuard dg(c->device);
    if (c->block) {
        hipError_t err = launch_block(c->pend_blk, (hipStream_t)stream);
        if (err != hipSuccess) return hip_fail(c, err, "block eviction launch");
        c->pending = false;
        c->step += 1;
        return H2O_OK;
    }
    CompactArgs a{};
    a.g = c->g;
    a.s = c->s;
    hipError_t err = launch_compact(a, c->g.cap, (hipStream_t)stream);
    if (err != hipSuccess) return hip_fail(c, err, "compact kernel launch");
    for (int b = 0; b < c->g.B; ++b) {
        c->count[b] = c->count[b] + 1 - c->pend_e[b];
        if (c->g.paged) release_pages(c, b);
    }
    c->pending = false;
    c->step += 1;
    return H2O_OK;
}

int h2o_read_indices(h2o_ctx* c, int32_t* pos, int32_t* count, double* scores, double* evicted_mass,
                     size_t cap, void* stream)
{
    if (!c) return H2O_EINVAL;
    if (c->pending && !c->block) return fail(c, H2O_ESTATE, "a compaction is pending: call h2o_compact first");
    if (!pos || !count) return fail(c, H2O_EINVAL, "null pos or count");
    const int B = c->g.B, Hkv = c->g.Hkv;
    int maxc = 0;
    for (int b = 0; b < B; ++b) maxc = std::max(maxc, visible_count(c, b));
    if (cap < (size_t)maxc || cap == 0 || cap > (size_t)(1 << 30))
        return fail(c, H2O_EINVAL, "cap is smaller than a retained count");
    DeviceGuard dg(c->device);
    const size_t units = (size_t)B * Hkv;
    int32_t* dpos = nullptr;
    double* dsc = nullptr;
    hipError_t e;
    if ((e = hipMalloc(&dpos, units * cap * 4)) != hipSuccess) return hip_fail(c, e, "read staging");
    if ((e = hipMalloc(&dsc, units * cap * 8)) != hipSuccess) {
        (void)hipFree(dpos);
        return hip_fail(c, e, "read staging");
    }
    GatherArgs ga{};
    ga.g = c->g;
    ga.s = c->s;
    ga.selector = c->sc.selector;
    ga.capo = (int)cap;
    ga.opos = dpos;
    ga.osc = dsc;
    std::vector<int32_t> hpos(units * cap), dcnt(units);
    std::vector<double> hsc(units * cap), hem(units);
    int32_t herr = 0;
    hipStream_t st = (hipStream_t)stream;
    if ((e = launch_gather(ga, st)) != hipSuccess ||
        (e = hipMemcpyAsync(hpos.data(), dpos, units * cap * 4, hipMemcpyDeviceToHost, st)) != hipSuccess ||
        (e = hipMemcpyAsync(hsc.data(), dsc, units * cap * 8, hipMemcpyDeviceToHost, st)) != hipSuccess ||
        (e = hipMemcpyAsync(dcnt.data(), c->s.cnt, units * 4, hipMemcpyDeviceToHost, st)) != hipSuccess ||
        (e = hipMemcpyAsync(hem.data(), c->s.emass, units * 8, hipMemcpyDeviceToHost, st)) != hipSuccess ||
        (e = hipMemcpyAsync(&herr, c->s.err, 4, hipMemcpyDeviceToHost, st)) != hipSuccess ||
        (e = hipStreamSynchronize(st)) != hipSuccess) {
        (void)hipFree(dpos);
        (void)hipFree(dsc);
        return hip_fail(c, e, "read back");
    }
    (void)hipFree(dpos);
    (void)hipFree(dsc);
    if (herr) {
        char m[96];
        std::snprintf(m, sizeof m, "kernel consistency check failed (error bits 0x%x)", herr);
        return fail(c, H2O_EDEVICE, m);
    }
    std::vector<int> order;
    for (size_t u = 0; u < units; ++u) {
        const int b = (int)(u / Hkv);
        const int n = visible_count(c, b);
        if (dcnt[u] != n) return fail(c, H2O_EDEVICE, "device retained count differs from the schedule");
        order.resize(n);
        for (int i = 0; i < n; ++i) order[i] = i;
        const int32_t* P = &hpos[u * cap];
        std::sort(order.begin(), order.end(), [&](int x, int y) { return P[x] < P[y]; });
        for (int i = 0; i < n; ++i) {
            pos[u * cap + i] = P[order[i]];
            if (scores) scores[u * cap + i] = hsc[u * cap + order[i]];
        }
        for (size_t i = n; i < cap; ++i) {
            pos[u * cap + i] = -1;
            if (scores) scores[u * cap + i] = 0.0;
        }
        if (evicted_mass) evicted_mass[u] = hem[u];
    }
    for (int b = 0; b < B; ++b) count[b] = visible_count(c, b);
    return H2O_OK;
}

int h2o_read_kv(h2o_ctx* c, void* k_rows, void* v_rows, float* k_scale, float* v_scale, size_t cap,
                void* stream)
{
    if (!c) return H2O_EINVAL;
    if (c->pending && !c->block) return fail(c, H2O_ESTATE, "a compaction is pending: call h2o_compact first");
    if (!k_rows || !v_rows) return fail(c, H2O_EINVAL, "null k_rows or v_rows");
    if (c->g.kv_i8 && (!k_scale || !v_scale)) return fail(c, H2O_EINVAL, "i8 storage needs k_scale and v_scale");
    const int B = c->g.B, Hkv = c->g.Hkv;
    int maxc = 0;
    for (int b = 0; b < B; ++b) maxc = std::max(maxc, visible_count(c, b));
    if (cap < (size_t)maxc || cap == 0 || cap > (size_t)(1 << 30))
        return fail(c, H2O_EINVAL, "cap is smaller than a retained count");
    DeviceGuard dg(c->device);
    const size_t units = (size_t)B * Hkv;
    const size_t rb = c->g.kv_i8 ? kRowBytesI8 : kRowBytes;
    std::vector<void*> tmp;
    auto dfree = [&]() {
        for (void* p : tmp) (void)hipFree(p);
    };
    auto dmal = [&](void** p, size_t bytes) {
        hipError_t e = hipMalloc(p, bytes);
        if (e == hipSuccess) tmp.push_back(*p);
        return e;
    };
    int32_t* dpos = nullptr;
    double* dsc = nullptr;
    unsigned char *dk = nullptr, *dv = nullptr;
    float *dks = nullptr, *dvs = nullptr;
    hipError_t e;
    if ((e = dmal((void**)&dpos, units * cap * 4)) != hipSuccess || (e = dmal((void**)&dsc, units * cap * 8)) != hipSuccess ||
        (e = dmal((void**)&dk, units * cap * rb)) != hipSuccess || (e = dmal((void**)&dv, units * cap * rb)) != hipSuccess ||
        (c->g.kv_i8 && ((e = dmal((void**)&dks, units * cap * 4)) != hipSuccess ||
                        (e = dmal((void**)&dvs, units * cap * 4)) != hipSuccess))) {
        dfree();
        return hip_fail(c, e, "read staging");
    }
    GatherArgs ga{};
    ga.g = c->g;
    ga.s = c->s;
    ga.selector = c->sc.selector;
    ga.capo = (int)cap;
    ga.opos = dpos;
    ga.osc = dsc;
    RowGatherArgs ra{};
    ra.g = c->g;
    ra.s = c->s;
    ra.capo = (int)cap;
    ra.ok = dk;
    ra.ov = dv;
    ra.oks = dks;
    ra.ovs = dvs;
    std::vector<int32_t> hpos(units * cap);
    std::vector<unsigned char> hk(units * cap * rb), hv(units * cap * rb);
    std::vector<float> hks(c->g.kv_i8 ? units * cap : 0), hvs(c->g.kv_i8 ? units * cap : 0);
    hipStream_t st = (hipStream_t)stream;
    if ((e = launch_gather(ga, st)) != hipSuccess || (e = launch_gather_rows(ra, st)) != hipSuccess ||
        (e = hipMemcpyAsync(hpos.data(), dpos, units * cap * 4, hipMemcpyDeviceToHost, st)) != hipSuccess ||
        (e = hipMemcpyAsync(hk.data(), dk, units * cap * rb, hipMemcpyDeviceToHost, st)) != hipSuccess ||
        (e = hipMemcpyAsync(hv.data(), dv, units * cap * rb, hipMemcpyDeviceToHost, st)) != hipSuccess ||
        (c->g.kv_i8 &&
         ((e = hipMemcpyAsync(hks.data(), dks, units * cap * 4, hipMemcpyDeviceToHost, st)) != hipSuccess ||
          (e = hipMemcpyAsync(hvs.data(), dvs, units * cap * 4, hipMemcpyDeviceToHost, st)) != hipSuccess)) ||
        (e = hipStreamSynchronize(st)) != hipSuccess) {
        dfree();
        return hip_fail(c, e, "read back");
    }
    dfree();
    unsigned char* K = (unsigned char*)k_rows;
    unsigned char* V = (unsigned char*)v_rows;
    std::vector<int> order;
    for (size_t u = 0; u < units; ++u) {
        const int n = visible_count(c, (int)(u / Hkv));
        order.resize(n);
        for (int i = 0; i < n; ++i) order[i] = i;
        const int32_t* Pp = &hpos[u * cap];
        std::sort(order.begin(), order.end(), [&](int x, int y) { return Pp[x] < Pp[y]; });
        for (size_t i = 0; i < cap; ++i) {
            unsigned char* kd = K + (u * cap + i) * rb;
            unsigned char* vd = V + (u * cap + i) * rb;
            if ((int)i < n) {
                const size_t from = u * cap + order[i];
                std::memcpy(kd, &hk[from * rb], rb);
                std::memcpy(vd, &hv[from * rb], rb);
                if (c->g.kv_i8) {
                    k_scale[u * cap + i] = hks[from];
                    v_scale[u * cap + i] = hvs[from];
                }
            } else {
                std::memset(kd, 0, rb);
                std::memset(vd, 0, rb);
                if (c->g.kv_i8) k_scale[u * cap + i] = v_scale[u * cap + i] = 0.f;
            }
        }
    }
    return H2O_OK;
}

int h2o_info(const h2o_ctx* c, int32_t* slot_capacity, int32_t* steps_done, int32_t* pages_in_use)
{
    if (!c) return H2O_EINVAL;
    if (slot_capacity) *slot_capacity = c->g.cap;
    if (steps_done) *steps_done = c->step;
    if (pages_in_use) {
        long long n = 0;
        if (c->block)  // every block-table entry but the last is full
            for (int b = 0; b < c->g.B; ++b) n += (visible_count(c, b) + kPageSize - 1) >> kPageShift;
        else
            for (const auto& p : c->pages) n += (long long)p.size();
        *pages_in_use = (int32_t)n;
    }
    return H2O_OK;
}

void h2o_destroy(h2o_ctx* c)
{
    if (!c) return;
    {
        DeviceGuard dg(c->device);
        (void)hipDeviceSynchronize();
        free_all(c);
    }
    delete c;
}

int h2o_prefill_scores(const h2o_config* cfg, const int32_t* prompt_len, const float* prompt_q,
                       const void* prompt_k, double* out, void* stream)
{
    return colsum_run(cfg, prompt_len, prompt_q, prompt_k, out, stream);
}

int h2o_snapkv_select(const h2o_config* cfg, const int32_t* prompt_len, int32_t window, int32_t pool,
                      int32_t keep, const float* prompt_q, const void* prompt_k, double* votes,
                      int32_t* kept, int32_t* kept_count, int32_t cap, void* stream)
{
    return snapkv_run(cfg, prompt_len, window, pool, keep, prompt_q, prompt_k, votes, kept, kept_count, cap,
                      stream);
}

int h2o_snapkv_select_noalloc(const h2o_config* cfg, const int32_t* prompt_len, int32_t window, int32_t pool,
                              int32_t keep, const float* prompt_q, const void* prompt_k, double* votes,
                              int32_t* kept, int32_t* kept_count, int32_t cap, void* stream)
{
    return snapkv_run_noalloc(cfg, prompt_len, window, pool, keep, prompt_q, prompt_k, votes, kept, kept_count,
                              cap, stream);
}

const char* h2o_last_error(const h2o_ctx* c)
{
    if (c) return c->err.c_str();
    std::lock_guard<std::mutex> lk(g_err_mu);
    static thread_local std::string copy;
    copy = g_init_err;
    return copy.c_str();
}

}  // extern "C"
