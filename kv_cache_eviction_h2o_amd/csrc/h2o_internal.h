// Internal interface between the host runtime (h2o_runtime.cpp) and the
// gfx950 kernels (h2o_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

namespace h2o {

constexpr int kPageShift = 4;           // 16-token KV pages
constexpr int kPageSize = 1 << kPageShift;
constexpr int kRowBytes = 256;          // one K or V row: 128 x bf16 or 64 x fp32
constexpr int kRowBytesI8 = 128;        // one int8 row of 128 (plus its scale)
constexpr int kRowVecs = kRowBytes / 16;  // 16-byte vectors per row = lanes per row
constexpr int kMaxArgBatch = 128;       // per-sequence step parameters travel in the kernel args
                                        // (larger batches read them from device memory)
constexpr int kLogitLdsBytes = 64 * 1024;  // logits kept in LDS up to this size per unit
constexpr int kMaxBlockPages = 5120;  // block eviction: block-table row held in LDS (with
                                      // importance and freed lists: 12 bytes per entry)
constexpr int kMaxDevices = 64;        // devices the per-device host records cover

// Dynamic LDS above the default 48 KB needs the kernel's limit raised on the
// device it runs on.  One record per kernel keeps the largest size granted on
// each device; raising it takes a mutex, so threads driving different contexts
// may launch the same kernel at once.
class DynLdsLimit {
public:
    DynLdsLimit()
    {
        for (auto& g : granted_) g.store(48 * 1024, std::memory_order_relaxed);
    }
    hipError_t allow(const void* kern, size_t bytes)
    {
        if (bytes <= 48 * 1024) return hipSuccess;
        int dev = -1;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
        if (bytes <= granted_[dev].load(std::memory_order_acquire)) return hipSuccess;
        std::lock_guard<std::mutex> lk(mu_);
        if (bytes <= granted_[dev].load(std::memory_order_relaxed)) return hipSuccess;
        if ((e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes)) != hipSuccess)
            return e;
        granted_[dev].store(bytes, std::memory_order_release);
        return hipSuccess;
    }

private:
    std::mutex mu_;
    std::atomic<size_t> granted_[kMaxDevices];
};

// Row stride of State::bimp: whole 16-byte groups, so rows can be read in words.
__host__ __device__ inline int bimp_stride(int maxp) { return (maxp + 15) & ~15; }

// Error bits a kernel may raise in State::err (checked by h2o_read_indices).
enum : int { kErrSelectCount = 1, kErrNoCandidate = 2, kErrCompact = 4, kErrBlock = 8 };

// Selectors (the values of h2o_config::selector).
enum : int { kSelH2O = 0, kSelRandom = 1, kSelBlock = 2 };

// Selectors that keep cumulative attention scores: H2O ranks tokens by them,
// block eviction ranks whole pages by its heads' heavy hitters among them.
__host__ __device__ inline bool scored(int selector) { return selector != kSelRandom; }

struct Geometry {
    int B, Hq, Hkv, G, D;
    int cap;        // slots per (b, h) unit (contiguous layout stride; scratch sizing)
    int paged;      // 1 = 16-token pages through the block table
    int maxp;       // paged: block-table row length (pages per sequence)
    int kv_bf16;    // 1 = bf16 rows (inputs and storage), 0 = fp32 rows
    int kv_i8;      // 1 = bf16 inputs stored as int8 rows of 128 with one fp32 scale per row
    int score_f64;  // 1 = fp64 cumulative scores
    int score_f16;  // 1 = IEEE binary16 cumulative scores (H2O only); neither: fp32
    int kv_tiles;   // 1 = K/V in matrix-instruction operand order (bf16, head_dim 128,
                    //     contiguous, cap a multiple of 32, GQA group of 4 or 8)
};

struct State {  // device pointers owned by the context
    void* kc;          // K rows
    void* vc;          // V rows
    float* kss;        // int8 storage: scale of each K row (else null)
    float* vss;        // int8 storage: scale of each V row (else null)
    void* sc;          // cumulative scores (H2O)
    int32_t* ps;       // position of each slot; -1 marks a victim awaiting compaction
    int32_t* cnt;      // [B*Hkv] slots in use
    double* emass;     // [B*Hkv] evicted score mass
    int32_t* vinfo;    // [B*Hkv][2] pending (e, victim slot) for the compaction kernel
    int32_t* bt;       // paged: [B][maxp] page of each 16-slot block
    int32_t* fstack;   // block eviction: [max_pages] free-page stack (depth kept by the host)
    uint8_t* bimp;     // block eviction: [B*Hkv][bimp_stride(maxp)] important tokens of each
                       // head in each candidate block-table entry
    const int32_t* t0; // [B] prompt lengths
    const int64_t* poff;  // [B+1] prompt offsets into the packed prompt arrays
    float* lscr;       // [B*Hkv][G][cap] logits when they do not fit LDS (or null)
    int32_t* iscr;     // [B*Hkv][2*cap] hole / live lists for bulk compaction
    int32_t* err;      // error bits
};

struct Sched {
    int selector;  // kSelH2O, kSelRandom or kSelBlock
    int n_sink, budget_fixed, hh_fixed, budget_num, budget_den;
    int rand_k, rand_r;
    unsigned long long seed;
    float decay;  // moving-sum decay of the scores per step (1 = exact cumulative sum)
};

// Budget K_t, heavy hitters HH_t and recent window W_t at length len = t + 1.
__host__ __device__ __attribute__((always_inline)) inline void schedule(const Sched& s, int len, int& K, int& HH, int& W)
{
    if (s.budget_fixed > 0) {
        K = s.budget_fixed;
        HH = s.hh_fixed;
    } else {
        K = (int)(((long long)len * s.budget_num) / s.budget_den);
        HH = (K - s.n_sink) / 2;
    }
    W = K - s.n_sink - HH;
}

// Tokens to evict at the step that appends position t, with n_att retained
// slots after the append and prompt length P.
__host__ __device__ __attribute__((always_inline)) inline int evict_count(const Sched& s, int t, int P, int n_att)
{
    if (s.selector == kSelH2O) {
        int K, HH, W;
        schedule(s, t + 1, K, HH, W);
        return n_att > K ? n_att - K : 0;
    }
    if (s.selector == kSelBlock) return 0;  // whole pages go after the step (launch_block)
    return (n_att - P == s.rand_k + s.rand_r) ? s.rand_r : 0;
}

// Bulk compaction of a paged H2O unit whose slots still hold the positions in
// order (the first decode step): the recent window's whole pages stay where
// they are and are linked in after a front of whole pages, so only the heavy
// hitters past the front, and at most 15 window rows at each end of the
// window, move.  The front, slots [0, front), keeps its survivors and takes
// every moved row; the window rows [src, src + m) become slots
// [front, front + m) by relinking their pages.  front and src are multiples
// of the page size, and the relinked pages do not overlap their destination
// entries of the block table.  False: plain compaction into [0, n_att - e).
struct WindowRemap {
    int front;  // slots kept in place (whole pages)
    int src;    // first window slot on a page boundary
    int m;      // window rows linked in
};
__host__ __device__ __attribute__((always_inline)) inline bool window_remap(const Sched& s, int t, int n_att, int e, WindowRemap& r)
{
    if (s.selector != kSelH2O) return false;
    int K, HH, W;
    schedule(s, t + 1, K, HH, W);
    if (W < 32 || e < 64 || e < 2 * W) return false;
    const int n2 = n_att - e;
    const int A = n_att - W;  // the window's first slot: positions t + 1 - W .. t
    r.src = (A + kPageSize - 1) & ~(kPageSize - 1);
    r.front = (r.src - e + kPageSize - 1) / kPageSize * kPageSize;  // r.src - e >= n_sink + HH >= 0
    r.m = n2 - r.front;
    const int pages = (r.m + kPageSize - 1) / kPageSize;
    return r.m > 0 && r.m <= n_att - r.src && r.src - r.front >= pages * kPageSize;
}

// One row of a step launch, read by its workgroups with a single 16-byte
// load: the sequences go longest first (a workgroup's time grows with its count).
struct alignas(16) SeqArg {
    int32_t b;        // the sequence
    int32_t n;        // its retained slots before the step
    int32_t p;        // its prompt length
    int32_t newpage;  // paged: the page for its append slot, or -1 (with pop_stack,
                      // the free-stack entry that holds it)
};

struct StepArgs {
    Geometry g;
    State s;
    Sched sc;
    const float* q;
    const void* kn;
    const void* vn;
    float* out;
    float qscale;   // logit scale * log2(e): logits are kept in the log2 domain
    int step;       // decode steps done before this one: t_b = P_b + step
    int fused;      // 1: the select's holes are filled in the same launch
    int lds_n;      // logit row stride in LDS (>= max n_att of the launch)
    int npg_lds;    // paged: block-table entries staged in LDS per unit
    int seq_in_args;             // 1: seq below is valid (B <= kMaxArgBatch)
    int pop_stack;               // 1: SeqArg::newpage indexes State::fstack
    int remap;                   // 1: the first decode step of paged H2O: bulk compaction
                                 // keeps the window's pages (window_remap)
    SeqArg seq[kMaxArgBatch];    // row i: the sequence whose units workgroups i * Hkv .. + Hkv take
};

static_assert(sizeof(StepArgs) <= 4096, "kernel arguments are limited to 4 KB");

// Block-granular eviction after a step (h2o_block.hip), for the nseq sequences
// that lose pages: candidate blocks are block-table entries [js, js + ncand)
// (whole pages past the sinks' pages and clear of the recent window), m of
// them go, their pages pushed on the free stack at push[i]...
struct BlockArgs {
    Geometry g;
    State s;
    Sched sc;
    int nseq;
    int js;                        // block-table entries holding sink positions
    int32_t seq_b[kMaxArgBatch];   // the sequence
    int32_t seq_len[kMaxArgBatch]; // its length after the step (t + 1)
    int32_t seq_n[kMaxArgBatch];   // its retained slots after the append (n_att)
    int32_t seq_c[kMaxArgBatch];   // candidate blocks
    int32_t seq_m[kMaxArgBatch];   // blocks to evict (1 <= m <= ncand)
    int32_t seq_push[kMaxArgBatch];  // first free-stack entry its pages go to
};

struct CompactArgs {
    Geometry g;
    State s;
};

struct LoadArgs {
    Geometry g;
    State s;
    const void* pk;
    const void* pv;
    const double* init_scores;
    int max_prompt;  // longest prompt (the grid's x extent covers its rows)
};

struct GatherArgs {
    Geometry g;
    State s;
    int selector;
    int capo;         // entries per unit in the staging buffers
    int32_t* opos;    // [B*Hkv][capo]
    double* osc;      // [B*Hkv][capo]
};

// Causal-attention column sums of packed prompts (h2o_prefill.hip): rows
// [seq_lo[b], seq_p[b]) of every unit, bf16 K rows of 128, fp32 q.
struct ColsumArgs {
    int B, Hq, Hkv, G;
    int nt8;          // 8-position tiles per unit in the scratch: tiles seq_lo[b] / 8 on, at
                      // most max_b (ceil(P_b / 8) - seq_lo[b] / 8)
    float qscale;     // logit scale * log2(e)
    int per_head;     // 1: out[(off_b + j) * Hq + h * G + g]; 0: out[(off_b + j) * Hkv + h]
    const float* q;   // [sum P][Hq][128]
    const void* k;    // [sum P][Hkv][128] bf16
    uint4* qs;        // scratch [unit][nt8][G][4][64] 16-byte A-operand pieces of q (hi/lo)
    float2* st;       // scratch [unit][nt8][G][8] (row max, 1 / row sum), log2 domain
    double* out;
    int32_t seq_p[kMaxArgBatch], seq_lo[kMaxArgBatch];
    int64_t seq_off[kMaxArgBatch];
};

// SnapKV's prompt selection from per-head window votes (h2o_prefill.hip).
struct SnapArgs {
    int B, Hq, Hkv, G;
    int pool_r;             // max pooling over positions within pool_r of j
    int keep;               // prefix positions kept per query head
    int cap;                // entries per unit in kept
    const double* votes;    // [sum P][Hq]
    double* pooled;         // scratch [sum P][Hq] (prefix positions only)
    int bits_words;         // selection: words of a kept-position bitmap (LDS, and hbits' stride)
    int stage_n;            // selection kernel: prefixes up to this length are staged in LDS
    unsigned* hbits;        // G > 1: scratch [B * Hkv][G][bits_words], each query head's kept bits
    int32_t* kept;          // [B * Hkv][cap] ascending positions, -1 past the count
    int32_t* count;         // [B * Hkv]
    int32_t seq_p[kMaxArgBatch], seq_w[kMaxArgBatch];
    int64_t seq_off[kMaxArgBatch];
};

// Stored rows of the retained slots, in slot order (h2o_read_kv).
struct RowGatherArgs {
    Geometry g;
    State s;
    int capo;              // entries per unit in the staging buffers
    unsigned char* ok;     // [B*Hkv][capo][row bytes] K rows as stored (natural element order)
    unsigned char* ov;     // [B*Hkv][capo][row bytes] V rows
    float* oks;            // [B*Hkv][capo] row scales (int8 storage; else null)
    float* ovs;
};

// Launchers (h2o_kernels.hip unless noted).  Each returns the launch's hipError_t.
hipError_t launch_step(const StepArgs& a, int max_n_att, hipStream_t st);
hipError_t launch_step_mfma(const StepArgs& a, int max_n_att, hipStream_t st);  // h2o_mfma.hip
// The FMA step kernel for one cumulative-score type (h2o_step_f32/f64/f16.hip);
// llds: logits in LDS (dyn bytes of dynamic LDS), else in State::lscr.
hipError_t launch_step_f32(const StepArgs& a, bool llds, size_t dyn, hipStream_t st);
hipError_t launch_step_f64(const StepArgs& a, bool llds, size_t dyn, hipStream_t st);
hipError_t launch_step_f16(const StepArgs& a, bool llds, size_t dyn, hipStream_t st);
hipError_t launch_colsum(const ColsumArgs& a, int max_p, hipStream_t st);  // h2o_prefill.hip
hipError_t launch_snapkv(const SnapArgs& a, int max_p, hipStream_t st);  // h2o_prefill.hip
// SnapKV's votes and selection in one pass (h2o_prefill.hip), for calls that
// fit it (snapkv_fused_fits: prompts up to 1024 positions, observation windows
// up to 32 rows): ca's q, K and scale, sa's selection (and, for groups of more
// than one query head, sa.hbits and the union kernel), the votes written to
// `votes`.
bool snapkv_fused_fits(const SnapArgs& a);
hipError_t launch_snapkv_fused(const ColsumArgs& ca, const SnapArgs& sa, double* votes, hipStream_t st);

// Fixed scratch of h2o_snapkv_select_noalloc: a file-scope device array in
// h2o_prefill.hip, one copy per device, kept until the process ends.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
// This device's copy of that array (its address looked up once per device).
hipError_t noalloc_scratch(char** ptr);  // h2o_prefill.hip
hipError_t launch_compact(const CompactArgs& a, int max_slots, hipStream_t st);
// Relinking the window pages after a window_remap compaction: per sequence,
// block-table entries [front, front + cnt) take entries [src, src + cnt).
struct RemapArgs {
    int32_t* bt;
    int maxp;
    int nseq;
    int32_t seq_b[kMaxArgBatch], seq_front[kMaxArgBatch], seq_src[kMaxArgBatch], seq_cnt[kMaxArgBatch];
};
hipError_t launch_remap(const RemapArgs& a, hipStream_t st);
hipError_t launch_load(const LoadArgs& a, int max_prompt, hipStream_t st);
hipError_t launch_gather(const GatherArgs& a, hipStream_t st);
hipError_t launch_gather_rows(const RowGatherArgs& a, hipStream_t st);
hipError_t launch_block(const BlockArgs& a, hipStream_t st);  // h2o_block.hip

}  // namespace h2o
