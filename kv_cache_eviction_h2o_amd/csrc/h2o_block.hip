// Block-granular eviction on the paged layout ("Attention Sinks and KV cache
// eviction", sec. 5): the cache is managed in 16-token pages, so eviction frees
// whole pages, and the pages whose share of important tokens is lowest go
// first.  A token is important for a KV head when it is among that head's HH
// highest-scored candidate tokens (the heavy hitters of sec. 4.2, equal scores
// favouring the older token); a page's importance is its count of important
// (token, head) pairs over the sequence's KV heads; equal importance sends the
// older page first.
//
// Pages hold 16 consecutive positions and nothing ever moves inside the cache:
// the retained set is a union of whole pages, the block-table row lists them in
// position order, and each page carries its slots' scores and positions.  An
// eviction therefore rewrites one block-table row and hands the pages back;
// no K/V row, score or position is copied.  The candidates -- whole pages past
// the pages holding sink positions and clear of the recent window -- are the
// row entries [js, js + ncand); the host knows ncand and how many pages go (m)
// from the schedule alone (the window's start never moves back, so every page
// evicted so far lay before it), which keeps the host's page accounting exact
// without reading anything back.
//
//   block_importance_kernel  one workgroup per (sequence, KV head): radix
//       select of the head's (c - HH)-th smallest candidate key (score, then
//       newer first; c = 16 ncand tokens), then per candidate page the count
//       of keys above it -> bimp[unit][page entry].
//   block_evict_kernel  one workgroup per sequence: importance summed over the
//       heads, radix select of the m smallest (importance, entry) keys, the
//       row compacted (kept entries in order), the freed pages pushed on the
//       free stack, and per head the evicted score mass added and the count
//       set.  A freed page's slots keep their old contents until an append
//       reuses them; nothing reads a slot past a unit's count.
#include "h2o_device.h"

namespace h2o {
namespace {

constexpr int kBNT = 256;  // threads per workgroup (4 waves)

template <typename ST>
__device__ inline void score_key(ST v, unsigned (&wk)[3])
{
    if constexpr (sizeof(ST) == 4) {
        wk[2] = 0;
        wk[1] = ord32((float)v);
    } else {
        const unsigned long long u = ord64((double)v);
        wk[2] = (unsigned)(u >> 32);
        wk[1] = (unsigned)u;
    }
}

template <typename ST>
__global__ __launch_bounds__(kBNT) void block_importance_kernel(const BlockArgs a)
{
    extern __shared__ int32_t cpage[];  // [ncand] page of each candidate entry
    __shared__ RadixSmem rs;
    const Geometry& gm = a.g;
    const State& S = a.s;
    const int i = blockIdx.x / gm.Hkv, h = blockIdx.x - i * gm.Hkv;
    const int b = a.seq_b[i], nc = a.seq_c[i];
    const int tid = threadIdx.x;
    const int32_t* row = S.bt + (size_t)b * gm.maxp + a.js;
    for (int j = tid; j < nc; j += kBNT) cpage[j] = row[j];
    __syncthreads();
    int K, HH, W;
    schedule(a.sc, a.seq_len[i], K, HH, W);
    const int c = nc * kPageSize;
    const int e = c - HH;  // candidate tokens that are not heavy hitters of this head
    const ST* scp = reinterpret_cast<const ST*>(S.sc);
    const int Hkv = gm.Hkv;
    // key of candidate token jl (entry jl / 16, slot jl % 16): score, then the
    // newer token first (~jl: entries are in position order)
    auto key_of = [&](int jl, unsigned (&wk)[3]) -> bool {
        score_key(scp[((size_t)cpage[jl >> kPageShift] * Hkv + h) * kPageSize + (jl & (kPageSize - 1))], wk);
        wk[0] = ~(unsigned)jl;
        return true;
    };
    const bool all_imp = e <= 0, none_imp = e >= c;
    if (!all_imp && !none_imp) radix_select<kBNT>(key_of, c, e, sizeof(ST) == 4 ? 4 : 0, rs);
    uint8_t* out = S.bimp + ((size_t)b * Hkv + h) * bimp_stride(gm.maxp);
    for (int jb = tid; jb < nc; jb += kBNT) {
        int cnt = all_imp ? kPageSize : 0;
        if (!all_imp && !none_imp) {
#pragma unroll 4
            for (int r = 0; r < kPageSize; ++r) {
                unsigned wk[3];
                key_of(jb * kPageSize + r, wk);
                cnt += key_le(wk, rs) ? 0 : 1;
            }
        }
        out[jb] = (uint8_t)cnt;
    }
}

struct EvictSmem {
    RadixSmem rs;
    ScanSmem scan;
};

template <typename ST>
__global__ __launch_bounds__(kBNT) void block_evict_kernel(const BlockArgs a)
{
    // dynamic LDS: hsum[Hkv] (fp64) | row[npg] | imp[ncand] | freed[m]
    extern __shared__ double dsm_d[];
    __shared__ EvictSmem sm;
    const Geometry& gm = a.g;
    const State& S = a.s;
    const int i = blockIdx.x;
    const int b = a.seq_b[i], n = a.seq_n[i], nc = a.seq_c[i], m = a.seq_m[i];
    const int js = a.js, Hkv = gm.Hkv;
    const int tid = threadIdx.x;
    const int npg = (n + kPageSize - 1) >> kPageShift;
    double* hsum = dsm_d;
    int32_t* row = reinterpret_cast<int32_t*>(hsum + Hkv);
    int32_t* imp = row + npg;
    int32_t* freed = imp + nc;
    int32_t* grow = S.bt + (size_t)b * gm.maxp;
    for (int j = tid; j < npg; j += kBNT) row[j] = grow[j];
    for (int h = tid; h < Hkv; h += kBNT) hsum[h] = 0.0;
    // importance of each candidate entry: the heads' counts (bytes, rows of
    // bimp_stride) read four entries per word and summed in two 16-bit lanes
    // per word (even entries, odd entries): a count is at most 16 per head
    const int bstr = bimp_stride(gm.maxp);
    const uint32_t* bw = reinterpret_cast<const uint32_t*>(S.bimp + (size_t)b * Hkv * bstr);
    for (int wj = tid; wj < (nc + 3) / 4; wj += kBNT) {
        uint32_t ev = 0, od = 0;
#pragma unroll 8
        for (int h = 0; h < Hkv; ++h) {
            const uint32_t x = bw[(size_t)h * (bstr / 4) + wj];
            ev += x & 0x00ff00ffu;
            od += (x >> 8) & 0x00ff00ffu;
        }
        const int j0 = 4 * wj;
        const int v[4] = {(int)(ev & 0xffffu), (int)(od & 0xffffu), (int)(ev >> 16), (int)(od >> 16)};
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (j0 + k < nc) imp[j0 + k] = v[k];
    }
    __syncthreads();

    // the host's candidate range, checked against the stored positions (head
    // 0's; every head of a page holds the same positions): its first page starts
    // past the sinks on a page boundary, its last ends before the recent
    // window, the entry after it reaches into the window, the one before it
    // holds a sink
    {
        int K, HH, W;
        schedule(a.sc, a.seq_len[i], K, HH, W);
        const int wlo = a.seq_len[i] - W;  // first window position
        auto pos0 = [&](int j) { return S.ps[(size_t)row[j] * Hkv * kPageSize]; };
        bool ok = m >= 1 && m <= nc && js + nc <= npg;
        if (ok) {
            const int first = pos0(js);
            const int last = S.ps[(size_t)row[js + nc - 1] * Hkv * kPageSize + kPageSize - 1];
            ok = first >= a.sc.n_sink && (first & (kPageSize - 1)) == 0 && last < wlo &&
                 last - first >= nc * kPageSize - 1;
            if (ok && js + nc < npg) ok = pos0(js + nc) + kPageSize - 1 >= wlo;
            if (ok && js > 0) ok = pos0(js - 1) < a.sc.n_sink;
        }
        if (!ok) {
            if (tid == 0) atomicOr(S.err, kErrBlock);
            return;
        }
    }

    // key: importance, then the entry (older first), packed in one word; the
    // radix passes start at the key's highest nonzero byte
    constexpr int kEntryBits = 13;  // entries < kMaxBlockPages <= 8192
    static_assert(kMaxBlockPages <= (1 << kEntryBits), "entry field too narrow");
    auto key_of = [&](int jb, unsigned (&wk)[3]) -> bool {
        wk[2] = 0;
        wk[1] = 0;
        wk[0] = ((unsigned)imp[jb] << kEntryBits) | (unsigned)jb;
        return true;
    };
    const bool all = m >= nc;
    if (!all) {
        const unsigned top = ((unsigned)(kPageSize * Hkv) << kEntryBits) | ((1u << kEntryBits) - 1);
        const int bytes = (32 - __builtin_clz(top) + 7) / 8;  // 1..4
        radix_select<kBNT>(key_of, nc, m, 12 - bytes, sm.rs);
    }
    auto gone = [&](int jb) {
        if (all) return true;
        unsigned wk[3];
        key_of(jb, wk);
        return key_le(wk, sm.rs);
    };

    // ordered compaction of the candidate entries: thread chunks, block scan
    const int chunk = (nc + kBNT - 1) / kBNT;
    const int lo = tid * chunk, hi = min(nc, lo + chunk);
    int kept = 0;
    for (int jb = lo; jb < hi; ++jb) kept += gone(jb) ? 0 : 1;
    int kept_total;
    int koff = block_excl_scan<kBNT>(kept, sm.scan, &kept_total);
    int voff = (lo < nc ? lo : nc) - koff;  // freed entries before this chunk
    for (int jb = lo; jb < hi; ++jb) {
        const int pg = row[js + jb];
        if (gone(jb)) {
            if (voff < m) {  // exactly m keys are selected (the keys are distinct)
                freed[voff] = pg;
                S.fstack[a.seq_push[i] + voff] = pg;
            }
            ++voff;
        } else {
            grow[js + koff] = pg;
            ++koff;
        }
    }
    if (kept_total != nc - m) {
        if (tid == 0) atomicOr(S.err, kErrBlock);
        return;
    }
    for (int j = js + nc + tid; j < npg; j += kBNT) grow[j - m] = row[j];
    for (int j = npg - m + tid; j < npg; j += kBNT) grow[j] = -1;
    __syncthreads();  // freed[] complete

    // evicted score mass per head over all (head, freed slot) pairs at once;
    // a thread's run of pairs within one head is summed before it goes to LDS
    const ST* scp = reinterpret_cast<const ST*>(S.sc);
    const int nf = m * kPageSize;
    const long long pairs = (long long)Hkv * nf;
    double acc = 0.0;
    int hc = -1;
    for (long long idx = tid; idx < pairs; idx += kBNT) {
        const int h = (int)(idx / nf), q = (int)(idx - (long long)h * nf);
        if (h != hc) {
            if (hc >= 0) atomicAdd(&hsum[hc], acc);
            acc = 0.0;
            hc = h;
        }
        acc += (double)scp[((size_t)freed[q >> kPageShift] * Hkv + h) * kPageSize + (q & (kPageSize - 1))];
    }
    if (hc >= 0) atomicAdd(&hsum[hc], acc);
    __syncthreads();
    for (int h = tid; h < Hkv; h += kBNT) {
        const size_t u = (size_t)b * Hkv + h;
        S.emass[u] += hsum[h];
        S.cnt[u] = n - nf;
    }
}

}  // namespace

hipError_t launch_block(const BlockArgs& a, hipStream_t st)
{
    if (a.nseq <= 0) return hipSuccess;
    int max_c = 1, max_dyn = 1;
    for (int i = 0; i < a.nseq; ++i) {
        const int npg = (a.seq_n[i] + kPageSize - 1) >> kPageShift;
        max_c = max(max_c, a.seq_c[i]);
        max_dyn = max(max_dyn, npg + a.seq_c[i] + a.seq_m[i]);
    }
    const size_t dyn1 = (size_t)max_c * 4, dyn2 = (size_t)a.g.Hkv * 8 + (size_t)max_dyn * 4;
    const bool f64 = a.g.score_f64 != 0;
    const void* k1 = f64 ? (const void*)block_importance_kernel<double> : (const void*)block_importance_kernel<float>;
    const void* k2 = f64 ? (const void*)block_evict_kernel<double> : (const void*)block_evict_kernel<float>;
    hipError_t e;
    static DynLdsLimit lim1[2], lim2[2];  // per kernel: [fp32 scores, fp64 scores]
    if ((e = lim1[f64].allow(k1, dyn1)) != hipSuccess || (e = lim2[f64].allow(k2, dyn2)) != hipSuccess) return e;
    if (f64)
        hipLaunchKernelGGL(block_importance_kernel<double>, dim3(a.nseq * a.g.Hkv), dim3(kBNT), dyn1, st, a);
    else
        hipLaunchKernelGGL(block_importance_kernel<float>, dim3(a.nseq * a.g.Hkv), dim3(kBNT), dyn1, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (f64)
        hipLaunchKernelGGL(block_evict_kernel<double>, dim3(a.nseq), dim3(kBNT), dyn2, st, a);
    else
        hipLaunchKernelGGL(block_evict_kernel<float>, dim3(a.nseq), dim3(kBNT), dyn2, st, a);
    return hipGetLastError();
}

}  // namespace h2o
