// gfx950 kernels of the H2O decode step.
//
// One workgroup owns one (sequence b, KV head h) unit for the whole step, so
// the softmax normaliser, the score update, the selection and the hole fill
// need no cross-workgroup traffic:
//
//   phase 1  stream the unit's retained K and V rows from HBM once, 16-byte
//            vector loads, 16 lanes per 256-byte row, several rows in flight
//            per lane; q.k by FMA with a 16-lane DPP row reduction; online
//            softmax (running max / sum / output per lane group), combined
//            across lane groups with shuffles and across waves in LDS.  The
//            logits (log2 domain) are parked in LDS for phase 2.
//   phase 2  (H2O) p = 2^(s - M) / L per slot, summed over the GQA group,
//            added to the cumulative score (read-modify-write, fp32 or fp64);
//            the masked arg-min (score ascending, position descending) over
//            the candidates outside the sinks and the recent window gives the
//            victim when one token is to go.
//   phase 3  bulk eviction (first step, Random Attention events): workgroup
//            radix select of the e smallest 96-bit keys, victims marked; then
//            the hole fill moves live tail slots into the holes in place.
//
// Definitions followed: "Attention Sinks and KV cache eviction" sec. 3.1
// (softmax), sec. 4.1 (sinks), sec. 4.2 (cumulative score, sinks + heavy
// hitters + recent window); "H2O: Heavy-Hitter Oracle" summary (budget K,
// greedy eviction of the lowest cumulative score); "Random Attention"
// method (prompt kept, per-head uniform eviction, period K with buffer r);
// Philox4x64-10 from Salmon et al., SC'11.
#include "h2o_internal.h"

#include <hip/hip_runtime.h>

#include <type_traits>

namespace h2o {
namespace {

// ---------------------------------------------------------------- row formats
struct RowBf16 {  // 8 bf16 per 16-byte vector; widening is exact
    static constexpr int EPL = 8;
    __device__ static inline void unpack(const uint4& r, float (&x)[8])
    {
        x[0] = __uint_as_float(r.x << 16);
        x[1] = __uint_as_float(r.x & 0xffff0000u);
        x[2] = __uint_as_float(r.y << 16);
        x[3] = __uint_as_float(r.y & 0xffff0000u);
        x[4] = __uint_as_float(r.z << 16);
        x[5] = __uint_as_float(r.z & 0xffff0000u);
        x[6] = __uint_as_float(r.w << 16);
        x[7] = __uint_as_float(r.w & 0xffff0000u);
    }
};

struct RowF32 {  // 4 fp32 per 16-byte vector
    static constexpr int EPL = 4;
    __device__ static inline void unpack(const uint4& r, float (&x)[4])
    {
        x[0] = __uint_as_float(r.x);
        x[1] = __uint_as_float(r.y);
        x[2] = __uint_as_float(r.z);
        x[3] = __uint_as_float(r.w);
    }
};

// -------------------------------------------------------------- reductions
template <int CTRL>
__device__ inline float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over each row of 16 lanes, result in every lane of the row:
// quad_perm(1,0,3,2), quad_perm(2,3,0,1), row_half_mirror, row_mirror.
__device__ inline float sum16(float v)
{
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    v += dpp<0x140>(v);
    return v;
}

// sum16 of N independent values, one DPP stage at a time across them so the
// wait states each DPP read needs are filled by the other rows' work.
template <int N>
__device__ inline void sum16_n(float (&v)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp<0xB1>(v[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp<0x4E>(v[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp<0x141>(v[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp<0x140>(v[i]);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-row exchange within a wave (gfx950 permlane swaps).  Swapping a value
// with itself leaves, in every lane, the pair (own row's value, partner row's
// value) in some order; a commutative combine of the pair then gives every
// lane the result for rows {r, r^1} (x16) or halves {lo, hi} (x32).
struct Pair {
    unsigned a, b;
};
__device__ inline Pair xrow16(unsigned v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return {r[0], r[1]};
}
__device__ inline Pair xrow32(unsigned v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return {r[0], r[1]};
}

// Raw buffer access (gfx9 family resource word 3): reads past num_records
// bytes return zero without touching memory.
constexpr int kBufWord3 = 0x00020000;
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufWord3);
}
__device__ inline uint4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    uint4 v;
    __builtin_memcpy(&v, &x, 16);
    return v;
}

// Barrier for exchanges through LDS only: waits for this wave's LDS accesses,
// not for its global stores (which __syncthreads' release fence would wait for).
__device__ inline void lds_barrier()
{
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct ScanSmem {
    int wsum[16];
    int total;
};

// Exclusive scan of one int per thread over the workgroup; returns the
// thread's offset, *total receives the sum.  Contains barriers.
template <int NT>
__device__ int block_excl_scan(int v, ScanSmem& ss, int* total)
{
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
    }
    if (lane == 63) ss.wsum[w] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int i = 0; i < NW; ++i) {
            const int x = ss.wsum[i];
            ss.wsum[i] = run;
            run += x;
        }
        ss.total = run;
    }
    __syncthreads();
    const int r = ss.wsum[w] + inc - v;
    *total = ss.total;
    __syncthreads();
    return r;
}

template <int NT>
__device__ double block_sum_f64(double v, double* sh)
{
    constexpr int NW = NT / 64;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) sh[w] = v;
    __syncthreads();
    double s = 0.0;
    if (threadIdx.x == 0)
        for (int i = 0; i < NW; ++i) s += sh[i];
    __syncthreads();
    return s;  // valid in thread 0
}

template <int NT>
__device__ int block_sum_i32(int v, int* sh)
{
    constexpr int NW = NT / 64;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) sh[w] = v;
    __syncthreads();
    int s = 0;
    for (int i = 0; i < NW; ++i) s += sh[i];
    __syncthreads();
    return s;  // valid in every thread
}

// ------------------------------------------------------------- wave arg-min
// (score, position, slot) triples; smaller score wins, equal scores go to the
// higher position (so the lower position is kept); slot < 0 = no candidate.
template <typename ST>
__device__ inline void take_better(ST& bs, int& bp, int& bj, ST os, int op, int oj)
{
    if (oj >= 0 && (bj < 0 || os < bs || (os == bs && op > bp))) {
        bs = os;
        bp = op;
        bj = oj;
    }
}

template <int CTRL>
__device__ inline int dpp_i(int v)
{
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

template <int CTRL, typename ST>
__device__ inline ST dpp_s(ST v)
{
    if constexpr (sizeof(ST) == 4) {
        return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
    } else {
        const long long u = __double_as_longlong(v);
        const int lo = dpp_i<CTRL>((int)(u & 0xffffffffll)), hi = dpp_i<CTRL>((int)(u >> 32));
        return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
    }
}

template <int CTRL, typename ST>
__device__ inline void argmin_step(ST& bs, int& bp, int& bj)
{
    take_better(bs, bp, bj, dpp_s<CTRL>(bs), dpp_i<CTRL>(bp), dpp_i<CTRL>(bj));
}

// Every lane ends with the wave's best: four DPP stages within each row of
// 16 lanes (quad_perm 1,0,3,2 / 2,3,0,1, row_half_mirror, row_mirror), then
// two lane shuffles across the rows.
template <bool X32, typename ST>
__device__ inline void argmin_xrow(ST& bs, int& bp, int& bj)
{
    auto sw = [](unsigned v) { return X32 ? xrow32(v) : xrow16(v); };
    const Pair p = sw((unsigned)bp), j = sw((unsigned)bj);
    ST s0, s1;
    if constexpr (sizeof(ST) == 4) {
        const Pair q = sw(__float_as_uint(bs));
        s0 = __uint_as_float(q.a);
        s1 = __uint_as_float(q.b);
    } else {
        const unsigned long long u = (unsigned long long)__double_as_longlong(bs);
        const Pair lo = sw((unsigned)u), hi = sw((unsigned)(u >> 32));
        s0 = __longlong_as_double((long long)(((unsigned long long)hi.a << 32) | lo.a));
        s1 = __longlong_as_double((long long)(((unsigned long long)hi.b << 32) | lo.b));
    }
    ST rs = s0;
    int rp = (int)p.a, rj = (int)j.a;
    take_better(rs, rp, rj, s1, (int)p.b, (int)j.b);
    bs = rs;
    bp = rp;
    bj = rj;
}

template <typename ST>
__device__ inline void wave_argmin(ST& bs, int& bp, int& bj)
{
    argmin_step<0xB1>(bs, bp, bj);
    argmin_step<0x4E>(bs, bp, bj);
    argmin_step<0x141>(bs, bp, bj);
    argmin_step<0x140>(bs, bp, bj);
    argmin_xrow<false>(bs, bp, bj);
    argmin_xrow<true>(bs, bp, bj);
}

// ------------------------------------------------------------------ Philox
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): word 0 of the block at
// counter (c0, c1, c2, c3) under key (k0, k1).
__device__ inline unsigned long long philox_word0(unsigned long long c0, unsigned long long c1,
                                                  unsigned long long c2, unsigned long long c3,
                                                  unsigned long long k0, unsigned long long k1)
{
    constexpr unsigned long long M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    constexpr unsigned long long W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += W0;
            k1 += W1;
        }
        const unsigned long long hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
        const unsigned long long hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
        const unsigned long long y0 = hi1 ^ c1 ^ k0, y2 = hi0 ^ c3 ^ k1;
        c0 = y0;
        c1 = lo1;
        c2 = y2;
        c3 = lo0;
    }
    return c0;
}

// Order-preserving unsigned image of a float / double (for radix keys).
__device__ inline unsigned ord32(float f)
{
    const unsigned u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline unsigned long long ord64(double f)
{
    const unsigned long long u = (unsigned long long)__double_as_longlong(f);
    return (u >> 63) ? ~u : (u | (1ull << 63));
}

// ----------------------------------------------------------- radix select
// Workgroup radix select of the e smallest 96-bit keys (w[2] most
// significant) among the candidates key_of() accepts, 8 bits per pass,
// starting at digit d0 (digits 0..3 of w[2], 4..7 of w[1], 8..11 of w[0]).
// Keys are unique (the low word holds ~position).  On return the selected
// prefix p[] / mask mk[] satisfy: victim <=> (w & mk) <= p lexicographically.
struct RadixSmem {
    unsigned hist[256];
    unsigned p[3], mk[3];
    unsigned rem, sel_bin, sel_below, sel_cnt;
    int done;
};

template <int NT, typename KeyFn>
__device__ void radix_select(KeyFn key_of, int n_att, int e, int d0, RadixSmem& rs)
{
    const int tid = threadIdx.x;
    if (tid == 0) {
        rs.p[0] = rs.p[1] = rs.p[2] = 0;
        rs.mk[0] = rs.mk[1] = rs.mk[2] = 0;
        rs.rem = (unsigned)e;
        rs.sel_bin = rs.sel_below = rs.sel_cnt = 0;
        rs.done = 0;
    }
    __syncthreads();
    for (int d = d0; d < 12; ++d) {
        for (int i = tid; i < 256; i += NT) rs.hist[i] = 0;
        __syncthreads();
        const int wi = 2 - (d >> 2);
        const int sh = 24 - 8 * (d & 3);
        const unsigned p0 = rs.p[0], p1 = rs.p[1], p2 = rs.p[2];
        const unsigned m0 = rs.mk[0], m1 = rs.mk[1], m2 = rs.mk[2];
        for (int j = tid; j < n_att; j += NT) {
            unsigned w[3];
            if (key_of(j, w) && (w[0] & m0) == p0 && (w[1] & m1) == p1 && (w[2] & m2) == p2)
            {
                const unsigned word = wi == 2 ? w[2] : (wi == 1 ? w[1] : w[0]);
                atomicAdd(&rs.hist[(word >> sh) & 255u], 1u);
            }
        }
        __syncthreads();
        if (tid < 64) {
            unsigned c[4], loc = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                c[k] = rs.hist[tid * 4 + k];
                loc += c[k];
            }
            unsigned inc = loc;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const unsigned y = __shfl_up(inc, off);
                if (tid >= off) inc += y;
            }
            unsigned run = inc - loc;
            const unsigned rem = rs.rem;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (run < rem && rem <= run + c[k]) {
                    rs.sel_bin = (unsigned)(tid * 4 + k);
                    rs.sel_below = run;
                    rs.sel_cnt = c[k];
                }
                run += c[k];
            }
        }
        __syncthreads();
        if (tid == 0) {
            rs.rem -= rs.sel_below;
            rs.p[wi] |= rs.sel_bin << sh;
            rs.mk[wi] |= 255u << sh;
            if (rs.sel_cnt == rs.rem) rs.done = 1;
        }
        __syncthreads();
        if (rs.done) break;
    }
}

__device__ inline bool key_le(const unsigned (&w)[3], const RadixSmem& rs)
{
    const unsigned a2 = w[2] & rs.mk[2], a1 = w[1] & rs.mk[1], a0 = w[0] & rs.mk[0];
    if (a2 != rs.p[2]) return a2 < rs.p[2];
    if (a1 != rs.p[1]) return a1 < rs.p[1];
    return a0 <= rs.p[0];
}

// ------------------------------------------------------------- hole fill
// Writes, in slot order, the slots j in [lo, hi) for which pred(j) holds into
// list[0..count), returns count (in every thread).  Contains barriers.
template <int NT, typename Pred>
__device__ int collect(int lo, int hi, Pred pred, int32_t* list, ScanSmem& ss)
{
    const int n = hi > lo ? hi - lo : 0;
    const int chunk = (n + NT - 1) / NT;
    const int a = lo + (int)threadIdx.x * chunk;
    const int z = min(hi, a + chunk);
    int c = 0;
    for (int j = a; j < z; ++j) c += pred(j) ? 1 : 0;
    int total;
    int off = block_excl_scan<NT>(c, ss, &total);
    for (int j = a; j < z; ++j)
        if (pred(j)) list[off++] = j;
    return total;
}

// In-place compaction of one unit: live slots of [n2, n_att) move into the
// holes (ps == -1) of [0, n2), n2 = n_att - e.  Sources and destinations are
// disjoint, so every move is independent.  Contains barriers.
template <int NT, typename ST, typename SlotFn>
__device__ void fill_holes(const State& s, SlotFn sidx, int unit, int cap, int n_att, int e,
                           bool has_scores, ScanSmem& ss)
{
    const int n2 = n_att - e;
    int32_t* hl = s.iscr + (size_t)unit * 2 * cap;
    int32_t* ll = hl + cap;
    int32_t* ps = s.ps;
    const int nh = collect<NT>(0, n2, [&](int j) { return ps[sidx(j)] < 0; }, hl, ss);
    const int nl = collect<NT>(n2, n_att, [&](int j) { return ps[sidx(j)] >= 0; }, ll, ss);
    __syncthreads();
    if (nh != nl) {
        if (threadIdx.x == 0) atomicOr(s.err, kErrCompact);
        return;
    }
    uint4* kc = (uint4*)s.kc;
    uint4* vc = (uint4*)s.vc;
    ST* sc = (ST*)s.sc;
    const int sub = threadIdx.x & 15, grp = threadIdx.x >> 4;
    for (int i = grp; i < nh; i += NT / 16) {
        const size_t src = sidx(ll[i]), dst = sidx(hl[i]);
        kc[dst * kRowVecs + sub] = kc[src * kRowVecs + sub];
        vc[dst * kRowVecs + sub] = vc[src * kRowVecs + sub];
        if (sub == 0) {
            if (has_scores) sc[dst] = sc[src];
            ps[dst] = ps[src];
        }
    }
}

template <bool PAGED>
struct SlotMap {
    size_t base;        // contiguous: first slot of the unit
    const int32_t* bt;  // paged: the sequence's block-table row
    int h, Hkv;
    __device__ inline size_t operator()(int slot) const
    {
        if constexpr (PAGED)
            return ((size_t)bt[slot >> kPageShift] * Hkv + h) * kPageSize + (slot & (kPageSize - 1));
        else
            return base + (size_t)slot;
    }
};

// ------------------------------------------------------------- step kernel
template <int G>
struct StepTune {
    static constexpr int NT = G <= 2 ? 512 : 256;             // threads per unit
    static constexpr int U = G <= 2 ? 4 : (G == 4 ? 4 : 2);   // rows per lane group per batch
    static constexpr int PF = G <= 2 ? 2 : 5;                 // slots per thread whose score and
                                                              // position are fetched up front
};

template <typename Row, int G, typename ST, bool PAGED, bool LLDS>
__global__ void __launch_bounds__(StepTune<G>::NT) step_kernel(const StepArgs a)
{
    constexpr int NT = StepTune<G>::NT;
    constexpr int U = StepTune<G>::U;
    constexpr int PF = StepTune<G>::PF;
    constexpr int EPL = Row::EPL;
    constexpr int NGRP = NT / 16;
    constexpr int NW = NT / 64;
    constexpr int DR = 16 * EPL;  // head_dim

    extern __shared__ __align__(16) unsigned char dsm[];
    __shared__ float red_m[NW][G], red_l[NW][G];
    __shared__ __align__(16) float red_o[NW][G][DR];
    __shared__ ST s_new_score;
    __shared__ ST s_bs[NW];
    __shared__ int s_bp[NW], s_bj[NW];
    __shared__ double s_dsum[NW];
    __shared__ int s_isum[NW];
    __shared__ ScanSmem s_scan;
    __shared__ RadixSmem s_rad;

    const Geometry& gm = a.g;
    const State& S = a.s;
    const int unit = blockIdx.x;
    const int b = unit / gm.Hkv, h = unit - b * gm.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, sub = tid & 15, grp = tid >> 4;

    // the host knows every sequence's prompt length and retained count: taking
    // them from the arguments saves a dependent memory round trip at the start
    const int P = a.seq_in_args ? a.seq_p[b] : S.t0[b];
    const int t = P + a.step;
    const int n = a.seq_in_args ? a.seq_n[b] : S.cnt[unit];
    const int n_att = n + 1;
    const bool h2o = a.sc.selector == 0;
    const int e = evict_count(a.sc, t, P, n_att);
    const bool inplace_new = a.fused && h2o && e == 1;  // new token goes straight into the hole

    float* logit = LLDS ? reinterpret_cast<float*>(dsm) : S.lscr + (size_t)unit * G * gm.cap;
    const int lstride = LLDS ? a.lds_n : gm.cap;

    SlotMap<PAGED> sidx;
    sidx.base = (size_t)unit * gm.cap;
    sidx.h = h;
    sidx.Hkv = gm.Hkv;
    sidx.bt = nullptr;
    if constexpr (PAGED) {
        int32_t* bts = reinterpret_cast<int32_t*>(dsm + (LLDS ? (size_t)G * a.lds_n * 4 : 0));
        const int npg = (n + kPageSize - 1) >> kPageShift;
        for (int i = tid; i < npg; i += NT) bts[i] = S.bt[(size_t)b * gm.maxp + i];
        if (!inplace_new && (n & (kPageSize - 1)) == 0) {
            const int np = a.newpage[b];
            if (np < 0) {  // the host did not provide the append page: do nothing
                if (tid == 0) atomicOr(S.err, kErrCompact);
                return;
            }
            if (tid == 0) {
                bts[n >> kPageShift] = np;
                if (h == 0) S.bt[(size_t)b * gm.maxp + (n >> kPageShift)] = np;
            }
        }
        sidx.bt = bts;
        __syncthreads();
    }

    // ---- phase 1: q.K, online softmax, P.V over the n_att slots -----------
    // Loads are issued in the order their data is needed (q and the new token,
    // then the first batch of K and V rows, then phase 2's scores): the vector
    // memory counter retires in order, so waiting for an early load never
    // waits for the ones behind it.
    ST* scp = reinterpret_cast<ST*>(S.sc);
    int32_t* psp = S.ps;
    float4 qraw[G][EPL / 4];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float4* qp = reinterpret_cast<const float4*>(
            a.q + ((size_t)b * gm.Hq + (size_t)h * G + g) * DR + sub * EPL);
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i) qraw[g][i] = qp[i];
    }
    const uint4 knr = reinterpret_cast<const uint4*>(a.kn)[(size_t)unit * kRowVecs + sub];
    const uint4 vnr = reinterpret_cast<const uint4*>(a.vn)[(size_t)unit * kRowVecs + sub];
    const uint4* kc = reinterpret_cast<const uint4*>(S.kc);
    const uint4* vc = reinterpret_cast<const uint4*>(S.vc);
    // evicted mass of the unit, read now so its update at the end is no round trip
    const double emass0 = S.emass[unit];
    __builtin_amdgcn_sched_barrier(0);  // keep q and the new token ahead of the K/V stream

    // Rows j >= n are masked out by their logit; the new token (j == n) is
    // folded in after the loop.  Every load is unconditional (a conditional
    // load would make the compiler's wait counts conservative at the join and
    // serialise the pipeline).  Contiguous layout: raw buffer loads over the
    // unit's n rows, so rows past them read as zero without a memory access.
    // Paged layout: rows past n read slot 0 (a cache hit).
    __amdgpu_buffer_rsrc_t rk, rv;
    if constexpr (!PAGED) {
        const size_t ub = sidx.base * kRowBytes;
        rk = make_rsrc(reinterpret_cast<const char*>(S.kc) + ub, (unsigned)n * kRowBytes);
        rv = make_rsrc(reinterpret_cast<const char*>(S.vc) + ub, (unsigned)n * kRowBytes);
    }
    auto load_batch = [&](int base, uint4 (&kr)[U], uint4 (&vr)[U]) {
        if constexpr (!PAGED) {
            const unsigned off0 = (unsigned)(base + grp) * kRowBytes + (unsigned)sub * 16u;
#pragma unroll
            for (int u = 0; u < U; ++u) kr[u] = buf_load16(rk, off0 + (unsigned)(u * NGRP * kRowBytes));
#pragma unroll
            for (int u = 0; u < U; ++u) vr[u] = buf_load16(rv, off0 + (unsigned)(u * NGRP * kRowBytes));
        } else {
            size_t r[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = base + grp + NGRP * u;
                r[u] = sidx(j < n ? j : 0) * kRowVecs + sub;
                kr[u] = kc[r[u]];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) vr[u] = vc[r[u]];
        }
    };
    uint4 ka[U], va[U], kb[U], vb[U];
    load_batch(0, ka, va);
    __builtin_amdgcn_sched_barrier(0);

    // scores and positions of this thread's first PF phase-2 slots
    ST pf_s[PF];
    int pf_p[PF];
    if (h2o) {
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            const int j = tid + k * NT;
            const size_t si = sidx(j < n ? j : 0);
            pf_s[k] = scp[si];
            pf_p[k] = psp[si];
        }
    }

    float qr[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i) {
            qr[g][4 * i + 0] = qraw[g][i].x * a.qscale;
            qr[g][4 * i + 1] = qraw[g][i].y * a.qscale;
            qr[g][4 * i + 2] = qraw[g][i].z * a.qscale;
            qr[g][4 * i + 3] = qraw[g][i].w * a.qscale;
        }
    // running max starts at a finite floor: a lane group that owns no valid
    // row keeps m = floor, l = 0, and 2^(-inf - floor) = 0 for masked rows
    constexpr float kMaxFloor = -1e30f;
    float m[G], l[G], o[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = kMaxFloor;
        l[g] = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) o[g][i] = 0.f;
    }

    // logits of nr rows (K), running max, then P.V (V); rows with !valid[u]
    // take no weight
    auto accumulate = [&](float (&s)[U][G], const uint4 (&vr)[U], int nr) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float mx = m[g];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (u < nr) mx = fmaxf(mx, s[u][g]);
            const float al = fast_exp2(m[g] - mx);
            l[g] *= al;
#pragma unroll
            for (int i = 0; i < EPL; ++i) o[g][i] *= al;
            m[g] = mx;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u >= nr) continue;
            float vx[EPL];
            Row::unpack(vr[u], vx);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float p = fast_exp2(s[u][g] - m[g]);  // 2^-inf = 0 for masked rows
                l[g] += p;
#pragma unroll
                for (int i = 0; i < EPL; ++i) o[g][i] = fmaf(p, vx[i], o[g][i]);
            }
        }
    };
    auto logits = [&](const uint4 (&kr)[U], float (&s)[U][G]) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float acc[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float kx[EPL];
                Row::unpack(kr[u], kx);
                acc[u] = 0.f;
#pragma unroll
                for (int i = 0; i < EPL; ++i) acc[u] = fmaf(qr[g][i], kx[i], acc[u]);
            }
            sum16_n<U>(acc);
#pragma unroll
            for (int u = 0; u < U; ++u) s[u][g] = acc[u];
        }
    };
    auto process = [&](int base, const uint4 (&kr)[U], const uint4 (&vr)[U]) {
        float s[U][G];
        logits(kr, s);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + grp + NGRP * u;
            if (j < n) {
                if (h2o) {
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        if (sub == g) logit[(size_t)g * lstride + j] = s[u][g];
                }
            } else {
#pragma unroll
                for (int g = 0; g < G; ++g) s[u][g] = -INFINITY;
            }
        }
        accumulate(s, vr, U);
    };
    // the new token (position t, slot n) is lane group 0's first row; this
    // runs while the first K/V batch is still in flight
    if (grp == 0) {
        uint4 kn1[U], vn1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            kn1[u] = knr;
            vn1[u] = vnr;
        }
        float s1[U][G];
        logits(kn1, s1);
        if (h2o) {
#pragma unroll
            for (int g = 0; g < G; ++g)
                if (sub == g) logit[(size_t)g * lstride + n] = s1[0][g];
        }
        accumulate(s1, vn1, 1);
    }
    // Batch b+1 is requested before batch b is consumed.  Two register sets
    // alternate (no copies, which would wait for the loads in flight) and the
    // tail is peeled so that the loop body holds no conditional load.
    constexpr int BR = NGRP * U;  // rows per batch
    const int nbatch = (n_att + BR - 1) / BR;
    int bi = 0;
    for (; bi + 2 < nbatch; bi += 2) {
        load_batch((bi + 1) * BR, kb, vb);
        process(bi * BR, ka, va);
        load_batch((bi + 2) * BR, ka, va);
        process((bi + 1) * BR, kb, vb);
    }
    if (bi + 1 < nbatch) {
        load_batch((bi + 1) * BR, kb, vb);
        process(bi * BR, ka, va);
        process((bi + 1) * BR, kb, vb);
    } else {
        process(bi * BR, ka, va);
    }
    // the new token's row goes to slot n unless it fills a victim's hole later
    if (!inplace_new && tid < 16) {
        const size_t r = sidx(n) * kRowVecs + sub;
        reinterpret_cast<uint4*>(S.kc)[r] = knr;
        reinterpret_cast<uint4*>(S.vc)[r] = vnr;
    }

    // merge the four lane groups (rows) of each wave with permlane swaps,
    // then the waves through LDS: one barrier, after which every thread
    // derives the normaliser itself
    auto merge = [&](auto xrow) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const Pair pm = xrow(__float_as_uint(m[g])), pl = xrow(__float_as_uint(l[g]));
            const float m0 = __uint_as_float(pm.a), m1 = __uint_as_float(pm.b);
            const float M = fmaxf(m0, m1);
            const float a0 = fast_exp2(m0 - M), a1 = fast_exp2(m1 - M);
            l[g] = __uint_as_float(pl.a) * a0 + __uint_as_float(pl.b) * a1;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const Pair po = xrow(__float_as_uint(o[g][i]));
                o[g][i] = __uint_as_float(po.a) * a0 + __uint_as_float(po.b) * a1;
            }
            m[g] = M;
        }
    };
    merge([](unsigned v) { return xrow16(v); });
    merge([](unsigned v) { return xrow32(v); });
    if (lane < 16) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int i = 0; i < EPL; ++i) red_o[w][g][sub * EPL + i] = o[g][i];
            if (sub == 0) {
                red_m[w][g] = m[g];
                red_l[w][g] = l[g];
            }
        }
    }
    // logits kept in global scratch (very long units) need the full fence
    if constexpr (LLDS) lds_barrier(); else __syncthreads();
    float Mg[G], invLg[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float M = kMaxFloor;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, red_m[ww][g]);
        float L = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) L += red_l[ww][g] * fast_exp2(red_m[ww][g] - M);
        Mg[g] = M;
        invLg[g] = 1.0f / L;
    }
    for (int idx = tid; idx < G * 16; idx += NT) {
        const int g = idx >> 4, sb = idx & 15;
        float acc[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) acc[i] = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float f = fast_exp2(red_m[ww][g] - Mg[g]);
#pragma unroll
            for (int i = 0; i < EPL; ++i) acc[i] += red_o[ww][g][sb * EPL + i] * f;
        }
        float4* op = reinterpret_cast<float4*>(a.out + ((size_t)b * gm.Hq + (size_t)h * G + g) * DR +
                                               sb * EPL);
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i)
            op[i] = make_float4(acc[4 * i] * invLg[g], acc[4 * i + 1] * invLg[g],
                                acc[4 * i + 2] * invLg[g], acc[4 * i + 3] * invLg[g]);
    }

    int K = 0, HH = 0, W = 0;
    if (h2o) schedule(a.sc, t + 1, K, HH, W);
    const int lo_c = a.sc.n_sink, hi_c = t + 1 - W;  // H2O candidates: lo_c <= pos < hi_c

    // ---- phase 2 (H2O): accumulate scores; arg-min when one token goes ---
    if (h2o) {
        ST bs = (ST)0;
        int bp = -1, bj = -1;
        // slot j: add its weights of this step (summed over the group) to its
        // score; the new token (j == n) starts from zero
        auto visit = [&](int j, ST old, int pos) {
            float p = 0.f;
#pragma unroll
            for (int g = 0; g < G; ++g)
                p += fast_exp2(logit[(size_t)g * lstride + j] - Mg[g]) * invLg[g];
            const ST nw = old + (ST)p;
            if (j < n) {
                scp[sidx(j)] = nw;
            } else {
                s_new_score = nw;
                if (!inplace_new) {
                    const size_t si = sidx(n);
                    scp[si] = nw;
                    psp[si] = t;
                }
            }
            if (e == 1 && pos >= lo_c && pos < hi_c) {
                if (bj < 0 || nw < bs || (nw == bs && pos > bp)) {
                    bs = nw;
                    bp = pos;
                    bj = j;
                }
            }
        };
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            const int j = tid + k * NT;
            if (j < n_att) visit(j, j < n ? pf_s[k] : (ST)0, j < n ? pf_p[k] : t);
        }
        for (int j = tid + PF * NT; j < n_att; j += NT) {
            if (j < n) {
                const size_t si = sidx(j);
                visit(j, scp[si], psp[si]);
            } else {
                visit(j, (ST)0, t);
            }
        }
        if (e == 1) {
            wave_argmin(bs, bp, bj);
            if (lane == 0) {
                s_bs[w] = bs;
                s_bp[w] = bp;
                s_bj[w] = bj;
            }
            lds_barrier();
            ST vs = s_bs[0];
            int vp = s_bp[0], vjj = s_bj[0];
#pragma unroll
            for (int ww = 1; ww < NW; ++ww) take_better(vs, vp, vjj, s_bs[ww], s_bp[ww], s_bj[ww]);
            const int vj = vjj;
            if (vj < 0) {
                if (tid == 0) atomicOr(S.err, kErrNoCandidate);
                return;
            }
            if (tid == 0) S.emass[unit] = emass0 + (double)vs;
            // the victim slot's score / position are written by the thread that
            // wrote its updated score above: same thread, same address, in order
            const bool owner = (vj - tid) % NT == 0;
            if (a.fused) {
                if (vj != n) {
                    if (tid < 16) {
                        const size_t r = sidx(vj) * kRowVecs + sub;
                        reinterpret_cast<uint4*>(S.kc)[r] = knr;
                        reinterpret_cast<uint4*>(S.vc)[r] = vnr;
                    }
                    if (owner) {
                        scp[sidx(vj)] = s_new_score;
                        psp[sidx(vj)] = t;
                    }
                }
                // the count stays n: one in, one out
            } else {
                if (owner) psp[sidx(vj)] = -1;
                if (tid == 0) {
                    S.vinfo[2 * unit] = 1;
                    S.vinfo[2 * unit + 1] = vj;
                    S.cnt[unit] = n_att;
                }
            }
            return;
        }
    } else if (tid == 0) {
        psp[sidx(n)] = t;  // Random: no score pass; record the appended position
    }

    if (e == 0) {
        if (tid == 0) {
            S.cnt[unit] = n_att;
            if (!a.fused) {
                S.vinfo[2 * unit] = 0;
                S.vinfo[2 * unit + 1] = -1;
            }
        }
        return;
    }

    // ---- phase 3: bulk selection (e > 1, or a Random Attention event) -----
    __syncthreads();
    int d0;
    double vmass = 0.0;
    int nv = 0;
    if (h2o) {
        auto key_of = [&](int j, unsigned (&wk)[3]) -> bool {
            const size_t si = sidx(j);
            const int pos = psp[si];
            if (pos < lo_c || pos >= hi_c) return false;
            if constexpr (sizeof(ST) == 4) {
                wk[2] = 0;
                wk[1] = ord32((float)scp[si]);
            } else {
                const unsigned long long u = ord64((double)scp[si]);
                wk[2] = (unsigned)(u >> 32);
                wk[1] = (unsigned)u;
            }
            wk[0] = ~(unsigned)pos;
            return true;
        };
        d0 = sizeof(ST) == 4 ? 4 : 0;
        radix_select<NT>(key_of, n_att, e, d0, s_rad);
        for (int j = tid; j < n_att; j += NT) {
            unsigned wk[3];
            if (key_of(j, wk) && key_le(wk, s_rad)) {
                const size_t si = sidx(j);
                vmass += (double)scp[si];
                psp[si] = -1;
                ++nv;
            }
        }
    } else {
        const unsigned long long k0 = a.sc.seed;
        auto key_of = [&](int j, unsigned (&wk)[3]) -> bool {
            const int pos = psp[sidx(j)];
            if (pos < P) return false;
            const unsigned long long x =
                philox_word0((unsigned long long)b, (unsigned long long)h, (unsigned long long)t,
                             (unsigned long long)pos, k0, 0ull);
            wk[2] = (unsigned)(x >> 32);
            wk[1] = (unsigned)x;
            wk[0] = ~(unsigned)pos;
            return true;
        };
        radix_select<NT>(key_of, n_att, e, 0, s_rad);
        for (int j = tid; j < n_att; j += NT) {
            unsigned wk[3];
            if (key_of(j, wk) && key_le(wk, s_rad)) {
                psp[sidx(j)] = -1;
                ++nv;
            }
        }
    }
    const int nv_all = block_sum_i32<NT>(nv, s_isum);
    const double vm = block_sum_f64<NT>(vmass, s_dsum);
    if (tid == 0) {
        if (nv_all != e) atomicOr(S.err, kErrSelectCount);
        if (h2o) S.emass[unit] = emass0 + vm;
    }
    if (a.fused) {
        __syncthreads();
        fill_holes<NT, ST>(S, sidx, unit, gm.cap, n_att, e, h2o, s_scan);
        if (tid == 0) S.cnt[unit] = n_att - e;
    } else if (tid == 0) {
        S.vinfo[2 * unit] = e;
        S.vinfo[2 * unit + 1] = -1;
        S.cnt[unit] = n_att;
    }
}

// ---------------------------------------------------------- compact kernel
constexpr int kCompactNT = 256;

template <typename ST, bool PAGED>
__global__ void __launch_bounds__(kCompactNT) compact_kernel(const CompactArgs a)
{
    __shared__ ScanSmem s_scan;
    const Geometry& gm = a.g;
    const State& S = a.s;
    const int unit = blockIdx.x;
    const int b = unit / gm.Hkv, h = unit - b * gm.Hkv;
    const int e = S.vinfo[2 * unit], v = S.vinfo[2 * unit + 1];
    if (e <= 0) return;
    const int n_att = S.cnt[unit];
    SlotMap<PAGED> sidx;
    sidx.base = (size_t)unit * gm.cap;
    sidx.bt = S.bt + (size_t)b * gm.maxp;
    sidx.h = h;
    sidx.Hkv = gm.Hkv;
    const bool has_scores = S.sc != nullptr;
    if (e == 1) {
        const int last = n_att - 1;
        if (v != last && v >= 0) {
            const int sub = threadIdx.x & 15;
            const size_t src = sidx(last), dst = sidx(v);
            if (threadIdx.x < 16) {
                uint4* kc = (uint4*)S.kc;
                uint4* vc = (uint4*)S.vc;
                kc[dst * kRowVecs + sub] = kc[src * kRowVecs + sub];
                vc[dst * kRowVecs + sub] = vc[src * kRowVecs + sub];
            }
            if (threadIdx.x == 0) {
                if (has_scores) ((ST*)S.sc)[dst] = ((ST*)S.sc)[src];
                S.ps[dst] = S.ps[src];
            }
        }
    } else {
        fill_holes<kCompactNT, ST>(S, sidx, unit, gm.cap, n_att, e, has_scores, s_scan);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        S.cnt[unit] = n_att - e;
        S.vinfo[2 * unit] = 0;
        S.vinfo[2 * unit + 1] = -1;
    }
}

// ------------------------------------------------------------- prompt load
template <typename ST, bool PAGED>
__global__ void __launch_bounds__(256) load_kernel(const LoadArgs a)
{
    const Geometry& gm = a.g;
    const State& S = a.s;
    const int b = blockIdx.y;
    const int P = S.t0[b];
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long total = (long long)P * gm.Hkv * kRowVecs;
    if (idx >= total) return;
    const int tok = (int)(idx / (gm.Hkv * kRowVecs));
    const int rem = (int)(idx - (long long)tok * gm.Hkv * kRowVecs);
    const int h = rem / kRowVecs, c = rem - h * kRowVecs;
    const int unit = b * gm.Hkv + h;
    SlotMap<PAGED> sidx;
    sidx.base = (size_t)unit * gm.cap;
    sidx.bt = S.bt + (size_t)b * gm.maxp;
    sidx.h = h;
    sidx.Hkv = gm.Hkv;
    const size_t src = ((size_t)(S.poff[b] + tok) * gm.Hkv + h) * kRowVecs + c;
    const size_t si = sidx(tok);
    reinterpret_cast<uint4*>(S.kc)[si * kRowVecs + c] = reinterpret_cast<const uint4*>(a.pk)[src];
    reinterpret_cast<uint4*>(S.vc)[si * kRowVecs + c] = reinterpret_cast<const uint4*>(a.pv)[src];
    if (c == 0) {
        if (S.sc)
            ((ST*)S.sc)[si] = a.init_scores
                                  ? (ST)a.init_scores[(size_t)(S.poff[b] + tok) * gm.Hkv + h]
                                  : (ST)0;
        S.ps[si] = tok;
        if (tok == 0) {
            S.cnt[unit] = P;
            S.emass[unit] = 0.0;
            S.vinfo[2 * unit] = 0;
            S.vinfo[2 * unit + 1] = -1;
        }
    }
}

// ------------------------------------------------------------ state gather
template <typename ST, bool PAGED>
__global__ void __launch_bounds__(256) gather_kernel(const GatherArgs a)
{
    const Geometry& gm = a.g;
    const State& S = a.s;
    const int unit = blockIdx.x;
    const int b = unit / gm.Hkv, h = unit - b * gm.Hkv;
    SlotMap<PAGED> sidx;
    sidx.base = (size_t)unit * gm.cap;
    sidx.bt = S.bt + (size_t)b * gm.maxp;
    sidx.h = h;
    sidx.Hkv = gm.Hkv;
    const int n = S.cnt[unit];
    for (int j = threadIdx.x; j < a.capo; j += 256) {
        int32_t p = -1;
        double s = 0.0;
        if (j < n) {
            const size_t si = sidx(j);
            p = S.ps[si];
            if (S.sc && a.selector == 0) s = (double)((const ST*)S.sc)[si];
        }
        a.opos[(size_t)unit * a.capo + j] = p;
        a.osc[(size_t)unit * a.capo + j] = s;
    }
}

// --------------------------------------------------------------- dispatch
template <typename Row, int G, typename ST, bool PAGED, bool LLDS>
hipError_t launch_step_t(const StepArgs& a, size_t dyn, hipStream_t st)
{
    auto k = step_kernel<Row, G, ST, PAGED, LLDS>;
    static size_t dyn_set = 48 * 1024;  // largest dynamic LDS size granted so far
    if (dyn > dyn_set) {
        hipError_t err = hipFuncSetAttribute((const void*)k,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (err != hipSuccess) return err;
        dyn_set = dyn;
    }
    hipLaunchKernelGGL(k, dim3(a.g.B * a.g.Hkv), dim3(StepTune<G>::NT), dyn, st, a);
    return hipGetLastError();
}

template <typename Row, int G, typename ST>
hipError_t dispatch_pl(const StepArgs& a, bool llds, size_t dyn, hipStream_t st)
{
    if (a.g.paged) {
        if constexpr (std::is_same<Row, RowBf16>::value) {  // pages hold bf16 rows only
            return llds ? launch_step_t<Row, G, ST, true, true>(a, dyn, st)
                        : launch_step_t<Row, G, ST, true, false>(a, dyn, st);
        }
        return hipErrorInvalidValue;
    }
    return llds ? launch_step_t<Row, G, ST, false, true>(a, dyn, st)
                : launch_step_t<Row, G, ST, false, false>(a, dyn, st);
}

template <typename Row, typename ST>
hipError_t dispatch_g(const StepArgs& a, bool llds, size_t dyn, hipStream_t st)
{
    switch (a.g.G) {
    case 1: return dispatch_pl<Row, 1, ST>(a, llds, dyn, st);
    case 2: return dispatch_pl<Row, 2, ST>(a, llds, dyn, st);
    case 4: return dispatch_pl<Row, 4, ST>(a, llds, dyn, st);
    case 8: return dispatch_pl<Row, 8, ST>(a, llds, dyn, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_step(const StepArgs& a, int max_n_att, hipStream_t st)
{
    const bool llds = (size_t)a.g.G * (size_t)max_n_att * 4 <= (size_t)kLogitLdsBytes;
    size_t dyn = 0;
    if (llds) dyn += (size_t)a.g.G * (size_t)a.lds_n * 4;
    if (a.g.paged) dyn += (size_t)a.npg_lds * 4;
    dyn = (dyn + 15) & ~(size_t)15;
    if (!llds && a.s.lscr == nullptr) return hipErrorInvalidValue;
    if (a.g.kv_bf16) {
        return a.g.score_f64 ? dispatch_g<RowBf16, double>(a, llds, dyn, st)
                             : dispatch_g<RowBf16, float>(a, llds, dyn, st);
    }
    return a.g.score_f64 ? dispatch_g<RowF32, double>(a, llds, dyn, st)
                         : dispatch_g<RowF32, float>(a, llds, dyn, st);
}

hipError_t launch_compact(const CompactArgs& a, int /*max_slots*/, hipStream_t st)
{
    const dim3 grid(a.g.B * a.g.Hkv), block(kCompactNT);
    if (a.g.paged) {
        if (a.g.score_f64) hipLaunchKernelGGL((compact_kernel<double, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((compact_kernel<float, true>), grid, block, 0, st, a);
    } else {
        if (a.g.score_f64) hipLaunchKernelGGL((compact_kernel<double, false>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((compact_kernel<float, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_load(const LoadArgs& a, int max_prompt, hipStream_t st)
{
    const long long per_seq = (long long)max_prompt * a.g.Hkv * kRowVecs;
    const dim3 grid((unsigned)((per_seq + 255) / 256), a.g.B), block(256);
    if (a.g.paged) {
        if (a.g.score_f64) hipLaunchKernelGGL((load_kernel<double, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((load_kernel<float, true>), grid, block, 0, st, a);
    } else {
        if (a.g.score_f64) hipLaunchKernelGGL((load_kernel<double, false>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((load_kernel<float, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t st)
{
    const dim3 grid(a.g.B * a.g.Hkv), block(256);
    if (a.g.paged) {
        if (a.g.score_f64) hipLaunchKernelGGL((gather_kernel<double, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((gather_kernel<float, true>), grid, block, 0, st, a);
    } else {
        if (a.g.score_f64) hipLaunchKernelGGL((gather_kernel<double, false>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((gather_kernel<float, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace h2o
