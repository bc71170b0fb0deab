// Device-side building blocks shared by the decode-step kernels
// (h2o_kernels.hip: FMA path; h2o_mfma.hip: matrix-core path): lane and wave
// reductions, raw buffer loads, workgroup scans, the arg-min and radix
// selections, Philox4x64-10, the two K/V slot layouts, the hole fill, and the
// part of the step that follows the softmax statistics (score accumulation,
// selection, eviction bookkeeping and in-place compaction).
#pragma once

#include "h2o_internal.h"

#include <hip/hip_runtime.h>

#include <type_traits>

namespace h2o {
namespace {

// ---------------------------------------------------------------- row formats
// A row is read by 16 lanes, EPL elements each from one Vec.  SCALED rows
// stand for code * the row's scale (kept beside the rows).
struct RowBf16 {  // 8 bf16 per 16-byte vector; widening is exact
    static constexpr int EPL = 8;
    static constexpr bool SCALED = false;
    using Vec = uint4;
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
    static constexpr bool SCALED = false;
    using Vec = uint4;
    __device__ static inline void unpack(const uint4& r, float (&x)[4])
    {
        x[0] = __uint_as_float(r.x);
        x[1] = __uint_as_float(r.y);
        x[2] = __uint_as_float(r.z);
        x[3] = __uint_as_float(r.w);
    }
};

struct RowI8 {  // 8 int8 codes per 8-byte vector; the row's scale multiplies them
    static constexpr int EPL = 8;
    static constexpr bool SCALED = true;
    using Vec = uint2;
    __device__ static inline void unpack(const uint2& r, float (&x)[8])
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = (float)(signed char)(r.x >> (8 * i));
            x[4 + i] = (float)(signed char)(r.y >> (8 * i));
        }
    }
};

// -------------------------------------------------------------- reductions
template <int CTRL>
__device__ inline float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Maximum over each row of 16 lanes (same DPP stages as sum16).
__device__ inline float max16(float v)
{
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    return v;
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
// K / V rows (and int8 row scales) are read once per step: their loads carry
// the non-temporal cache policy (the `nt` bit), which streams them past the
// caches instead of allocating lines no later access of the step will hit
// (measured: OPT layer step 13.34 -> 12.26 us, GQA layer 24.77 -> 23.64 us).
constexpr int kStreamPolicy = 2;  // cache-policy operand: nt
__device__ inline uint2 buf_load8(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kStreamPolicy);
    uint2 v;
    __builtin_memcpy(&v, &x, 8);
    return v;
}
__device__ inline uint4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kStreamPolicy);
    uint4 v;
    __builtin_memcpy(&v, &x, 16);
    return v;
}
__device__ inline float buf_load4f(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kStreamPolicy));
}
// One double through the vector memory path (counted by vmcnt, so waits for
// LDS or scalar data never wait for it).
__device__ inline double load_f64(const double* p)
{
    const uint2 v = buf_load8(make_rsrc(p, 8u), 0u);
    return __hiloint2double((int)v.y, (int)v.x);
}
// The same policy on plain global loads (paged rows reached through the block table).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ inline uint4 stream_load(const uint4* p)
{
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ inline uint2 stream_load(const uint2* p)
{
    const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(x[0], x[1]);
}
__device__ inline float stream_load(const float* p) { return __builtin_nontemporal_load(p); }
// Non-temporal stores, for rows written once and not read again by the same
// launch (the moves of a compaction).
__device__ inline void stream_store(uint4* p, const uint4& v)
{
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}
__device__ inline void stream_store(uint2* p, const uint2& v)
{
    __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(p));
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
// higher position (so the lower position is kept).  "No candidate" is
// (+inf, -1, -1): every candidate beats it, a +inf score through the higher
// position.  Branch-free: the compare masks feed selects.
template <typename ST>
__device__ inline void take_better(ST& bs, int& bp, int& bj, ST os, int op, int oj)
{
    const bool take = (os < bs) | ((os == bs) & (op > bp));
    bs = take ? os : bs;
    bp = take ? op : bp;
    bj = take ? oj : bj;
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

// Slots j in [lo, hi), thread tid taking lo + tid, lo + tid + NT, ..., fetched
// UNR at a time: fetch(j) issues slot j's loads and returns them unconsumed,
// then body(j, fetched) runs for each, so a thread keeps UNR slots' loads in
// flight instead of waiting on one dependent load per slot.  Past hi the
// fetch repeats an in-range slot and the body is skipped.
template <int NT, int UNR, typename Fetch, typename Body>
__device__ inline void for_slots_batched(int lo, int hi, Fetch fetch, Body body)
{
    using Raw = decltype(fetch(lo));
    for (int j0 = lo + (int)threadIdx.x; j0 < hi; j0 += NT * UNR) {
        Raw r[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int j = j0 + u * NT;
            r[u] = fetch(j < hi ? j : j0);
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int j = j0 + u * NT;
            if (j < hi) body(j, r[u]);
        }
    }
}

// radix_select with the candidates' data fetched UNR slots at a time:
// src.fetch(j) returns slot j's raw data, src.key(raw, w) its 96-bit key
// (false: not a candidate).  Same contract and result as radix_select.
template <int NT, int UNR, typename Src>
__device__ void radix_select_batched(const Src& src, int n_att, int e, int d0, RadixSmem& rs)
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
        for_slots_batched<NT, UNR>(
            0, n_att, [&](int j) { return src.fetch(j); },
            [&](int, const auto& r) {
                unsigned w[3];
                if (src.key(r, w) && (w[0] & m0) == p0 && (w[1] & m1) == p1 && (w[2] & m2) == p2) {
                    const unsigned word = wi == 2 ? w[2] : (wi == 1 ? w[1] : w[0]);
                    atomicAdd(&rs.hist[(word >> sh) & 255u], 1u);
                }
            });
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

// Shared memory of collect_ordered: per round, the count of each (batch
// index u, wave) cell, then its offset; two buffers alternate between rounds.
template <int NT, int UNR>
struct OrderSmem {
    int off[2][UNR * (NT / 64)];
    int total[2];
};

// The slots j in [lo, hi) with test(fetch(j)) into list[0..count) in
// ascending slot order; returns count (in every thread).  One pass in rounds
// of NT * UNR slots (slot j0 + u * NT + tid: every load coalesced): each
// wave ballots its flags, the first wave turns the (u, wave) counts into
// offsets, and every flagged slot writes itself at its offset plus its rank
// among the lower lanes.  Two barriers per round.
template <int NT, int UNR, typename Fetch, typename Test>
__device__ int collect_ordered(int lo, int hi, Fetch fetch, Test test, int32_t* list, OrderSmem<NT, UNR>& os)
{
    constexpr int NW = NT / 64, E = UNR * NW, PER = (E + 63) / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    using Raw = decltype(fetch(lo));
    int base = 0, r = 0;
    for (int j0 = lo; j0 < hi; j0 += NT * UNR, r ^= 1) {
        Raw v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int j = j0 + u * NT + (int)threadIdx.x;
            v[u] = fetch(j < hi ? j : lo);
        }
        unsigned long long m[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int j = j0 + u * NT + (int)threadIdx.x;
            m[u] = __ballot(j < hi && test(v[u]));
            if (lane == 0) os.off[r][u * NW + w] = __popcll(m[u]);
        }
        __syncthreads();
        if (w == 0) {  // exclusive scan of the E cells in (u, wave) order, PER per lane
            int c[PER], sum = 0;
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int e = lane * PER + k;
                c[k] = e < E ? os.off[r][e] : 0;
                sum += c[k];
            }
            int inc = sum;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int y = __shfl_up(inc, d);
                if (lane >= d) inc += y;
            }
            int run = inc - sum;
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int e = lane * PER + k;
                if (e < E) os.off[r][e] = run;
                run += c[k];
            }
            if (lane == 63) os.total[r] = inc;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            if ((m[u] >> lane) & 1ull) {
                const int rank = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m[u] >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((unsigned)m[u], 0u));
                list[base + os.off[r][u * NW + w] + rank] = j0 + u * NT + (int)threadIdx.x;
            }
        }
        base += os.total[r];
    }
    return base;
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

// ------------------------------------------- bf16 matrix-instruction tiles
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ inline bf16x8 as_bf16x8(const uint4& v)
{
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

__device__ inline f32x4 mma(const bf16x8& a, const bf16x8& b, const f32x4& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The bf16 part of x that a B column holds: x rounded to bf16 (hi column) or
// the rounding residual rounded to bf16 (lo column).
__device__ inline __bf16 split_part(float x, bool lo)
{
    const __bf16 hi = (__bf16)x;
    return lo ? (__bf16)(x - (float)hi) : hi;
}

// ------------------------------------------------------- K/V slot layouts
// A slot index si (the unit's first slot + slot, or the page-derived index)
// names one token's K row and V row.  Rows move as 16 chunks of 16 bytes;
// chunk c holds elements 8c..8c+7 (bf16) or 4c..4c+3 (fp32).
//
// KvRows: the K row of slot si is 16-byte vectors [16 si, 16 si + 16); V alike.
struct KvRows {
    __device__ static inline size_t kvec(size_t si, int c) { return si * kRowVecs + (size_t)c; }
    __device__ static inline void store(void* kc, void* vc, size_t si, int c, uint4 k, uint4 v)
    {
        reinterpret_cast<uint4*>(kc)[kvec(si, c)] = k;
        reinterpret_cast<uint4*>(vc)[kvec(si, c)] = v;
    }
    __device__ static inline void copy(const State& S, size_t src, size_t dst, int c)
    {
        uint4* K = reinterpret_cast<uint4*>(S.kc);
        uint4* V = reinterpret_cast<uint4*>(S.vc);
        K[kvec(dst, c)] = K[kvec(src, c)];
        V[kvec(dst, c)] = V[kvec(src, c)];
    }
    // copy split in two, so several moves' loads can be in flight; the rows
    // moved are read and written once, with the non-temporal policy (paged
    // bulk first step 10.6 -> 9.8 ms)
    struct Chunk {
        uint4 k, v;
    };
    __device__ static inline Chunk fetch(const State& S, size_t si, int c)
    {
        return {stream_load(reinterpret_cast<const uint4*>(S.kc) + kvec(si, c)),
                stream_load(reinterpret_cast<const uint4*>(S.vc) + kvec(si, c))};
    }
    __device__ static inline void put(const State& S, size_t si, int c, const Chunk& x)
    {
        stream_store(reinterpret_cast<uint4*>(S.kc) + kvec(si, c), x.k);
        stream_store(reinterpret_cast<uint4*>(S.vc) + kvec(si, c), x.v);
    }
};

// KvRows8: int8 rows of 128 codes, 16 chunks of 8 bytes; scales beside.
struct KvRows8 {
    __device__ static inline size_t kvec(size_t si, int c) { return si * kRowVecs + (size_t)c; }
    __device__ static inline void copy(const State& S, size_t src, size_t dst, int c)
    {
        uint2* K = reinterpret_cast<uint2*>(S.kc);
        uint2* V = reinterpret_cast<uint2*>(S.vc);
        K[kvec(dst, c)] = K[kvec(src, c)];
        V[kvec(dst, c)] = V[kvec(src, c)];
        if (c == 0) {
            S.kss[dst] = S.kss[src];
            S.vss[dst] = S.vss[src];
        }
    }
    struct Chunk {
        uint2 k, v;
        float ks, vs;  // chunk 0 only
    };
    __device__ static inline Chunk fetch(const State& S, size_t si, int c)
    {
        Chunk x;
        x.k = stream_load(reinterpret_cast<const uint2*>(S.kc) + kvec(si, c));
        x.v = stream_load(reinterpret_cast<const uint2*>(S.vc) + kvec(si, c));
        x.ks = c == 0 ? S.kss[si] : 0.f;
        x.vs = c == 0 ? S.vss[si] : 0.f;
        return x;
    }
    __device__ static inline void put(const State& S, size_t si, int c, const Chunk& x)
    {
        stream_store(reinterpret_cast<uint2*>(S.kc) + kvec(si, c), x.k);
        stream_store(reinterpret_cast<uint2*>(S.vc) + kvec(si, c), x.v);
        if (c == 0) {
            S.kss[si] = x.ks;
            S.vss[si] = x.vs;
        }
    }
};

// Int8 quantisation of one row of 128 held by the 16 lanes of a row group,
// 8 values x[] per lane: scale = max |x| / 127, code = rint(x / scale) in
// [-127, 127] (fp32 throughout; a zero row has scale 0 and codes 0).
__device__ inline void quantize_row8(const float (&x)[8], uint2& codes, float& scale)
{
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[i]));
    a = max16(a);
    scale = a / 127.0f;
    unsigned w[2] = {0u, 0u};
    if (scale > 0.f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float q = fminf(fmaxf(rintf(x[i] / scale), -127.f), 127.f);
            w[i >> 2] |= ((unsigned)(int)q & 0xffu) << (8 * (i & 3));
        }
    }
    codes = make_uint2(w[0], w[1]);
}

// KvTiles (bf16 rows of 128, contiguous slots, unit capacity a multiple of
// 32): the operand orders of the 16x16x32 bf16 matrix instruction.
//   K: 16-slot blocks laid out [chunk c][slot % 16][16 B]: a wave's 16-byte
//      load at vector (block * 256 + kb * 64 + lane) gives lane l the d range
//      32 kb + 8 (l / 16) .. +8 of slot l % 16 -- a 16 x 32 A operand.
//   V: 32-slot blocks laid out [d / 16][lane group q][d % 16][8 slots], lane
//      group q holding slots {4q..4q+3, 16+4q..16+4q+3} in that order: the
//      load at vector (block * 512 + db * 64 + lane) gives lane l, for
//      d = 16 db + l % 16, the 8 slots of its group -- a 16 x 32 A operand
//      of V^T whose k order matches the logit tile's C layout.
// Each wave-wide load reads 1 KB in one piece.
struct KvTiles {
    __device__ static inline size_t kvec(size_t si, int c)
    {
        return (si >> 4) * 256 + (size_t)c * 16 + (si & 15);
    }
    __device__ static inline size_t velem(size_t si, int d)
    {
        const unsigned u = (unsigned)(si & 31);
        return (si >> 5) * 4096 +
               (size_t)((d >> 4) * 512 + (int)((u & 15) >> 2) * 128 + (d & 15) * 8 +
                        (int)(((u >> 4) << 2) | (u & 3)));
    }
    __device__ static inline void store(void* kc, void* vc, size_t si, int c, uint4 k, uint4 v)
    {
        reinterpret_cast<uint4*>(kc)[kvec(si, c)] = k;
        unsigned short* V = reinterpret_cast<unsigned short*>(vc);
        const unsigned w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) V[velem(si, 8 * c + e)] = (unsigned short)(w4[e >> 1] >> (16 * (e & 1)));
    }
    __device__ static inline void copy(const State& S, size_t src, size_t dst, int c)
    {
        uint4* K = reinterpret_cast<uint4*>(S.kc);
        K[kvec(dst, c)] = K[kvec(src, c)];
        unsigned short* V = reinterpret_cast<unsigned short*>(S.vc);
#pragma unroll
        for (int e = 0; e < 8; ++e) V[velem(dst, 8 * c + e)] = V[velem(src, 8 * c + e)];
    }
    struct Chunk {
        uint4 k;
        unsigned short v[8];
    };
    __device__ static inline Chunk fetch(const State& S, size_t si, int c)
    {
        Chunk x;
        x.k = stream_load(reinterpret_cast<const uint4*>(S.kc) + kvec(si, c));
        const unsigned short* V = reinterpret_cast<const unsigned short*>(S.vc);
#pragma unroll
        for (int e = 0; e < 8; ++e) x.v[e] = V[velem(si, 8 * c + e)];
        return x;
    }
    __device__ static inline void put(const State& S, size_t si, int c, const Chunk& x)
    {
        stream_store(reinterpret_cast<uint4*>(S.kc) + kvec(si, c), x.k);
        unsigned short* V = reinterpret_cast<unsigned short*>(S.vc);
#pragma unroll
        for (int e = 0; e < 8; ++e) V[velem(si, 8 * c + e)] = x.v[e];
    }
};

// In-place compaction of one unit: the live slots (ps >= 0) of [l0, l1) and
// then of [l2, l3) move into the holes (ps == -1) of [0, h_end) -- for plain
// compaction [n2, n_att) into [0, n2), n2 = n_att - e.  Sources and
// destinations are disjoint, so every move is independent.  Contains barriers.
// Unroll of the hole fill's list collection (rounds of NT * kCollectUnroll slots).
constexpr int kCollectUnroll = 16;

template <int NT, typename ST, typename KV, typename SlotFn>
__device__ __attribute__((always_inline)) inline void fill_holes(const State& s, SlotFn sidx, int unit, int cap,
                                                                 int h_end, int l0, int l1, int l2, int l3,
                                                                 bool has_scores,
                                                                 OrderSmem<NT, kCollectUnroll>& os)
{
    int32_t* hl = s.iscr + (size_t)unit * 2 * cap;
    int32_t* ll = hl + cap;
    int32_t* ps = s.ps;
    auto pos_at = [&](int j) { return ps[sidx(j)]; };
    // both lists in ascending slot order: the moves of one round then read and
    // write neighbouring rows (a few pages), not rows spread over the pool
    const int nh = collect_ordered<NT, kCollectUnroll>(0, h_end, pos_at, [](int p) { return p < 0; }, hl, os);
    int nl = collect_ordered<NT, kCollectUnroll>(l0, l1, pos_at, [](int p) { return p >= 0; }, ll, os);
    if (l2 < l3) nl += collect_ordered<NT, kCollectUnroll>(l2, l3, pos_at, [](int p) { return p >= 0; }, ll + nl, os);
    __syncthreads();
    if (nh != nl) {
        if (threadIdx.x == 0) atomicOr(s.err, kErrCompact);
        return;
    }
    // moves: a 16-lane group per move, MU moves' loads in flight before their
    // stores (sources and destinations are disjoint, so no move reads another's
    // destination); the list entries of a group's next round are fetched while
    // the current round's rows are in flight, so a round costs one memory
    // round trip, not two
    constexpr int MU = 8, NG = NT / 16;
    ST* sc = (ST*)s.sc;
    const int sub = threadIdx.x & 15, grp = threadIdx.x >> 4;
    int li[MU], hi[MU];
    auto fetch_lists = [&](int i0) {  // entries past the lists re-read the last one (unused)
#pragma unroll
        for (int u = 0; u < MU; ++u) {
            const int i = max(0, min(i0 + u * NG, nh - 1));
            li[u] = ll[i];
            hi[u] = hl[i];
        }
    };
    fetch_lists(grp);
    for (int i0 = grp; i0 < nh; i0 += NG * MU) {
        size_t src[MU], dst[MU];
#pragma unroll
        for (int u = 0; u < MU; ++u) {
            src[u] = sidx(li[u]);
            dst[u] = sidx(hi[u]);
        }
        typename KV::Chunk ch[MU];
        ST scv[MU];
        int32_t psv[MU];
#pragma unroll
        for (int u = 0; u < MU; ++u) {
            ch[u] = KV::fetch(s, src[u], sub);
            scv[u] = has_scores ? sc[src[u]] : ST(0);
            psv[u] = ps[src[u]];
        }
        fetch_lists(i0 + NG * MU);
#pragma unroll
        for (int u = 0; u < MU; ++u) {
            if (i0 + u * NG >= nh) continue;
            KV::put(s, dst[u], sub, ch[u]);
            if (sub == 0) {
                if (has_scores) sc[dst[u]] = scv[u];
                ps[dst[u]] = psv[u];
            }
        }
    }
}


// ------------------------------------------------------------ step tail
// Scores are compared (arg-min, radix keys) in MinT: binary16 scores widen
// exactly to fp32, the others compare as stored.
template <typename ST>
using MinT = std::conditional_t<sizeof(ST) == 2, float, ST>;

// Shared memory of the tail.
template <typename ST, int NW>
struct TailSmem {
    ST new_score;
    MinT<ST> bs[NW];
    int bp[NW], bj[NW];
    double dsum[NW];
    int isum[NW];
    ScanSmem scan;
    RadixSmem rad;
    OrderSmem<NW * 64, kCollectUnroll> ord;
};

// Everything the step does once the softmax maximum Mg and normaliser 1/L
// of every query head of the group are known (all threads call it):
//   H2O: p = 2^(s - M) / L per slot (logits in the log2 domain at
//        logit[g * lstride + j], the new token at j = n), summed over the
//        group, added to the cumulative score after the score is multiplied
//        by the decay (a moving sum; decay 1 is the exact sum), as one fused
//        multiply-add in the score's precision (fp32 for binary16 scores,
//        rounded to nearest once when stored); with one token to go, the
//        arg-min over the candidates (score ascending, position descending)
//        names the victim, which the new token replaces in place when fused.
//   bulk (e > 1, Random Attention events): radix select of the e smallest
//        keys, victims marked, holes filled when fused.
// pf_s / pf_p: score and position of slots tid + k * NT (k < PF), fetched
// early by the caller; write_new(si): every thread calls it to store the new
// token's row at slot index si (the writer picks its threads); emass0: the
// unit's evicted mass before the step.
// Definitions: "Attention Sinks and KV cache eviction" sec. 4.2 (cumulative
// score; sinks, heavy hitters and recent window) and sec. 6.2 (compressed
// score state: FP16 storage, a moving average instead of the exact sum),
// "H2O: Heavy-Hitter Oracle" (greedy eviction under budget K), "Random
// Attention" (method).  Always inlined: a call would take the address of the
// launch's argument block, which the compiler then copies to scratch memory.
template <int NT, int G, int PF, typename ST, bool PAGED, typename KV, typename WriteNew>
__device__ __attribute__((always_inline)) inline void step_tail(const StepArgs& a, const SlotMap<PAGED>& sidx,
                                 TailSmem<ST, NT / 64>& sm,
                                 int unit, int b, int h, int P, int t, int n, int e, bool inplace_new,
                                 const float* logit, int lstride, const float (&Mg)[G],
                                 const float (&invLg)[G], const ST (&pf_s)[PF], const int (&pf_p)[PF],
                                 WriteNew write_new, double emass0)
{
    constexpr int NW = NT / 64;
    const Geometry& gm = a.g;
    const State& S = a.s;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n_att = n + 1;
    const bool h2o = scored(a.sc.selector);
    ST* scp = reinterpret_cast<ST*>(S.sc);
    int32_t* psp = S.ps;

    int K = 0, HH = 0, W = 0;
    if (h2o) schedule(a.sc, t + 1, K, HH, W);
    const int lo_c = a.sc.n_sink, hi_c = t + 1 - W;  // H2O candidates: lo_c <= pos < hi_c

    // ---- phase 2 (H2O): accumulate scores; arg-min when one token goes ---
    if (h2o) {
        using MT = MinT<ST>;
        const float lam = a.sc.decay;
        MT bs = (MT)INFINITY;
        int bp = -1, bj = -1;
        // slot j: decay its score and add its weights of this step (summed over
        // the group; lg = its G logits); the new token (j == n) starts from
        // zero.  With decay 1 the fused multiply-add is the plain sum, rounded once.
        auto visit = [&](int j, ST old, int pos, const float (&lg)[G]) {
            float p = 0.f;
#pragma unroll
            for (int g = 0; g < G; ++g) p += fast_exp2(lg[g] - Mg[g]) * invLg[g];
            ST nw;
            if constexpr (sizeof(ST) == 8) nw = fma((double)lam, old, (double)p);
            else nw = (ST)fmaf(lam, (float)old, p);
            if (j < n) {
                scp[sidx(j)] = nw;
            } else {
                sm.new_score = nw;
                if (!inplace_new) {
                    const size_t si = sidx(n);
                    scp[si] = nw;
                    psp[si] = t;
                }
            }
            if (e == 1 && pos >= lo_c && pos < hi_c) take_better(bs, bp, bj, (MT)nw, pos, j);
        };
        auto logits_of = [&](int j, float (&lg)[G]) {
#pragma unroll
            for (int g = 0; g < G; ++g) lg[g] = logit[(size_t)g * lstride + j];
        };
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            const int j = tid + k * NT;
            if (j < n_att) {
                float lg[G];
                logits_of(j, lg);
                visit(j, j < n ? pf_s[k] : (ST)0, j < n ? pf_p[k] : t, lg);
            }
        }
        // the rest four slots at a time (score, position and logits of each
        // fetched before any is used: long units would otherwise wait on one
        // dependent load per slot)
        struct Slot {
            ST s;
            int p;
            float lg[G];
        };
        for_slots_batched<NT, 4>(
            PF * NT, n_att,
            [&](int j) {
                // slot n is the append slot, which has no page yet when the new
                // token is to fill a hole in place: slot 0 stands in (unused)
                const size_t si = sidx(j < n ? j : 0);
                Slot r;
                r.s = scp[si];
                r.p = psp[si];
                logits_of(j, r.lg);
                return r;
            },
            [&](int j, const Slot& r) {
                if (j < n) visit(j, r.s, r.p, r.lg);
                else visit(j, (ST)0, t, r.lg);
            });
        if (e == 1) {
            wave_argmin(bs, bp, bj);
            if (lane == 0) {
                sm.bs[w] = bs;
                sm.bp[w] = bp;
                sm.bj[w] = bj;
            }
            lds_barrier();
            // lanes 0..NW-1 of every wave take one wave's best; three DPP
            // stages within 8 lanes leave the workgroup's best in lane 0
            static_assert(NW <= 8, "cross-wave arg-min covers up to 8 waves");
            MT vs = lane < NW ? sm.bs[lane] : (MT)INFINITY;
            int vp = lane < NW ? sm.bp[lane] : -1, vjj = lane < NW ? sm.bj[lane] : -1;
            argmin_step<0xB1>(vs, vp, vjj);
            argmin_step<0x4E>(vs, vp, vjj);
            argmin_step<0x141>(vs, vp, vjj);
            if constexpr (sizeof(MT) == 4) {
                vs = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(vs)));
            } else {
                const long long u = __double_as_longlong(vs);
                const int lo = __builtin_amdgcn_readfirstlane((int)(u & 0xffffffffll));
                const int hi = __builtin_amdgcn_readfirstlane((int)(u >> 32));
                vs = __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
            }
            const int vj = __builtin_amdgcn_readfirstlane(vjj);
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
                    write_new(sidx(vj));
                    if (owner) {
                        scp[sidx(vj)] = sm.new_score;
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
    // candidates' keys are built from data fetched UNR slots at a time
    constexpr int UNR = 8;
    if (h2o) {
        // 64- or 96-bit keys: the score's order-preserving bits, then ~position
        // (equal scores: the higher position is the smaller key, evicted first)
        struct Raw {
            int pos;
            ST score;
        };
        struct Src {
            SlotMap<PAGED> sidx;
            const int32_t* psp;
            const ST* scp;
            int lo_c, hi_c;
            __device__ Raw fetch(int j) const
            {
                const size_t si = sidx(j);
                return {psp[si], scp[si]};
            }
            __device__ bool key(const Raw& r, unsigned (&wk)[3]) const
            {
                if (r.pos < lo_c || r.pos >= hi_c) return false;
                if constexpr (sizeof(ST) <= 4) {
                    wk[2] = 0;
                    wk[1] = ord32((float)r.score);
                } else {
                    const unsigned long long u = ord64((double)r.score);
                    wk[2] = (unsigned)(u >> 32);
                    wk[1] = (unsigned)u;
                }
                wk[0] = ~(unsigned)r.pos;
                return true;
            }
        };
        const Src src{sidx, psp, scp, lo_c, hi_c};
        d0 = sizeof(ST) <= 4 ? 4 : 0;
        radix_select_batched<NT, UNR>(src, n_att, e, d0, sm.rad);
        for_slots_batched<NT, UNR>(0, n_att, [&](int j) { return src.fetch(j); }, [&](int j, const Raw& r) {
            unsigned wk[3];
            if (src.key(r, wk) && key_le(wk, sm.rad)) {
                vmass += (double)r.score;
                psp[sidx(j)] = -1;
                ++nv;
            }
        });
    } else {
        // Random Attention: word 0 of Philox4x64-10 at counter (b, h, t, position)
        struct Src {
            SlotMap<PAGED> sidx;
            const int32_t* psp;
            int P, b, h, t;
            unsigned long long k0;
            __device__ int fetch(int j) const { return psp[sidx(j)]; }
            __device__ bool key(int pos, unsigned (&wk)[3]) const
            {
                if (pos < P) return false;
                const unsigned long long x =
                    philox_word0((unsigned long long)b, (unsigned long long)h, (unsigned long long)t,
                                 (unsigned long long)pos, k0, 0ull);
                wk[2] = (unsigned)(x >> 32);
                wk[1] = (unsigned)x;
                wk[0] = ~(unsigned)pos;
                return true;
            }
        };
        const Src src{sidx, psp, P, b, h, t, a.sc.seed};
        radix_select_batched<NT, UNR>(src, n_att, e, 0, sm.rad);
        for_slots_batched<NT, UNR>(0, n_att, [&](int j) { return src.fetch(j); }, [&](int j, int pos) {
            unsigned wk[3];
            if (src.key(pos, wk) && key_le(wk, sm.rad)) {
                psp[sidx(j)] = -1;
                ++nv;
            }
        });
    }
    const int nv_all = block_sum_i32<NT>(nv, sm.isum);
    const double vm = block_sum_f64<NT>(vmass, sm.dsum);
    if (tid == 0) {
        if (nv_all != e) atomicOr(S.err, kErrSelectCount);
        if (h2o) S.emass[unit] = emass0 + vm;
    }
    if (a.fused) {
        __syncthreads();
        const int n2 = n_att - e;
        // holes of [0, h_end) take the live slots of [l0, l1) and [l2, l3)
        int h_end = n2, l0 = n2, l1 = n_att, l2 = n_att;
        WindowRemap r;
        if (PAGED && a.remap && window_remap(a.sc, t, n_att, e, r)) {  // the host relinks the pages
            h_end = r.front;
            l0 = r.front;
            l1 = r.src;
            l2 = r.src + r.m;
        }
        fill_holes<NT, ST, KV>(S, sidx, unit, gm.cap, h_end, l0, l1, l2, n_att, h2o, sm.ord);
        if (tid == 0) S.cnt[unit] = n2;
    } else if (tid == 0) {
        S.vinfo[2 * unit] = e;
        S.vinfo[2 * unit + 1] = -1;
        S.cnt[unit] = n_att;
    }
}

}  // namespace
}  // namespace h2o
