// Matrix-core decode step for GQA groups of 4 or 8 query heads per KV head
// (bf16 K/V rows of 128, contiguous slots in the KvTiles layout).
//
// With G query heads sharing one KV head, q.K over a tile of slots is a
// (slots x 128) by (128 x G) product and P.V a (128 x slots) by (slots x G)
// one, so both run on v_mfma_f32_16x16x32_bf16.  q and the softmax weights p
// are fp32: each value x is split into bf16 parts hi = bf16(x) and
// lo = bf16(x - hi) (x = hi + lo to about 2^-16 relative), hi of head g in B
// column g and lo in column g + 8.  K and V enter exactly (bf16), products
// are exact and the sums fp32, so the logits and the output keep about
// 16 significant bits of q and p.
//
// One workgroup of 8 waves owns one (sequence, KV head) unit.  Wave w takes
// the 32-slot tiles w, w + 8, w + 16, ... (handing tiles out from an LDS
// counter instead balances the waves but streams ~5 % slower).  Per tile:
//   S  = K_tile (32 x 128) . [q_hi | q_lo]^T     two 16-slot C blocks, 4 k-steps each
//   s  = S[:, g] + S[:, g + 8]                   DPP row rotate by 8
//   online softmax per head: running max / sum / output, the tile maximum
//        across the wave's four lane groups by permlane swaps
//   O += V_tile^T (128 x 32) . [p_hi | p_lo]     8 d-blocks, 1 k-step each
// The logit tile's C layout (lane l: slots 4(l/16)+r and 16+4(l/16)+r of
// column l%16) already is the layout of the P^T B operand, and the V tiles
// list each lane group's slots in that order, so p never moves between
// lanes.  K and V tiles are read with wave-wide 16-byte loads of 1 KB each,
// one tile in flight per wave.  The new token (slot n, from k_new / v_new)
// seeds the running state of wave 0; every wave knows its logit, so the wave
// that stores the tile holding slot n stores that logit there.  The waves
// then merge through LDS and the shared tail (h2o_device.h) accumulates
// scores, selects and compacts.
//
// Definitions followed: "Attention Sinks and KV cache eviction" sec. 3.1
// (softmax attention of the new query over the kept keys and values),
// sec. 1.1 (grouped-query attention: a group of query heads shares one KV
// head) and sec. 4.2 (cumulative score summed over the decode steps).
#include "h2o_device.h"

namespace h2o {
namespace {

constexpr int kMNT = 512;  // threads per unit (8 waves, 2 per SIMD)
constexpr int kMNW = kMNT / 64;
constexpr int kMPF = 3;    // slots per thread whose score and position are fetched up front
constexpr int kTile = 32;  // slots per tile

__device__ inline float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

struct MTile {
    uint4 k[8];  // [half * 4 + kb]: slots 16 half .. +16, d 32 kb .. +32
    uint4 v[8];  // [db]: d 16 db .. +16, the lane group's 8 slots
};

template <int G, typename ST, bool LLDS>
__global__ void __launch_bounds__(kMNT) mfma_step_kernel(const StepArgs a)
{
    static_assert(G == 4 || G == 8, "the matrix-core step takes GQA groups of 4 or 8");
    constexpr int NT = kMNT, NW = kMNW, PF = kMPF, D = 128;
    constexpr float kMaxFloor = -1e30f;

    extern __shared__ __align__(16) unsigned char dsm[];
    __shared__ float red_m[NW][G], red_l[NW][G];
    __shared__ __align__(16) float red_o[NW][G][D];
    __shared__ TailSmem<ST, NW> tsm;
    // the group's q rows and the new token's K and V rows, fetched once per
    // workgroup (every wave needs all of them, each lane a different part)
    __shared__ __align__(16) float q_s[G * D];
    __shared__ __align__(16) uint4 kvn_s[2 * kRowVecs];

    const Geometry& gm = a.g;
    const State& S = a.s;
    // the head is the fast index (XCDs round-robin), sequences longest first
    const int sq = (int)blockIdx.x / gm.Hkv, h = (int)blockIdx.x - sq * gm.Hkv;
    // this row's sequence, retained count and prompt length: scalar loads of
    // the arguments (without them in the arguments, from the state; those
    // reads are volatile so that the compiler cannot merge the two paths into
    // vector loads through a selected pointer)
    SeqArg sa;
    if (a.seq_in_args) {
        sa = a.seq[sq];
    } else {
        sa.b = sq;
        sa.n = *reinterpret_cast<const volatile int32_t*>(S.cnt + (size_t)sq * gm.Hkv + h);
        sa.p = *reinterpret_cast<const volatile int32_t*>(S.t0 + sq);
        sa.newpage = -1;
    }
    const int b = __builtin_amdgcn_readfirstlane(sa.b);
    const int unit = b * gm.Hkv + h;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (scalar)
    const int lc = lane & 15, lg = lane >> 4;  // C column, lane group
    const int head = lc & 7;                   // query head of column lc (a real head when < G)
    const bool lo_col = lc >= 8;

    // uniform over the workgroup: readfirstlane keeps them (and the buffer
    // descriptors built from them) in scalar registers
    const int P = __builtin_amdgcn_readfirstlane(sa.p);
    const int t = P + a.step;
    const int n = __builtin_amdgcn_readfirstlane(sa.n);
    const bool h2o = scored(a.sc.selector);
    const int e = evict_count(a.sc, t, P, n + 1);
    const bool inplace_new = a.fused && h2o && e == 1;

    float* logit = LLDS ? reinterpret_cast<float*>(dsm) : S.lscr + (size_t)unit * G * gm.cap;
    const int lstride = LLDS ? a.lds_n : gm.cap;
    SlotMap<false> sidx;
    sidx.base = (size_t)unit * gm.cap;
    sidx.h = h;
    sidx.Hkv = gm.Hkv;
    sidx.bt = nullptr;
    ST* scp = reinterpret_cast<ST*>(S.sc);
    int32_t* psp = S.ps;

    // ---- loads, issued in the order their data is needed ------------------
    // q and the new token's rows: one 16-byte vector per thread (threads past
    // them read out of range: zero, no memory access), staged in LDS below
    constexpr int QV = G * D / 4;  // 16-byte vectors of the group's q rows
    const auto rq = make_rsrc(a.q + ((size_t)b * gm.Hq + (size_t)h * G) * D, (unsigned)QV * 16u);
    const auto rkn = make_rsrc(reinterpret_cast<const uint4*>(a.kn) + (size_t)unit * kRowVecs, kRowBytes);
    const auto rvn = make_rsrc(reinterpret_cast<const uint4*>(a.vn) + (size_t)unit * kRowVecs, kRowBytes);
    const uint4 qv = buf_load16(rq, (unsigned)tid * 16u);
    const uint4 knv = buf_load16(rkn, min((unsigned)(tid - QV), (unsigned)kRowVecs) * 16u);
    const uint4 vnv = buf_load16(rvn, min((unsigned)(tid - QV - kRowVecs), (unsigned)kRowVecs) * 16u);
    // the unit's evicted mass, for its update at the end: a vector load (a
    // scalar one would hold up the barrier below for a memory round trip)
    const double emass0 = load_f64(S.emass + unit);
    // every wave's loads above enter the memory queues before any tile load
    // of the workgroup (the older wave of a SIMD would otherwise issue all of
    // its tile loads first); the barrier waits for none of that data
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // K / V tiles through raw buffer loads over the unit's first ntiles
    // tiles: a tile index past them reads zeros without a memory access
    const int ntiles = (n + kTile - 1) / kTile;
    const size_t ub = (size_t)unit * gm.cap * kRowBytes;
    const unsigned tile_bytes = (unsigned)kTile * kRowBytes;
    const auto rk = make_rsrc(reinterpret_cast<const char*>(S.kc) + ub, (unsigned)ntiles * tile_bytes);
    const auto rv = make_rsrc(reinterpret_cast<const char*>(S.vc) + ub, (unsigned)ntiles * tile_bytes);
    auto load_tile = [&](int tl, MTile& T) {
        const unsigned base = (unsigned)tl * tile_bytes + (unsigned)lane * 16u;
#pragma unroll
        for (int i = 0; i < 8; ++i) T.k[i] = buf_load16(rk, base + (unsigned)i * 1024u);
#pragma unroll
        for (int i = 0; i < 8; ++i) T.v[i] = buf_load16(rv, base + (unsigned)i * 1024u);
    };
    MTile T;
    load_tile(w, T);
    __builtin_amdgcn_sched_barrier(0);


    // q and the new token's rows into LDS (their loads, issued before the
    // tiles', retire first), then every lane reads its parts:
    // q of column lc's head at d = 32 kb + 8 lg + i, the new token's K as an A
    // operand whose 16 rows are all that token, its V at d = 16 db + 4 lg + r
    if (tid < QV) reinterpret_cast<uint4*>(q_s)[tid] = qv;
    if ((unsigned)(tid - QV) < (unsigned)kRowVecs) kvn_s[tid - QV] = knv;
    if ((unsigned)(tid - QV - kRowVecs) < (unsigned)kRowVecs) kvn_s[tid - QV] = vnv;
    lds_barrier();
    const int qh = head < G ? head : 0;
    const float4* qs4 = reinterpret_cast<const float4*>(q_s + qh * D);
    uint4 kn4[4];
    uint2 vn8[8];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) kn4[kb] = kvn_s[4 * kb + lg];
#pragma unroll
    for (int db = 0; db < 8; ++db) vn8[db] = reinterpret_cast<const uint2*>(kvn_s + kRowVecs)[4 * db + lg];

    // B operand of q.K: column lc = hi (lc < 8) or lo part of head lc & 7
    bf16x8 qop[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const float4 q0 = qs4[8 * kb + 2 * lg], q1 = qs4[8 * kb + 2 * lg + 1];
        const float x[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            qop[kb][i] = head < G ? split_part(x[i] * a.qscale, lo_col) : (__bf16)0.0f;
    }

    // the new token's logit (every row of the product is that token)
    f32x4 cn = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) cn = mma(as_bf16x8(kn4[kb]), qop[kb], cn);
    const float s_new = cn[0] + dpp<0x128>(cn[0]);  // row_ror:8 adds the lo column

    // running state; wave 0 starts from the new token alone: m = its logit,
    // weight 1 (counted once, in lane group 0), O = its V row in the hi columns
    const bool own_new = w == 0;
    float m = own_new ? s_new : kMaxFloor;
    float l = (own_new && lg == 0) ? 1.f : 0.f;
    f32x4 O[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        const bool take = own_new && !lo_col;
        O[db][0] = take ? bf16_lo(vn8[db].x) : 0.f;
        O[db][1] = take ? bf16_hi(vn8[db].x) : 0.f;
        O[db][2] = take ? bf16_lo(vn8[db].y) : 0.f;
        O[db][3] = take ? bf16_hi(vn8[db].y) : 0.f;
    }

    auto process = [&](int tl, MTile& T) {
        f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) c0 = mma(as_bf16x8(T.k[kb]), qop[kb], c0);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) c1 = mma(as_bf16x8(T.k[4 + kb]), qop[kb], c1);
        float s[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s[r] = c0[r] + dpp<0x128>(c0[r]);
            s[4 + r] = c1[r] + dpp<0x128>(c1[r]);
        }
        // slots at or past n take no weight (their K / V may be stale); only
        // the unit's last tile holds such slots (a wave-uniform test)
        const int j0 = tl * kTile + 4 * lg;
        const bool last_tile = (tl + 1) * kTile > n;
        if (last_tile) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (j0 + r >= n) s[r] = -INFINITY;
                if (j0 + 16 + r >= n) s[4 + r] = -INFINITY;
            }
        }
        if (h2o && lc < G) {  // slot n of this tile (if any) takes the new token's logit
            float4* lp = reinterpret_cast<float4*>(logit + (size_t)lc * lstride + j0);
            if (last_tile) {
                lp[0] = make_float4(j0 == n ? s_new : s[0], j0 + 1 == n ? s_new : s[1],
                                    j0 + 2 == n ? s_new : s[2], j0 + 3 == n ? s_new : s[3]);
                lp[4] = make_float4(j0 + 16 == n ? s_new : s[4], j0 + 17 == n ? s_new : s[5],
                                    j0 + 18 == n ? s_new : s[6], j0 + 19 == n ? s_new : s[7]);
            } else {
                lp[0] = make_float4(s[0], s[1], s[2], s[3]);
                lp[4] = make_float4(s[4], s[5], s[6], s[7]);
            }
        }
        float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                         fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
        {
            const Pair x = xrow16(__float_as_uint(mx));
            mx = fmaxf(__uint_as_float(x.a), __uint_as_float(x.b));
        }
        {
            const Pair x = xrow32(__float_as_uint(mx));
            mx = fmaxf(__uint_as_float(x.a), __uint_as_float(x.b));
        }
        const float mn = fmaxf(m, mx);
        const float al = fast_exp2(m - mn);
        m = mn;
        l *= al;
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) O[db][r] *= al;
        bf16x8 pb;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float p = fast_exp2(s[k] - mn);  // 2^-inf = 0 for masked slots
            l += p;
            pb[k] = split_part(p, lo_col);
        }
        // the last, partial tile: zero V of the slots past n so stale values
        // cannot reach the sum through 0 * inf
        if (tl == ntiles - 1 && (n % kTile) != 0) {
            const int lim = n - tl * kTile;
            unsigned mk[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int s0 = (2 * k < 4 ? 4 * lg + 2 * k : 16 + 4 * lg + 2 * k - 4);
                mk[k] = (s0 < lim ? 0xffffu : 0u) | (s0 + 1 < lim ? 0xffff0000u : 0u);
            }
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                T.v[db].x &= mk[0];
                T.v[db].y &= mk[1];
                T.v[db].z &= mk[2];
                T.v[db].w &= mk[3];
            }
        }
#pragma unroll
        for (int db = 0; db < 8; ++db) O[db] = mma(as_bf16x8(T.v[db]), pb, O[db]);
    };

    // one tile in flight per wave (eight per workgroup): the registers of the
    // tile just consumed take the wave's next; the last tile is peeled so the
    // loop holds no conditional load.  Two per wave streamed slower: the
    // CU's memory queue only grows, and the first tiles arrive later.
    const int cnt = w < ntiles ? (ntiles - 1 - w) / NW + 1 : 0;  // this wave's tiles
    int i = 0;
    for (; i + 1 < cnt; ++i) {
        process(w + NW * i, T);
        __builtin_amdgcn_sched_barrier(0);
        load_tile(w + NW * (i + 1), T);
        __builtin_amdgcn_sched_barrier(0);
    }
    // scores and positions of this thread's first PF phase-2 slots, requested
    // after the last tile (the CU's memory queue is served in order: earlier,
    // they would delay every later tile)
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
    if (i < cnt) process(w + NW * i, T);
    // slot n outside every tile (n a multiple of 32): its logit slot is free
    if (h2o && own_new && (n % kTile) == 0 && lc < G && lg == 0) logit[(size_t)lc * lstride + n] = s_new;

    // ---- merge: lane groups (sum of l), hi + lo columns, then waves -------
    {
        const Pair x = xrow16(__float_as_uint(l));
        l = __uint_as_float(x.a) + __uint_as_float(x.b);
    }
    {
        const Pair x = xrow32(__float_as_uint(l));
        l = __uint_as_float(x.a) + __uint_as_float(x.b);
    }
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) O[db][r] += dpp<0x128>(O[db][r]);
    if (lc < G) {
#pragma unroll
        for (int db = 0; db < 8; ++db)
            *reinterpret_cast<float4*>(&red_o[w][lc][16 * db + 4 * lg]) =
                make_float4(O[db][0], O[db][1], O[db][2], O[db][3]);
        if (lg == 0) {
            red_m[w][lc] = m;
            red_l[w][lc] = l;
        }
    }
    // logits kept in global scratch (very long units) need the full fence
    if constexpr (LLDS) lds_barrier(); else __syncthreads();
    // one lane per (wave, head) pair (lane i: wave (i % NP) / G, head i % G)
    // reduces over the waves by butterflies; M_g, 1/L_g and the per-wave
    // factors 2^(m - M_g) are then read from those lanes into scalars
    constexpr int NP = NW * G;  // 32 or 64 pairs
    const int pi = lane % NP;
    const float mi = red_m[pi / G][pi % G], li = red_l[pi / G][pi % G];
    // the butterflies over one head's lanes (partners at xor G, 2G, .. < NP):
    // row rotations by 4 (G = 4) and 8 within 16 lanes, then the swaps of
    // 16-lane rows and (G = 8) of 32-lane halves -- register moves, no LDS
    auto head_reduce = [](float v, auto op) {
        if constexpr (G == 4) v = op(v, dpp<0x124>(v));  // row_ror:4
        v = op(v, dpp<0x128>(v));                         // row_ror:8
        {
            const Pair x = xrow16(__float_as_uint(v));
            v = op(__uint_as_float(x.a), __uint_as_float(x.b));
        }
        if constexpr (G == 8) {
            const Pair x = xrow32(__float_as_uint(v));
            v = op(__uint_as_float(x.a), __uint_as_float(x.b));
        }
        return v;
    };
    const float Mx = head_reduce(mi, [](float x, float y) { return fmaxf(x, y); });
    const float fi = fast_exp2(mi - Mx);
    const float Lx = head_reduce(li * fi, [](float x, float y) { return x + y; });
    const float il_x = 1.0f / Lx;
    auto bcast = [](float v, int src) {
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
    };
    float Mg[G], invLg[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        Mg[g] = bcast(Mx, g);
        invLg[g] = bcast(il_x, g);
    }
    // output: NW / G waves per head, each a contiguous part of the row
    {
        constexpr int WPH = NW / G, DPW = D / WPH, EPT = DPW / 64;
        const int g = w / WPH, d0 = (w % WPH) * DPW + lane * EPT;
        float acc[EPT];
#pragma unroll
        for (int k = 0; k < EPT; ++k) acc[k] = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float f = bcast(fi, ww * G + g);
#pragma unroll
            for (int k = 0; k < EPT; ++k) acc[k] += red_o[ww][g][d0 + k] * f;
        }
        const float il = bcast(il_x, g);
        float* op = a.out + ((size_t)b * gm.Hq + (size_t)h * G + g) * D + d0;
#pragma unroll
        for (int k = 0; k < EPT; ++k) op[k] = acc[k] * il;
    }
    // the new token's rows go to slot n unless they fill a victim's hole later
    auto write_new = [&](size_t si) {  // the new token's row into slot index si
        if (tid < 16) KvTiles::store(S.kc, S.vc, si, tid, kvn_s[tid], kvn_s[kRowVecs + tid]);
    };
    if (!inplace_new) write_new(sidx(n));

    step_tail<NT, G, PF, ST, false, KvTiles>(a, sidx, tsm, unit, b, h, P, t, n, e, inplace_new, logit,
                                             lstride, Mg, invLg, pf_s, pf_p, write_new, emass0);
}

template <int G, typename ST, bool LLDS>
hipError_t launch_mfma_t(const StepArgs& a, size_t dyn, hipStream_t st)
{
    auto k = mfma_step_kernel<G, ST, LLDS>;
    static DynLdsLimit lim;
    const hipError_t err = lim.allow((const void*)k, dyn);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k, dim3(a.g.B * a.g.Hkv), dim3(kMNT), dyn, st, a);
    return hipGetLastError();
}

template <int G, typename ST>
hipError_t launch_mfma_g(const StepArgs& a, bool llds, size_t dyn, hipStream_t st)
{
    return llds ? launch_mfma_t<G, ST, true>(a, dyn, st) : launch_mfma_t<G, ST, false>(a, 0, st);
}

template <typename ST>
hipError_t launch_mfma_s(const StepArgs& a, bool llds, size_t dyn, hipStream_t st)
{
    return a.g.G == 4 ? launch_mfma_g<4, ST>(a, llds, dyn, st) : launch_mfma_g<8, ST>(a, llds, dyn, st);
}

}  // namespace

hipError_t launch_step_mfma(const StepArgs& a0, int max_n_att, hipStream_t st)
{
    const Geometry& g = a0.g;
    if (!g.kv_tiles || !g.kv_bf16 || g.D != 128 || g.paged || (g.G != 4 && g.G != 8) ||
        (g.cap % kTile) != 0)
        return hipErrorInvalidValue;
    StepArgs a = a0;
    a.lds_n = (max_n_att + kTile - 1) / kTile * kTile;  // whole tiles of logits
    bool llds = true;
    size_t dyn = 0;
    if (a.sc.selector == 0) {  // H2O keeps the logits for the score pass
        llds = (size_t)g.G * a.lds_n * 4 <= (size_t)kLogitLdsBytes;
        if (llds) dyn = (size_t)g.G * a.lds_n * 4;
        else if (a.s.lscr == nullptr) return hipErrorInvalidValue;
    }
    if (g.score_f64) return launch_mfma_s<double>(a, llds, dyn, st);
    if (g.score_f16) return launch_mfma_s<_Float16>(a, llds, dyn, st);
    return launch_mfma_s<float>(a, llds, dyn, st);
}

}  // namespace h2o
