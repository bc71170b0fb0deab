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
#include "h2o_device.h"

namespace h2o {
namespace {

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
    __shared__ TailSmem<ST, NW> tsm;

    const Geometry& gm = a.g;
    const State& S = a.s;
    // workgroups reach the XCDs round-robin: with the head as the fast index
    // every XCD gets the same heads of every sequence, and within an XCD the
    // longest sequences are dispatched first
    const int sq = (int)blockIdx.x / gm.Hkv, h = (int)blockIdx.x - sq * gm.Hkv;
    const int b = a.seq_in_args ? (int)a.seq_order[sq] : sq;
    const int unit = b * gm.Hkv + h;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, sub = tid & 15, grp = tid >> 4;

    // the host knows every sequence's prompt length and retained count: taking
    // them from the arguments saves a dependent memory round trip at the start
    // uniform over the workgroup: readfirstlane keeps them (and the buffer
    // descriptors built from them) in scalar registers
    const int P = __builtin_amdgcn_readfirstlane(a.seq_in_args ? a.seq_p[b] : S.t0[b]);
    const int t = P + a.step;
    const int n = __builtin_amdgcn_readfirstlane(a.seq_in_args ? a.seq_n[b] : S.cnt[unit]);
    const int n_att = n + 1;
    const bool h2o = scored(a.sc.selector);
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
            // the append page: from the host, or (pop_stack) the free-stack entry it names
            const int np = a.newpage[b] < 0 ? -1 : (a.pop_stack ? S.fstack[a.newpage[b]] : a.newpage[b]);
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
    using Vec = typename Row::Vec;
    using KVL = std::conditional_t<Row::SCALED, KvRows8, KvRows>;  // stored row layout
    constexpr unsigned RB = Row::SCALED ? kRowBytesI8 : kRowBytes;  // stored row bytes
    constexpr unsigned VBY = sizeof(Vec);                           // bytes of a row per lane
    const Vec* kc = reinterpret_cast<const Vec*>(S.kc);
    const Vec* vc = reinterpret_cast<const Vec*>(S.vc);
    // evicted mass of the unit, read now so its update at the end is no round trip
    const double emass0 = S.emass[unit];
    __builtin_amdgcn_sched_barrier(0);  // keep q and the new token ahead of the K/V stream
    // the new token's row as stored; int8 rows are quantised here, and the
    // cache then holds -- and this step attends over -- exactly that row
    Vec knv, vnv;
    float kns = 1.f, vns = 1.f;
    if constexpr (Row::SCALED) {
        float xk[8], xv[8];
        RowBf16::unpack(knr, xk);
        RowBf16::unpack(vnr, xv);
        quantize_row8(xk, knv, kns);
        quantize_row8(xv, vnv, vns);
    } else {
        knv = knr;
        vnv = vnr;
    }
    auto write_new = [&](size_t si) {  // the new token's row into slot index si
        if (tid < 16) {
            if constexpr (Row::SCALED) {
                reinterpret_cast<uint2*>(S.kc)[si * kRowVecs + sub] = knv;
                reinterpret_cast<uint2*>(S.vc)[si * kRowVecs + sub] = vnv;
                if (sub == 0) {
                    S.kss[si] = kns;
                    S.vss[si] = vns;
                }
            } else {
                KvRows::store(S.kc, S.vc, si, sub, knr, vnr);
            }
        }
    };

    // Rows j >= n are masked out by their logit; the new token (j == n) is
    // folded in after the loop.  Every load is unconditional (a conditional
    // load would make the compiler's wait counts conservative at the join and
    // serialise the pipeline).  Contiguous layout: raw buffer loads over the
    // unit's n rows, so rows past them read as zero without a memory access.
    // Paged layout: rows past n read slot 0 (a cache hit).
    __amdgpu_buffer_rsrc_t rk, rv, rks, rvs;
    if constexpr (!PAGED) {
        const size_t ub = sidx.base * RB;
        rk = make_rsrc(reinterpret_cast<const char*>(S.kc) + ub, (unsigned)n * RB);
        rv = make_rsrc(reinterpret_cast<const char*>(S.vc) + ub, (unsigned)n * RB);
        if constexpr (Row::SCALED) {
            rks = make_rsrc(S.kss + sidx.base, (unsigned)n * 4u);
            rvs = make_rsrc(S.vss + sidx.base, (unsigned)n * 4u);
        }
    }
    auto ld = [](__amdgpu_buffer_rsrc_t r, unsigned off) -> Vec {
        if constexpr (sizeof(Vec) == 16) return buf_load16(r, off);
        else return buf_load8(r, off);
    };
    // rows (and, for int8 rows, their scales) of one batch
    auto load_batch = [&](int base, Vec (&kr)[U], Vec (&vr)[U], float (&ks)[U], float (&vs)[U]) {
        if constexpr (!PAGED) {
            const unsigned off0 = (unsigned)(base + grp) * RB + (unsigned)sub * VBY;
#pragma unroll
            for (int u = 0; u < U; ++u) kr[u] = ld(rk, off0 + (unsigned)(u * NGRP) * RB);
#pragma unroll
            for (int u = 0; u < U; ++u) vr[u] = ld(rv, off0 + (unsigned)(u * NGRP) * RB);
            if constexpr (Row::SCALED) {
                const unsigned so = (unsigned)(base + grp) * 4u;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    ks[u] = buf_load4f(rks, so + (unsigned)(u * NGRP * 4));
                    vs[u] = buf_load4f(rvs, so + (unsigned)(u * NGRP * 4));
                }
            }
        } else {
            size_t r[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = base + grp + NGRP * u;
                r[u] = sidx(j < n ? j : 0);
                kr[u] = stream_load(kc + r[u] * kRowVecs + sub);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) vr[u] = stream_load(vc + r[u] * kRowVecs + sub);
            if constexpr (Row::SCALED) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    ks[u] = stream_load(S.kss + r[u]);
                    vs[u] = stream_load(S.vss + r[u]);
                }
            }
        }
    };
    Vec ka[U], va[U], kb[U], vb[U];
    float ksa[U], vsa[U], ksb[U], vsb[U];
    load_batch(0, ka, va, ksa, vsa);
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
    // take no weight; vs: the V rows' scales (int8 rows)
    auto accumulate = [&](float (&s)[U][G], const Vec (&vr)[U], const float (&vs)[U], int nr) {
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
                const float pv = Row::SCALED ? p * vs[u] : p;
#pragma unroll
                for (int i = 0; i < EPL; ++i) o[g][i] = fmaf(pv, vx[i], o[g][i]);
            }
        }
    };
    auto logits = [&](const Vec (&kr)[U], const float (&ks)[U], float (&s)[U][G]) {
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
            for (int u = 0; u < U; ++u) s[u][g] = Row::SCALED ? acc[u] * ks[u] : acc[u];
        }
    };
    auto process = [&](int base, const Vec (&kr)[U], const Vec (&vr)[U], const float (&ks)[U],
                       const float (&vs)[U]) {
        float s[U][G];
        logits(kr, ks, s);
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
        accumulate(s, vr, vs, U);
    };
    // the new token (position t, slot n) is lane group 0's first row; this
    // runs while the first K/V batch is still in flight
    if (grp == 0) {
        Vec kn1[U], vn1[U];
        float ks1[U], vs1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            kn1[u] = knv;
            vn1[u] = vnv;
            ks1[u] = kns;
            vs1[u] = vns;
        }
        float s1[U][G];
        logits(kn1, ks1, s1);
        if (h2o) {
#pragma unroll
            for (int g = 0; g < G; ++g)
                if (sub == g) logit[(size_t)g * lstride + n] = s1[0][g];
        }
        accumulate(s1, vn1, vs1, 1);
    }
    // Batch b+1 is requested before batch b is consumed.  Two register sets
    // alternate (no copies, which would wait for the loads in flight) and the
    // tail is peeled so that the loop body holds no conditional load.
    constexpr int BR = NGRP * U;  // rows per batch
    const int nbatch = (n_att + BR - 1) / BR;
    int bi = 0;
    for (; bi + 2 < nbatch; bi += 2) {
        load_batch((bi + 1) * BR, kb, vb, ksb, vsb);
        process(bi * BR, ka, va, ksa, vsa);
        load_batch((bi + 2) * BR, ka, va, ksa, vsa);
        process((bi + 1) * BR, kb, vb, ksb, vsb);
    }
    if (bi + 1 < nbatch) {
        load_batch((bi + 1) * BR, kb, vb, ksb, vsb);
        process(bi * BR, ka, va, ksa, vsa);
        process((bi + 1) * BR, kb, vb, ksb, vsb);
    } else {
        process(bi * BR, ka, va, ksa, vsa);
    }
    // the new token's row goes to slot n unless it fills a victim's hole later
    if (!inplace_new) write_new(sidx(n));

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
    // the output: one element per thread, the waves' partial sums rescaled to
    // the common maximum (consecutive threads read consecutive LDS words)
    for (int idx = tid; idx < G * DR; idx += NT) {
        const int g = idx / DR, d = idx - g * DR;
        float acc = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) acc += red_o[ww][g][d] * fast_exp2(red_m[ww][g] - Mg[g]);
        a.out[((size_t)b * gm.Hq + (size_t)h * G + g) * DR + d] = acc * invLg[g];
    }

    step_tail<NT, G, PF, ST, PAGED, KVL>(a, sidx, tsm, unit, b, h, P, t, n, e, inplace_new, logit, lstride,
                                         Mg, invLg, pf_s, pf_p, write_new, emass0);
}

// ---------------------------------------------------------- compact kernel
constexpr int kCompactNT = 256;

template <typename ST, bool PAGED, typename KV>
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
            if (threadIdx.x < 16) KV::copy(S, src, dst, sub);
            if (threadIdx.x == 0) {
                if (has_scores) ((ST*)S.sc)[dst] = ((ST*)S.sc)[src];
                S.ps[dst] = S.ps[src];
            }
        }
    } else {
        fill_holes<kCompactNT, ST, KV>(S, sidx, unit, gm.cap, n_att, e, has_scores, s_scan);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        S.cnt[unit] = n_att - e;
        S.vinfo[2 * unit] = 0;
        S.vinfo[2 * unit + 1] = -1;
    }
}

// ------------------------------------------------------------- prompt load
template <typename ST, bool PAGED, typename KV>
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
    const uint4 kin = reinterpret_cast<const uint4*>(a.pk)[src];
    const uint4 vin = reinterpret_cast<const uint4*>(a.pv)[src];
    if constexpr (std::is_same<KV, KvRows8>::value) {
        // the 16 threads of a row are the 16 lanes of a DPP row (idx % 16 == c)
        float xk[8], xv[8];
        RowBf16::unpack(kin, xk);
        RowBf16::unpack(vin, xv);
        uint2 kq, vq;
        float ks, vs;
        quantize_row8(xk, kq, ks);
        quantize_row8(xv, vq, vs);
        reinterpret_cast<uint2*>(S.kc)[si * kRowVecs + c] = kq;
        reinterpret_cast<uint2*>(S.vc)[si * kRowVecs + c] = vq;
        if (c == 0) {
            S.kss[si] = ks;
            S.vss[si] = vs;
        }
    } else {
        KV::store(S.kc, S.vc, si, c, kin, vin);
    }
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
            if (S.sc && scored(a.selector)) s = (double)((const ST*)S.sc)[si];
        }
        a.opos[(size_t)unit * a.capo + j] = p;
        a.osc[(size_t)unit * a.capo + j] = s;
    }
}

// ------------------------------------------------------------ row gather
// Every retained slot's stored K and V rows to staging, slot order, natural
// element order whatever the layout (16 chunks per row).
template <typename KV, bool PAGED>
__global__ void __launch_bounds__(256) gather_rows_kernel(const RowGatherArgs a)
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
    const int n = min(S.cnt[unit], a.capo);
    for (int idx = threadIdx.x; idx < n * kRowVecs; idx += 256) {
        const int j = idx / kRowVecs, c = idx - j * kRowVecs;
        const size_t si = sidx(j);
        const size_t o = (size_t)unit * a.capo + j;
        if constexpr (std::is_same<KV, KvRows8>::value) {
            reinterpret_cast<uint2*>(a.ok)[o * kRowVecs + c] = reinterpret_cast<const uint2*>(S.kc)[si * kRowVecs + c];
            reinterpret_cast<uint2*>(a.ov)[o * kRowVecs + c] = reinterpret_cast<const uint2*>(S.vc)[si * kRowVecs + c];
            if (c == 0) {
                a.oks[o] = S.kss[si];
                a.ovs[o] = S.vss[si];
            }
        } else if constexpr (std::is_same<KV, KvTiles>::value) {
            reinterpret_cast<uint4*>(a.ok)[o * kRowVecs + c] = reinterpret_cast<const uint4*>(S.kc)[KvTiles::kvec(si, c)];
            const unsigned short* V = reinterpret_cast<const unsigned short*>(S.vc);
            unsigned w4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w4[e] = (unsigned)V[KvTiles::velem(si, 8 * c + 2 * e)] |
                        ((unsigned)V[KvTiles::velem(si, 8 * c + 2 * e + 1)] << 16);
            reinterpret_cast<uint4*>(a.ov)[o * kRowVecs + c] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        } else {
            reinterpret_cast<uint4*>(a.ok)[o * kRowVecs + c] = reinterpret_cast<const uint4*>(S.kc)[si * kRowVecs + c];
            reinterpret_cast<uint4*>(a.ov)[o * kRowVecs + c] = reinterpret_cast<const uint4*>(S.vc)[si * kRowVecs + c];
        }
    }
}

// --------------------------------------------------------------- dispatch
template <typename Row, int G, typename ST, bool PAGED, bool LLDS>
hipError_t launch_step_t(const StepArgs& a, size_t dyn, hipStream_t st)
{
    auto k = step_kernel<Row, G, ST, PAGED, LLDS>;
    static DynLdsLimit lim;
    const hipError_t err = lim.allow((const void*)k, dyn);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k, dim3(a.g.B * a.g.Hkv), dim3(StepTune<G>::NT), dyn, st, a);
    return hipGetLastError();
}

template <typename Row, int G, typename ST>
hipError_t dispatch_pl(const StepArgs& a, bool llds, size_t dyn, hipStream_t st)
{
    if (a.g.paged) {
        if constexpr (!std::is_same<Row, RowF32>::value) {  // pages hold bf16 or int8 rows of 128
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
    if (a.g.kv_tiles) return launch_step_mfma(a, max_n_att, st);
    const bool llds = (size_t)a.g.G * (size_t)max_n_att * 4 <= (size_t)kLogitLdsBytes;
    size_t dyn = 0;
    if (llds) dyn += (size_t)a.g.G * (size_t)a.lds_n * 4;
    if (a.g.paged) dyn += (size_t)a.npg_lds * 4;
    dyn = (dyn + 15) & ~(size_t)15;
    if (!llds && a.s.lscr == nullptr) return hipErrorInvalidValue;
    if (a.g.kv_i8) {
        return a.g.score_f64 ? dispatch_g<RowI8, double>(a, llds, dyn, st)
                             : dispatch_g<RowI8, float>(a, llds, dyn, st);
    }
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
    if (a.g.kv_i8) {
        if (a.g.paged) {
            if (a.g.score_f64) hipLaunchKernelGGL((compact_kernel<double, true, KvRows8>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((compact_kernel<float, true, KvRows8>), grid, block, 0, st, a);
        } else {
            if (a.g.score_f64) hipLaunchKernelGGL((compact_kernel<double, false, KvRows8>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((compact_kernel<float, false, KvRows8>), grid, block, 0, st, a);
        }
    } else if (a.g.paged) {
        if (a.g.score_f64) hipLaunchKernelGGL((compact_kernel<double, true, KvRows>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((compact_kernel<float, true, KvRows>), grid, block, 0, st, a);
    } else if (a.g.kv_tiles) {
        if (a.g.score_f64) hipLaunchKernelGGL((compact_kernel<double, false, KvTiles>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((compact_kernel<float, false, KvTiles>), grid, block, 0, st, a);
    } else {
        if (a.g.score_f64) hipLaunchKernelGGL((compact_kernel<double, false, KvRows>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((compact_kernel<float, false, KvRows>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_load(const LoadArgs& a, int max_prompt, hipStream_t st)
{
    const long long per_seq = (long long)max_prompt * a.g.Hkv * kRowVecs;
    const dim3 grid((unsigned)((per_seq + 255) / 256), a.g.B), block(256);
    if (a.g.kv_i8) {
        if (a.g.paged) {
            if (a.g.score_f64) hipLaunchKernelGGL((load_kernel<double, true, KvRows8>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((load_kernel<float, true, KvRows8>), grid, block, 0, st, a);
        } else {
            if (a.g.score_f64) hipLaunchKernelGGL((load_kernel<double, false, KvRows8>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((load_kernel<float, false, KvRows8>), grid, block, 0, st, a);
        }
    } else if (a.g.paged) {
        if (a.g.score_f64) hipLaunchKernelGGL((load_kernel<double, true, KvRows>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((load_kernel<float, true, KvRows>), grid, block, 0, st, a);
    } else if (a.g.kv_tiles) {
        if (a.g.score_f64) hipLaunchKernelGGL((load_kernel<double, false, KvTiles>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((load_kernel<float, false, KvTiles>), grid, block, 0, st, a);
    } else {
        if (a.g.score_f64) hipLaunchKernelGGL((load_kernel<double, false, KvRows>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((load_kernel<float, false, KvRows>), grid, block, 0, st, a);
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

hipError_t launch_gather_rows(const RowGatherArgs& a, hipStream_t st)
{
    const dim3 grid(a.g.B * a.g.Hkv), block(256);
    if (a.g.kv_i8) {
        if (a.g.paged) hipLaunchKernelGGL((gather_rows_kernel<KvRows8, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((gather_rows_kernel<KvRows8, false>), grid, block, 0, st, a);
    } else if (a.g.kv_tiles) {
        hipLaunchKernelGGL((gather_rows_kernel<KvTiles, false>), grid, block, 0, st, a);
    } else if (a.g.paged) {
        hipLaunchKernelGGL((gather_rows_kernel<KvRows, true>), grid, block, 0, st, a);
    } else {
        hipLaunchKernelGGL((gather_rows_kernel<KvRows, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace h2o
