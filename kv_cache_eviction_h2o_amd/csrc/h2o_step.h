// The FMA decode-step kernel (template) and its launch dispatch, included by
// one translation unit per cumulative-score type (h2o_step_f32.hip,
// h2o_step_f64.hip, h2o_step_f16.hip) so the instantiations compile in
// parallel.  The kernel itself is described in h2o_kernels.hip.
#pragma once

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
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, sub = tid & 15, grp = tid >> 4;

    // the host knows every sequence's prompt length and retained count: taking
    // them from the arguments saves a dependent memory round trip at the start
    // uniform over the workgroup: readfirstlane keeps them (and the buffer
    // descriptors built from them) in scalar registers
    const int P = __builtin_amdgcn_readfirstlane(sa.p);
    const int t = P + a.step;
    const int n = __builtin_amdgcn_readfirstlane(sa.n);
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
            const int np = sa.newpage < 0 ? -1 : (a.pop_stack ? S.fstack[sa.newpage] : sa.newpage);
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
    // evicted mass of the unit, read now so its update at the end is no round
    // trip (a vector load: waits for scalar or LDS data never wait for it)
    const double emass0 = load_f64(S.emass + unit);
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

// The step launch for score type ST: the row format from the geometry.
template <typename ST>
hipError_t launch_step_scored(const StepArgs& a, bool llds, size_t dyn, hipStream_t st)
{
    if (a.g.kv_i8) return dispatch_g<RowI8, ST>(a, llds, dyn, st);
    if (a.g.kv_bf16) return dispatch_g<RowBf16, ST>(a, llds, dyn, st);
    return dispatch_g<RowF32, ST>(a, llds, dyn, st);
}

}  // namespace
}  // namespace h2o
