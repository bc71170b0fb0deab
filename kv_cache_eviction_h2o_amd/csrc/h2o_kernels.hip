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

// ---------------------------------------------------------- compact kernel
constexpr int kCompactNT = 256;

template <typename ST, bool PAGED, typename KV>
__global__ void __launch_bounds__(kCompactNT) compact_kernel(const CompactArgs a)
{
    __shared__ OrderSmem<kCompactNT, kCollectUnroll> s_ord;
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
        fill_holes<kCompactNT, ST, KV>(S, sidx, unit, gm.cap, n_att - e, n_att - e, n_att, n_att, n_att, has_scores,
                                       s_ord);
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
    if (a.g.score_f64) return launch_step_f64(a, llds, dyn, st);
    if (a.g.score_f16) return launch_step_f16(a, llds, dyn, st);
    return launch_step_f32(a, llds, dyn, st);
}

// Calls f with a value of the context's cumulative-score type (fp64, binary16
// or fp32; the Random selector keeps none and takes fp32, unused).
template <typename F>
hipError_t with_score_type(const Geometry& g, F f)
{
    if (g.score_f64) return f(double{});
    if (g.score_f16) return f(_Float16{});
    return f(float{});
}

// ... and with the slot layout: int8 rows, bf16/fp32 rows or operand-order tiles,
// contiguous or paged.
template <template <typename, bool, typename> class Launch, typename A>
hipError_t launch_by_layout(const A& a, hipStream_t st)
{
    return with_score_type(a.g, [&](auto st_tag) {
        using ST = decltype(st_tag);
        if (a.g.kv_i8) return a.g.paged ? Launch<ST, true, KvRows8>::run(a, st) : Launch<ST, false, KvRows8>::run(a, st);
        if (a.g.paged) return Launch<ST, true, KvRows>::run(a, st);
        if (a.g.kv_tiles) return Launch<ST, false, KvTiles>::run(a, st);
        return Launch<ST, false, KvRows>::run(a, st);
    });
}

template <typename ST, bool PAGED, typename KV>
struct CompactLaunch {
    static hipError_t run(const CompactArgs& a, hipStream_t st)
    {
        hipLaunchKernelGGL((compact_kernel<ST, PAGED, KV>), dim3(a.g.B * a.g.Hkv), dim3(kCompactNT), 0, st, a);
        return hipGetLastError();
    }
};

template <typename ST, bool PAGED, typename KV>
struct LoadLaunch {
    static hipError_t run(const LoadArgs& a, hipStream_t st)
    {
        const long long per_seq = (long long)a.max_prompt * a.g.Hkv * kRowVecs;
        hipLaunchKernelGGL((load_kernel<ST, PAGED, KV>), dim3((unsigned)((per_seq + 255) / 256), a.g.B), dim3(256), 0,
                           st, a);
        return hipGetLastError();
    }
};

hipError_t launch_compact(const CompactArgs& a, int /*max_slots*/, hipStream_t st)
{
    return launch_by_layout<CompactLaunch>(a, st);
}

// ------------------------------------------------------------ page relink
// After a window_remap compaction (every head of the sequence done, so no
// workgroup still reads the old entries): entries [front, front + cnt) of the
// sequence's block-table row take entries [src, src + cnt).  The two ranges
// are disjoint (window_remap), so the copy is one parallel pass.
__global__ void __launch_bounds__(256) remap_kernel(const RemapArgs a)
{
    const int i = blockIdx.x;
    int32_t* row = a.bt + (size_t)a.seq_b[i] * a.maxp;
    const int f = a.seq_front[i], src = a.seq_src[i], cnt = a.seq_cnt[i];
    for (int k = (int)threadIdx.x; k < cnt; k += 256) row[f + k] = row[src + k];
}

hipError_t launch_remap(const RemapArgs& a, hipStream_t st)
{
    if (a.nseq <= 0 || a.nseq > kMaxArgBatch || !a.bt) return hipErrorInvalidValue;
    hipLaunchKernelGGL(remap_kernel, dim3(a.nseq), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_load(const LoadArgs& a0, int max_prompt, hipStream_t st)
{
    LoadArgs a = a0;
    a.max_prompt = max_prompt;
    return launch_by_layout<LoadLaunch>(a, st);
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t st)
{
    return with_score_type(a.g, [&](auto st_tag) {
        using ST = decltype(st_tag);
        const dim3 grid(a.g.B * a.g.Hkv), block(256);
        if (a.g.paged) hipLaunchKernelGGL((gather_kernel<ST, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((gather_kernel<ST, false>), grid, block, 0, st, a);
        return hipGetLastError();
    });
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
