// Causal-attention column sums of packed prompts on the matrix cores:
//   out[j] = sum over query rows i in [lo, P) with i >= j, and over the G
//            query heads g of the unit, of softmax_{j' <= i}(scale q_i,g . k_j')[j]
// (per_head: one sum per query head).  With lo = 0 and the sum over the group
// these are the cumulative attention scores the prompt tokens would hold had
// the prompt's own rows been scored like decode steps -- the prefill-scored
// start of H2O's scores; with lo = P - w, per head, SnapKV's observation-window
// vote ("Attention Sinks and KV cache eviction", sec. 4.2 and 4.3).
//
// A row's weights need its softmax maximum and sum over all of its keys
// before any column can take them, so there are two passes:
//   rows   one workgroup per (unit, 4 waves x 8 PT query positions, GW query
//          heads; PT = 4 / G for small groups, else 1, and 1 when at most a
//          128-row window is scored; GW = G up to 4, else 4, and at most 2 for
//          a window):
//          S = Q_tile (8 positions x hi/lo = 16 rows) . K_tile^T (16 keys)
//          with v_mfma_f32_16x16x32_bf16 over 4 k-steps, hi + lo added in the
//          lane (rows 2p and 2p+1 of the C layout); online max / sum per lane
//          over the causal key tiles, then combined over the 16 key lanes by
//          DPP.  Writes the row statistics and the split q tiles (the A
//          operand, so the second pass reads it without converting again).
//   cols   one workgroup per (unit, 256 keys), one wave per 64 keys held as
//          four B operands: every query tile from the keys onwards gives
//          p = 2^(s - M_i) / L_i, summed per key lane (fp32 per tile, fp64
//          across tiles), then over the lane groups.  Each output element has
//          one writer; nothing needs clearing first.
// q is fp32: split into bf16 hi + lo parts as in the decode step; K enters
// exactly; logits keep ~16 significant bits of q.
#include "h2o_device.h"

#include <algorithm>

namespace h2o {
namespace {

constexpr int kCNT = 256;  // threads per workgroup (4 waves)
constexpr float kFloor = -1e30f;

__device__ inline uint4 as_u4(const bf16x8& v)
{
    uint4 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

// combine (max, sum) pairs of the 16 lanes of each row: sum16's DPP stages
template <int CTRL>
__device__ inline void ms_stage(float& m, float& l)
{
    const float mo = dpp<CTRL>(m), lo = dpp<CTRL>(l);
    const float M = fmaxf(m, mo);
    l = l * fast_exp2(m - M) + lo * fast_exp2(mo - M);
    m = M;
}

// PT query tiles of 8 positions per wave: more for small groups so a K tile
// load feeds more products; GW of the group's G query heads per workgroup: a
// group of 8 in two workgroups of 4 keeps the kernel at 3 waves per SIMD
// instead of 2 (qop holds PT * GW * 16 registers)
template <int G>
struct RowsTune {
    static constexpr int PT = G >= 4 ? 1 : 4 / G;
    static constexpr int GW = G > 4 ? 4 : G;
    // with only a window of rows to score (at most 128 per sequence, as for
    // SnapKV's observation window) one tile per wave, so the window's rows
    // spread over all four waves of a workgroup instead of landing on one, and
    // at most two query heads per workgroup, so a large group spreads over
    // G / 2 workgroups instead of running on one
    static constexpr int PT_WINDOW = 1;
    static constexpr int GW_WINDOW = G < 2 ? G : 2;
};

constexpr int kRCK = 4;  // rows pass: 16-key tiles per LDS chunk

// GW query heads per workgroup: heads GW z .. GW z + GW - 1 of the unit's a.G
template <int GW, int PT>
__global__ void __launch_bounds__(kCNT) colsum_rows_kernel(const ColsumArgs a)
{
    // K chunks in B-operand order: [buffer][tile][k-step][lane], lane (lg, lc)
    // holding key 16 tile + lc, elements 32 kb + 8 lg .. +8
    __shared__ uint4 ksm[2][kRCK][4][64];
    // workgroups go to the XCDs round-robin by linear id: with the unit as the
    // fast grid index every XCD gets every position block of an eighth of the
    // units; the longest causal prefixes (the last blocks) are dispatched first
    const int unit = blockIdx.x, b = unit / a.Hkv, h = unit - b * a.Hkv;
    const int pblk = (int)gridDim.y - 1 - (int)blockIdx.y;
    const int P = a.seq_p[b], lo = a.seq_lo[b];
    const int64_t off = a.seq_off[b];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lc = lane & 15, lg = lane >> 4;
    const int wg_base = pblk * 4 * 8 * PT;
    if (wg_base >= P || wg_base + 4 * 8 * PT <= lo) return;  // no row of this workgroup counts
    const int base = wg_base + w * 8 * PT;                   // this wave's first position
    const bool active = base < P && base + 8 * PT > lo;      // uniform over the wave

    // A operands: tile pt, lane (lg, lc) holds d = 32 kb + 8 lg .. +8 of row lc,
    // i.e. of position base + 8 pt + lc / 2, part lc & 1 (hi / lo)
    const bool lo_part = (lc & 1) != 0;
    const int g0 = (int)blockIdx.z * GW;  // the workgroup's first query head in the group
    bf16x8 qop[PT][GW][4];
    if (active) {
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const int prow = min(base + 8 * pt + (lc >> 1), P - 1);
#pragma unroll
            for (int g = 0; g < GW; ++g) {
                const float* qr = a.q + ((size_t)(off + prow) * a.Hq + (size_t)h * a.G + g0 + g) * 128;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const float4 x0 = *reinterpret_cast<const float4*>(qr + 32 * kb + 8 * lg);
                    const float4 x1 = *reinterpret_cast<const float4*>(qr + 32 * kb + 8 * lg + 4);
                    const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                    for (int i = 0; i < 8; ++i) qop[pt][g][kb][i] = split_part(x[i] * a.qscale, lo_part);
                }
            }
        }
    }

    // online row statistics over the causal key tiles; lane lc sees key 16 kt + lc
    const int wg_last = min(wg_base + 4 * 8 * PT - 1, P - 1);
    const int nkt = wg_last / 16 + 1;                                      // the workgroup's tiles
    const int nkt_w = active ? min(base + 8 * PT - 1, P - 1) / 16 + 1 : 0;  // this wave's
    const uint4* kp = reinterpret_cast<const uint4*>(a.k);
    float m[PT][GW][2], l[PT][GW][2];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int g = 0; g < GW; ++g) {
            m[pt][g][0] = m[pt][g][1] = kFloor;
            l[pt][g][0] = l[pt][g][1] = 0.f;
        }
    // chunk c (keys 64 c .. +64): wave w moves tile w, lane (lg, lc) fetching
    // key 16 tile + lc's vectors 4 kb + lg (one per k-step) into registers and
    // then into the B-operand slots it will read.  The loads for chunk c + 1
    // are issued right after a barrier and stay in flight while chunk c is
    // used; the barriers wait for LDS only.
    static_assert(kRCK == 4, "one tile per wave");
    uint4 st0, st1, st2, st3;
#define H2O_ROWS_FETCH(c)                                                                        \
    do {                                                                                         \
        const int key_ = min((c) * 16 * kRCK + 16 * w + lc, P - 1);                               \
        const uint4* src_ = kp + ((size_t)(off + key_) * a.Hkv + h) * kRowVecs + lg;              \
        st0 = src_[0];                                                                           \
        st1 = src_[4];                                                                           \
        st2 = src_[8];                                                                           \
        st3 = src_[12];                                                                          \
    } while (0)
#define H2O_ROWS_PUT(buf)                                                                        \
    do {                                                                                         \
        ksm[buf][w][0][lane] = st0;                                                              \
        ksm[buf][w][1][lane] = st1;                                                              \
        ksm[buf][w][2][lane] = st2;                                                              \
        ksm[buf][w][3][lane] = st3;                                                              \
    } while (0)
    // masked: the tile may hold keys after some of the wave's positions
    // (the causal diagonal); the other tiles skip the per-score test
    auto rows = [&](int kt, int buf, auto masked) {
        constexpr bool MASK = decltype(masked)::value;
        const int key = 16 * kt + lc;
        bf16x8 bt[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) bt[kb] = as_bf16x8(ksm[buf][kt % kRCK][kb][lane]);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const int pos0 = base + 8 * pt + 2 * lg, pos1 = pos0 + 1;  // C rows 4 lg .. +3
#pragma unroll
            for (int g = 0; g < GW; ++g) {
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) c = mma(qop[pt][g][kb], bt[kb], c);
                const float s[2] = {(!MASK || key <= pos0) ? c[0] + c[1] : -INFINITY,
                                    (!MASK || key <= pos1) ? c[2] + c[3] : -INFINITY};
                // one exp2 per score: with d = s - m, either the sum takes
                // 2^d (d <= 0, the maximum stays) or it is rescaled by 2^-d
                // and takes 2^0 = 1 (d > 0, s is the new maximum)
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const float d = s[r] - m[pt][g][r];
                    const float e = fast_exp2(-fabsf(d));
                    const bool up = d > 0.f;
                    l[pt][g][r] = up ? fmaf(l[pt][g][r], e, 1.f) : l[pt][g][r] + e;
                    m[pt][g][r] = up ? s[r] : m[pt][g][r];
                }
            }
        }
    };
    const int nch = (nkt + kRCK - 1) / kRCK;
    H2O_ROWS_FETCH(0);
    H2O_ROWS_PUT(0);
    lds_barrier();
    if (nch > 1) H2O_ROWS_FETCH(1);
    for (int c = 0; c < nch; ++c) {
        const int buf = c & 1;
        const int kt_end = min((c + 1) * kRCK, nkt_w);
        for (int kt = c * kRCK; kt < kt_end; ++kt) {
            if (16 * kt + 15 <= base) rows(kt, buf, std::false_type{});  // every key before every row
            else rows(kt, buf, std::true_type{});
        }
        // chunk c + 1 into the other buffer, which every wave finished reading
        // before the previous barrier
        if (c + 1 < nch) H2O_ROWS_PUT(buf ^ 1);
        lds_barrier();
        if (c + 2 < nch) H2O_ROWS_FETCH(c + 2);
    }
#undef H2O_ROWS_FETCH
#undef H2O_ROWS_PUT
    if (!active) return;
    // the split q tiles for the columns pass, stored only now: the vector
    // memory counter retires in order, so stores issued before the key loop
    // made every wait for a K chunk wait for them as well (storing them right
    // after the last K fetch instead measured no faster over both passes)
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
        const int ts = base / 8 + pt - lo / 8;  // the scratch keeps tiles from row lo's on
        if (ts < 0 || ts >= a.nt8) continue;
#pragma unroll
        for (int g = 0; g < GW; ++g)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                a.qs[(((size_t)unit * a.nt8 + ts) * a.G + g0 + g) * 256 + kb * 64 + lane] = as_u4(qop[pt][g][kb]);
    }
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int g = 0; g < GW; ++g)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                ms_stage<0xB1>(m[pt][g][r], l[pt][g][r]);
                ms_stage<0x4E>(m[pt][g][r], l[pt][g][r]);
                ms_stage<0x141>(m[pt][g][r], l[pt][g][r]);
                ms_stage<0x140>(m[pt][g][r], l[pt][g][r]);
            }
    if (lc == 0) {
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const int ts = base / 8 + pt - lo / 8;
            if (ts < 0 || ts >= a.nt8) continue;
#pragma unroll
            for (int g = 0; g < GW; ++g) {
                float4* sp =
                    reinterpret_cast<float4*>(a.st + (((size_t)unit * a.nt8 + ts) * a.G + g0 + g) * 8 + 2 * lg);
                *sp = make_float4(m[pt][g][0], 1.0f / l[pt][g][0], m[pt][g][1], 1.0f / l[pt][g][1]);
            }
        }
    }
}

__device__ inline double xrow_add(double v, bool x32)
{
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const Pair lo = x32 ? xrow32((unsigned)u) : xrow16((unsigned)u);
    const Pair hi = x32 ? xrow32((unsigned)(u >> 32)) : xrow16((unsigned)(u >> 32));
    const double a = __longlong_as_double((long long)(((unsigned long long)hi.a << 32) | lo.a));
    const double c = __longlong_as_double((long long)(((unsigned long long)hi.b << 32) | lo.b));
    return a + c;
}

constexpr int kKT = 4;  // 16-key B tiles per wave (64 keys)

// columns pass: query tiles (8 positions, all G heads) per LDS chunk
template <int G>
struct ColsTune {
    static constexpr int CQ = G >= 4 ? 1 : 4 / G;
};

template <int G, bool PH>
__global__ void __launch_bounds__(kCNT) colsum_cols_kernel(const ColsumArgs a)
{
    constexpr int NA = PH ? G : 1;
    constexpr int CQ = ColsTune<G>::CQ;
    // query chunks as the rows pass left them: [buffer][tile][head][k-step][lane]
    // A operands, and each (tile, head)'s row statistics
    __shared__ uint4 qsm[2][CQ][G][4][64];
    __shared__ float4 ssm[2][CQ][G][4];
    // lambdas below index the buffers through these (the host pass drops the
    // kernel's launch stub when a lambda names these dependent-size arrays)
    uint4* const qsm0 = &qsm[0][0][0][0][0];
    float4* const ssm0 = &ssm[0][0][0][0];
    constexpr int QB = CQ * G * 4 * 64, SB = CQ * G * 4;  // per buffer: 16-byte q vectors, statistics
    // the unit is the fast grid index (every XCD gets every key block of an
    // eighth of the units); the first key blocks, which walk the most query
    // tiles, are dispatched first
    const int unit = blockIdx.x, b = unit / a.Hkv, h = unit - b * a.Hkv;
    const int P = a.seq_p[b], lo = a.seq_lo[b];
    const int64_t off = a.seq_off[b];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lc = lane & 15, lg = lane >> 4;
    const int wk0 = blockIdx.y * 4 * 16 * kKT;  // the workgroup's first key
    if (wk0 >= P) return;
    const int k0 = wk0 + w * 16 * kKT;  // this wave's first key
    const bool active = k0 < P;
    const uint4* kp = reinterpret_cast<const uint4*>(a.k);
    uint4 kt4[kKT][4];
    if (active) {
#pragma unroll
        for (int x = 0; x < kKT; ++x) {
            const int kr = min(k0 + 16 * x + lc, P - 1);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) kt4[x][kb] = kp[((size_t)(off + kr) * a.Hkv + h) * kRowVecs + 4 * kb + lg];
        }
    }

    double acc[kKT][NA];
#pragma unroll
    for (int x = 0; x < kKT; ++x)
#pragma unroll
        for (int y = 0; y < NA; ++y) acc[x][y] = 0.0;
    // the workgroup walks query tiles from its first key (or row lo) to the end;
    // a wave skips the tiles wholly before its own keys
    const int t_first = max(wk0, lo) / 8, t_last = (P - 1) / 8;
    const int t_first_w = active ? max(k0, lo) / 8 : t_last + 1;
    const uint4* qg = a.qs + (size_t)unit * a.nt8 * G * 256;
    const float4* sg = reinterpret_cast<const float4*>(a.st + (size_t)unit * a.nt8 * G * 8);
    // a chunk (CQ tiles of G heads: CQ G 4 k-steps of 1 KB, plus CQ G 4 float4
    // of row statistics) is copied in the same order: every thread moves
    // vectors tid + 256 r through registers.  The loads for chunk c + 1 are
    // issued right after a barrier and stay in flight while chunk c is used;
    // the barriers wait for LDS only.
    constexpr int NV = CQ * G;  // 16-byte vectors per thread (CQ G 4 64 per chunk)
    static_assert(CQ * G * 4 <= 256, "statistics: one vector per thread");
    static_assert(NV == 4 || NV == 8, "staging registers");
    // named registers: an array here ends up in scratch memory
    uint4 s0, s1, s2, s3, s4, s5, s6, s7;
    float4 ss;
    const int t8lo = lo / 8;  // the scratch keeps tiles from row lo's on
    auto qvec = [&](int t0, int r) {
        const int q = tid + 256 * r;
        const int t8 = min(t0 + q / (G * 256), t_last);
        return qg[(size_t)(t8 - t8lo) * G * 256 + (q % (G * 256))];
    };
#define H2O_COLS_FETCH(t0)                                                                              \
    do {                                                                                                \
        s0 = qvec((t0), 0);                                                                             \
        s1 = qvec((t0), 1);                                                                             \
        s2 = qvec((t0), 2);                                                                             \
        s3 = qvec((t0), 3);                                                                             \
        if constexpr (NV == 8) {                                                                        \
            s4 = qvec((t0), 4);                                                                         \
            s5 = qvec((t0), 5);                                                                         \
            s6 = qvec((t0), 6);                                                                         \
            s7 = qvec((t0), 7);                                                                         \
        }                                                                                               \
        if (tid < CQ * G * 4) ss = sg[(size_t)(min((t0) + tid / (G * 4), t_last) - t8lo) * G * 4 + tid % (G * 4)]; \
    } while (0)
#define H2O_COLS_PUT(buf)                                                                               \
    do {                                                                                                \
        uint4* qd_ = qsm0 + (buf) * QB + tid;                                                           \
        qd_[0] = s0;                                                                                    \
        qd_[256] = s1;                                                                                  \
        qd_[512] = s2;                                                                                  \
        qd_[768] = s3;                                                                                  \
        if constexpr (NV == 8) {                                                                        \
            qd_[1024] = s4;                                                                             \
            qd_[1280] = s5;                                                                             \
            qd_[1536] = s6;                                                                             \
            qd_[1792] = s7;                                                                             \
        }                                                                                               \
        if (tid < CQ * G * 4) ssm0[(buf) * SB + tid] = ss;                                              \
    } while (0)
    // masked: the tile may hold rows before some of the wave's keys, or rows
    // outside [lo, P); the other tiles skip the per-score test
    auto tile = [&](int t8, int ci, int buf, auto masked) {
        constexpr bool MASK = decltype(masked)::value;
        const int pos0 = 8 * t8 + 2 * lg, pos1 = pos0 + 1;
        const bool r0 = pos0 < P && pos0 >= lo, r1 = pos1 < P && pos1 >= lo;
        float tacc[kKT][NA];
#pragma unroll
        for (int x = 0; x < kKT; ++x)
#pragma unroll
            for (int y = 0; y < NA; ++y) tacc[x][y] = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            bf16x8 q4[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) q4[kb] = as_bf16x8(qsm0[buf * QB + ((ci * G + g) * 4 + kb) * 64 + lane]);
            const float4 sv = ssm0[buf * SB + (ci * G + g) * 4 + lg];
#pragma unroll
            for (int x = 0; x < kKT; ++x) {
                const int key = k0 + 16 * x + lc;
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) c = mma(q4[kb], as_bf16x8(kt4[x][kb]), c);
                const float p0 = (!MASK || (r0 && key <= pos0)) ? fast_exp2(c[0] + c[1] - sv.x) * sv.y : 0.f;
                const float p1 = (!MASK || (r1 && key <= pos1)) ? fast_exp2(c[2] + c[3] - sv.z) * sv.w : 0.f;
                tacc[x][PH ? g : 0] += p0 + p1;
            }
        }
#pragma unroll
        for (int x = 0; x < kKT; ++x)
#pragma unroll
            for (int y = 0; y < NA; ++y) acc[x][y] += (double)tacc[x][y];
    };
    const int nch = (t_last - t_first) / CQ + 1;
    H2O_COLS_FETCH(t_first);
    H2O_COLS_PUT(0);
    lds_barrier();
    if (nch > 1) H2O_COLS_FETCH(t_first + CQ);
    for (int c = 0; c < nch; ++c) {
        const int buf = c & 1, t0 = t_first + c * CQ;
#pragma unroll
        for (int ci = 0; ci < CQ; ++ci) {
            const int t8 = t0 + ci;
            if (t8 >= t_first_w && t8 <= t_last) {
                // rows 8 t8 .. +7 all after the wave's last key and inside [lo, P)
                if (8 * t8 >= k0 + 16 * kKT - 1 && 8 * t8 >= lo && 8 * t8 + 7 < P) tile(t8, ci, buf, std::false_type{});
                else tile(t8, ci, buf, std::true_type{});
            }
        }
        // chunk c + 1 into the other buffer, which every wave finished reading
        // before the previous barrier
        if (c + 1 < nch) H2O_COLS_PUT(buf ^ 1);
        lds_barrier();
        if (c + 2 < nch) H2O_COLS_FETCH(t0 + 2 * CQ);
    }
#undef H2O_COLS_FETCH
#undef H2O_COLS_PUT
    if (!active) return;
    // sum over the four lane groups (the rows); every lane then holds its key's total
#pragma unroll
    for (int x = 0; x < kKT; ++x) {
#pragma unroll
        for (int y = 0; y < NA; ++y) {
            acc[x][y] = xrow_add(acc[x][y], false);
            acc[x][y] = xrow_add(acc[x][y], true);
        }
        const int key = k0 + 16 * x + lc;
        if (lg == 0 && key < P) {
            if constexpr (PH) {
#pragma unroll
                for (int g = 0; g < G; ++g) a.out[(size_t)(off + key) * a.Hq + (size_t)h * G + g] = acc[x][g];
            } else {
                a.out[(size_t)(off + key) * a.Hkv + h] = acc[x][0];
            }
        }
    }
}

template <int G>
hipError_t launch_colsum_g(const ColsumArgs& a, int max_p, hipStream_t st)
{
    const unsigned units = (unsigned)(a.B * a.Hkv);
    constexpr int PTF = RowsTune<G>::PT, GWF = RowsTune<G>::GW;
    constexpr int PTW = RowsTune<G>::PT_WINDOW, GWW = RowsTune<G>::GW_WINDOW;
    const bool window = a.nt8 <= 16;  // at most 128 rows per sequence from row lo on
    const int rows_per_wg = 4 * 8 * (window ? PTW : PTF), keys_per_wg = 4 * 16 * kKT;
    const unsigned pblocks = (unsigned)((max_p + rows_per_wg - 1) / rows_per_wg);
    if (window)
        hipLaunchKernelGGL((colsum_rows_kernel<GWW, PTW>), dim3(units, pblocks, G / GWW), dim3(kCNT), 0, st, a);
    else
        hipLaunchKernelGGL((colsum_rows_kernel<GWF, PTF>), dim3(units, pblocks, G / GWF), dim3(kCNT), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 gc(units, (max_p + keys_per_wg - 1) / keys_per_wg);
    if (a.per_head)
        hipLaunchKernelGGL((colsum_cols_kernel<G, true>), gc, dim3(kCNT), 0, st, a);
    else
        hipLaunchKernelGGL((colsum_cols_kernel<G, false>), gc, dim3(kCNT), 0, st, a);
    return hipGetLastError();
}

// ------------------------------------------------------------ SnapKV
// ("Attention Sinks and KV cache eviction", sec. 4.3) from the per-head window
// votes: max pooling over the prefix, each query head's top `keep` prefix
// positions, the union over the unit's heads, plus the window.
__global__ void __launch_bounds__(256) snapkv_pool_kernel(const SnapArgs a)
{
    const int b = blockIdx.y;
    const int P = a.seq_p[b], Pp = P - a.seq_w[b];
    const int64_t off = a.seq_off[b];
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;  // (j, query head)
    if (idx >= (long long)Pp * a.Hq) return;
    const int j = (int)(idx / a.Hq), hq = (int)(idx - (long long)j * a.Hq);
    const int x0 = max(0, j - a.pool_r), x1 = min(Pp - 1, j + a.pool_r);
    double m = -INFINITY;
    for (int x = x0; x <= x1; ++x) m = fmax(m, a.votes[(size_t)(off + x) * a.Hq + hq]);
    a.pooled[(size_t)(off + j) * a.Hq + hq] = m;
}

constexpr int kSNT = 256;
constexpr int kSnapStage = 4096;  // prefix positions whose pooled votes are staged in LDS

// One query head's selection: the bits of its `keep` highest-voted prefix
// positions OR-ed into the LDS bitmap.  Keys as in the decode step's bulk
// selection, (vote bits, ~position): the e smallest go, so equal votes keep
// the lower position.  When `staged` the head's votes are copied to `stage`
// and max-pooled there (through registers, then back in place), and the radix
// passes read LDS; otherwise they read the pooling kernel's output.
__device__ inline void snap_head(const SnapArgs& a, int hq, int Pp, int64_t off, bool staged, double* stage,
                                 unsigned* bits, RadixSmem& s_rad)
{
    const int tid = threadIdx.x;
    const int e = Pp - a.keep;  // prefix positions each head leaves out
    if (staged && e > 0) {
        for (int j = tid; j < Pp; j += kSNT) stage[j] = a.votes[(size_t)(off + j) * a.Hq + hq];
        __syncthreads();
        constexpr int NPT = kSnapStage / kSNT;  // staged positions per thread
        double pv[NPT];
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
            const int j = tid + k * kSNT;
            double m = -INFINITY;
            if (j < Pp) {
                const int x0 = max(0, j - a.pool_r), x1 = min(Pp - 1, j + a.pool_r);
                for (int x = x0; x <= x1; ++x) m = fmax(m, stage[x]);
            }
            pv[k] = m;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
            const int j = tid + k * kSNT;
            if (j < Pp) stage[j] = pv[k];
        }
        __syncthreads();
    }
    auto key_of = [&](int j, unsigned (&wk)[3]) -> bool {
        const unsigned long long u = ord64(staged ? stage[j] : a.pooled[(size_t)(off + j) * a.Hq + hq]);
        wk[2] = (unsigned)(u >> 32);
        wk[1] = (unsigned)u;
        wk[0] = ~(unsigned)j;
        return true;
    };
    if (e > 0) {
        radix_select<kSNT>(key_of, Pp, e, 0, s_rad);
        for (int j = tid; j < Pp; j += kSNT) {
            unsigned wk[3];
            key_of(j, wk);
            if (!key_le(wk, s_rad)) atomicOr(&bits[j >> 5], 1u << (j & 31));
        }
    } else {
        for (int j = tid; j < Pp; j += kSNT) atomicOr(&bits[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
}

// The window's positions added to the unit's bitmap, then the kept positions
// in ascending order, -1 past the count (NT threads).
template <int NT, typename SA>
__device__ inline void snap_finish(const SA& a, int unit, int P, int Pp, unsigned* bits, ScanSmem& s_scan)
{
    const int tid = threadIdx.x;
    for (int j = Pp + tid; j < P; j += NT) atomicOr(&bits[j >> 5], 1u << (j & 31));
    __syncthreads();
    int* out = a.kept + (size_t)unit * a.cap;
    const int n = collect<NT>(0, P, [&](int j) { return ((bits[j >> 5] >> (j & 31)) & 1u) != 0; }, out,
                              s_scan);
    for (int i = n + tid; i < a.cap; i += NT) out[i] = -1;
    if (tid == 0) a.count[unit] = n;
}

// G = 1: one workgroup per unit does the whole selection.
__global__ void __launch_bounds__(kSNT) snapkv_select_kernel(const SnapArgs a)
{
    // one bit per prompt position (kept), then the staged pooled votes
    extern __shared__ __align__(16) unsigned bits[];
    __shared__ RadixSmem s_rad;
    __shared__ ScanSmem s_scan;
    const int unit = blockIdx.x, b = unit / a.Hkv, h = unit - b * a.Hkv;
    const int P = a.seq_p[b], Pp = P - a.seq_w[b];
    const int64_t off = a.seq_off[b];
    const int tid = threadIdx.x;
    const int nw = (P + 31) / 32;
    double* stage = reinterpret_cast<double*>(bits + a.bits_words);
    for (int i = tid; i < nw; i += kSNT) bits[i] = 0u;
    __syncthreads();
    for (int g = 0; g < a.G; ++g) snap_head(a, h * a.G + g, Pp, off, Pp <= a.stage_n, stage, bits, s_rad);
    snap_finish<kSNT>(a, unit, P, Pp, bits, s_scan);
}

// G > 1, first kernel: one workgroup per (unit, query head) selects that
// head's positions and writes its bitmap to hbits[unit][g][bits_words].
__global__ void __launch_bounds__(kSNT) snapkv_head_kernel(const SnapArgs a)
{
    extern __shared__ __align__(16) unsigned bits[];
    __shared__ RadixSmem s_rad;
    const int unit = blockIdx.x, g = blockIdx.y, b = unit / a.Hkv, h = unit - b * a.Hkv;
    const int P = a.seq_p[b], Pp = P - a.seq_w[b];
    const int64_t off = a.seq_off[b];
    const int tid = threadIdx.x;
    const int nw = (Pp + 31) / 32;
    double* stage = reinterpret_cast<double*>(bits + a.bits_words);
    for (int i = tid; i < nw; i += kSNT) bits[i] = 0u;
    __syncthreads();
    snap_head(a, h * a.G + g, Pp, off, Pp <= a.stage_n, stage, bits, s_rad);
    unsigned* hb = a.hbits + ((size_t)unit * a.G + g) * a.bits_words;
    for (int i = tid; i < nw; i += kSNT) hb[i] = bits[i];
}

// G > 1, second kernel: one workgroup per unit ORs its heads' bitmaps (the
// launch boundary orders them after the first kernel's stores), adds the
// window and compacts.
__global__ void __launch_bounds__(kSNT) snapkv_union_kernel(const SnapArgs a)
{
    extern __shared__ __align__(16) unsigned bits[];
    __shared__ ScanSmem s_scan;
    const int unit = blockIdx.x, b = unit / a.Hkv;
    const int P = a.seq_p[b], Pp = P - a.seq_w[b];
    const int tid = threadIdx.x;
    const int nwp = (Pp + 31) / 32, nw = (P + 31) / 32;
    const unsigned* hb = a.hbits + (size_t)unit * a.G * a.bits_words;
    for (int i = tid; i < nw; i += kSNT) {
        unsigned x = 0u;
        if (i < nwp)
            for (int g = 0; g < a.G; ++g) x |= hb[(size_t)g * a.bits_words + i];
        bits[i] = x;
    }
    __syncthreads();
    snap_finish<kSNT>(a, unit, P, Pp, bits, s_scan);
}

// ------------------------------------------------------- SnapKV in one pass
// Prompts up to kFusedP positions and observation windows of at most 32 rows:
// one workgroup per (unit, query head) streams the unit's K once (the two
// column-sum passes read it twice and hand the row statistics and the votes
// over through memory; the G workgroups of a unit share its K through L2,
// see the id mapping below).  Wave v holds the window rows' logits for
// keys 128 v .. 128 v + 127 in registers (8 tiles of 16 keys, the same
// matrix-core products as the rows pass); the workgroup merges each row's
// softmax maximum and sum over the waves in LDS, and each key's vote is the
// sum over the window rows of its weight (fp32 per query tile, fp64 across
// them, as the columns pass sums).  The prefix's votes go straight into LDS,
// from which the selection pools into registers (snap_head_small).
constexpr int kFNT = 512;                   // threads (8 waves)
constexpr int kFKT = 8;                     // 16-key tiles per wave
constexpr int kFusedP = (kFNT / 64) * kFKT * 16;  // 1024 positions
constexpr int kFQT = 4;                     // query tiles of 8 window rows: 32 rows
constexpr float kMaskLogit = -1e30f;        // finite: this file assumes no NaN or infinity arithmetic

// Inclusive prefix sum over a wave: DPP row shifts within each row of 16
// lanes, then row broadcasts of lane 15 (into rows 1 and 3) and lane 31 (into
// rows 2 and 3).
template <int CTRL, int ROW_MASK>
__device__ inline unsigned dpp_src(unsigned v)
{
    return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, true);
}
__device__ inline unsigned wave_incl_scan(unsigned v)
{
    v += dpp_src<0x111, 0xF>(v);  // row_shr:1
    v += dpp_src<0x112, 0xF>(v);  // row_shr:2
    v += dpp_src<0x114, 0xF>(v);  // row_shr:4
    v += dpp_src<0x118, 0xF>(v);  // row_shr:8
    v += dpp_src<0x142, 0xA>(v);  // row_bcast:15
    v += dpp_src<0x143, 0xC>(v);  // row_bcast:31
    return v;
}

// Selection of the e smallest of n <= NT KPT keys held in registers, element
// tid + NT i in slot i of thread tid, each key (w2, w1, ~index) as the decode
// step's and radix_select's (96 bits, unique): the same 8-bit digits from the
// top, the same early stop (once the chosen bin holds exactly the victims
// still missing) and the same victims.  Each element keeps two flags, still
// in the chosen prefix and already below it, updated by one comparison a
// digit; a wave whose candidates of one digit fall in a single bin counts
// them with one atomic; every wave scans the histogram itself (one DPP prefix
// sum, then the chosen lane's four bins on scalars), and the histograms rotate
// over three buffers (one counted, one scanned, one cleared), so a digit costs
// one barrier.  For n <= 65536 the two top digits of ~index, 0xff for every
// key, are taken without a pass (such a pass leaves every candidate in the
// bin, so it can neither narrow the set nor stop the selection).
struct alignas(16) SmallSelSmem {
    unsigned hist[3][256];
};

template <int NT, int KPT>
__device__ inline void select_small(const unsigned (&w2)[KPT], const unsigned (&w1)[KPT], int n, int e,
                                    bool (&drop)[KPT], SmallSelSmem& sm)
{
    const int tid = threadIdx.x, lane = tid & 63;
    for (int i = tid; i < 256; i += NT) sm.hist[0][i] = 0u;
    lds_barrier();
    bool cand[KPT], below[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        cand[i] = tid + NT * i < n;
        below[i] = false;
    }
    unsigned rem = (unsigned)e;
    int c = 0;  // passes made: pass c counts into hist[c % 3]
#pragma unroll
    for (int d = 0; d < 12; ++d) {
        if ((d == 8 || d == 9) && n <= 65536) continue;  // digits 8 and 9 of ~index are 0xff for every key
        const int wi = 2 - (d >> 2), sh = 24 - 8 * (d & 3);
        unsigned* h = sm.hist[c % 3];
        unsigned bin[KPT];
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const unsigned word = wi == 2 ? w2[i] : (wi == 1 ? w1[i] : ~(unsigned)(tid + NT * i));
            bin[i] = (word >> sh) & 255u;
            const unsigned b = cand[i] ? bin[i] : 256u;  // 256: not counted
            const unsigned b0 = __builtin_amdgcn_readfirstlane(b);
            const unsigned long long act = __ballot(1);
            if (__ballot(b != b0) == 0ull) {
                if (b0 < 256u && lane == __ffsll((long long)act) - 1) atomicAdd(&h[b0], (unsigned)__popcll(act));
            } else if (b < 256u) {
                atomicAdd(&h[b], 1u);
            }
        }
        // the next pass's buffer: last scanned two passes ago, before the previous barrier
        for (int i = tid; i < 256; i += NT) sm.hist[(c + 1) % 3][i] = 0u;
        lds_barrier();
        const uint4 cb = reinterpret_cast<const uint4*>(h)[lane];
        const unsigned loc = cb.x + cb.y + cb.z + cb.w;
        const unsigned inc = wave_incl_scan(loc);
        // the rem-th smallest candidate lies in the first lane whose prefix reaches
        // rem (there is one: rem never exceeds the candidates left, lane 63's prefix)
        const int src = __ffsll((long long)__ballot(inc >= rem)) - 1;
        unsigned run = (unsigned)__builtin_amdgcn_readlane((int)(inc - loc), src);
        const unsigned c0 = (unsigned)__builtin_amdgcn_readlane((int)cb.x, src);
        const unsigned c1 = (unsigned)__builtin_amdgcn_readlane((int)cb.y, src);
        const unsigned c2 = (unsigned)__builtin_amdgcn_readlane((int)cb.z, src);
        const unsigned c3 = (unsigned)__builtin_amdgcn_readlane((int)cb.w, src);
        unsigned k = 0, cnt = c0;
        if (rem > run + c0) {
            run += c0;
            k = 1;
            cnt = c1;
            if (rem > run + c1) {
                run += c1;
                k = 2;
                cnt = c2;
                if (rem > run + c2) {
                    run += c2;
                    k = 3;
                    cnt = c3;
                }
            }
        }
        const unsigned sel = 4u * (unsigned)src + k;
        rem -= run;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            below[i] = below[i] || (cand[i] && bin[i] < sel);
            cand[i] = cand[i] && bin[i] == sel;
        }
        ++c;
        if (cnt == rem) break;  // every candidate left in the bin is a victim
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) drop[i] = below[i] || cand[i];
}

// snap_head for prefixes of at most NT KPT positions whose votes are staged:
// each thread max-pools its KPT positions straight into registers, and the
// selection runs on them (select_small).
template <int NT, int KPT, typename SA>
__device__ inline void snap_head_small(const SA& a, int Pp, const double* stage, unsigned* bits, SmallSelSmem& sm)
{
    const int tid = threadIdx.x;
    const int e = Pp - a.keep;  // prefix positions the head leaves out
    if (e > 0) {
        unsigned w2[KPT], w1[KPT];
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int j = tid + NT * i;
            double m = 0.0;
            if (j < Pp) {
                const int x0 = max(0, j - a.pool_r), x1 = min(Pp - 1, j + a.pool_r);
                m = stage[x0];
                for (int x = x0 + 1; x <= x1; ++x) m = fmax(m, stage[x]);
            }
            const unsigned long long u = ord64(m);
            w2[i] = (unsigned)(u >> 32);
            w1[i] = (unsigned)u;
        }
        bool drop[KPT];
        select_small<NT, KPT>(w2, w1, Pp, e, drop, sm);
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int j = tid + NT * i;
            if (j < Pp && !drop[i]) atomicOr(&bits[j >> 5], 1u << (j & 31));
        }
    } else {
        for (int j = tid; j < Pp; j += NT) atomicOr(&bits[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
}

// Orders a wave's LDS accesses around an exchange among its own lanes (the
// LDS serves one wave's accesses in issue order; this keeps the compiler
// from moving them across).
__device__ inline void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct SnapFusedArgs {
    const float* q;  // [sum P][Hq][128]
    const void* k;   // [sum P][Hkv][128] bf16
    float qscale;    // logit scale * log2(e)
    int Hq, Hkv, G;
    int units;              // B * Hkv
    int pool_r, keep, cap;
    double* votes;          // [sum P][Hq]
    const double* pooled;  // not read: the votes are staged
    int32_t* kept;          // G = 1: [B * Hkv][cap]
    int32_t* count;
    unsigned* hbits;        // G > 1: [B * Hkv][G][bits_words], each query head's kept prefix bits
    int bits_words;
    int32_t seq_p[kMaxArgBatch], seq_w[kMaxArgBatch];
    int64_t seq_off[kMaxArgBatch];
};

// Two workgroups per CU (at most 128 VGPRs: the q operands are read from LDS
// for each tile, and two K tiles are in flight per wave), so that one
// workgroup's selection overlaps another's K stream.
__global__ void __launch_bounds__(kFNT, 4) snapkv_fused_kernel(const SnapFusedArgs a)
{
    __shared__ uint4 qsm[kFQT][4][64];      // A operands of the window rows (hi / lo parts)
    __shared__ uint4 ktr[kFNT / 64][256];    // per wave: a K tile on its way to B-operand order
    __shared__ float2 wml[kFNT / 64][kFQT * 8];  // per wave and window row: (max, sum)
    __shared__ float2 rowf[kFQT * 8];       // per window row: (max, 1 / sum), 1 / sum = 0 past P
    __shared__ double stage[kFusedP];       // the prefix's votes, then pooled in place
    __shared__ unsigned bits[kFusedP / 32];
    __shared__ SmallSelSmem s_sel;
    __shared__ ScanSmem s_scan;
    // one workgroup per (unit, query head g of its group): ids 64 c + 8 g + u
    // serve unit 8 c + u, so the G workgroups of a unit reach the same XCD
    // (ids go to the XCDs round-robin) and are dispatched together, and the
    // unit's K, read by each of them, comes from that XCD's L2 after the first
    // (groups of one head: ids 64 c + 8 u + v serve unit 64 c + 8 v + u, so the 8
    // consecutive units whose votes share 64-byte segments of a vote row write
    // them from one XCD, whose L2 merges the 8-byte pieces into whole lines)
    const int id = blockIdx.x;
    int g, unit;
    if (a.G == 1) {
        g = 0;
        unit = (id & ~63) + 8 * (id & 7) + ((id >> 3) & 7);
    } else {
        const int c8 = id / (8 * a.G), r8 = id - c8 * 8 * a.G;
        g = r8 >> 3;
        unit = 8 * c8 + (r8 & 7);
    }
    if (unit >= a.units) return;  // the last group of units may be partial
    const int b = unit / a.Hkv, h = unit - b * a.Hkv, hq = h * a.G + g;
    const int P = a.seq_p[b], lo = P - a.seq_w[b];  // window rows [lo, P); prefix [0, lo)
    const int64_t off = a.seq_off[b];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lc = lane & 15, lg = lane >> 4;
    const int key0 = 128 * wv;
    const int nt = min(kFKT, max(0, (P - key0 + 15) / 16));  // tiles holding keys below P (uniform)

    // the window rows' q first (the vector memory counter retires in order, so
    // the staging below waits for these loads, not for the K tiles after them)
    float4 qx[4];
    int qv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int v = tid + kFNT * i;  // A-operand vector (tq, kb, lane)
        const int ln = v & 63, kb = (v >> 6) & 3, tq = v >> 8;
        const int pos = min(lo + 8 * tq + ((ln & 15) >> 1), P - 1);
        const float* qr = a.q + ((size_t)(off + pos) * a.Hq + hq) * 128 + 32 * kb + 8 * (ln >> 4);
        qx[2 * i] = *reinterpret_cast<const float4*>(qr);
        qx[2 * i + 1] = *reinterpret_cast<const float4*>(qr + 4);
        qv[i] = v;
    }
    for (int i = tid; i < kFusedP / 32; i += kFNT) bits[i] = 0u;
    // K tiles in whole rows: load i of lane (lg, lc) is key key0 + 16 x + 4 i + lg's
    // vector lc, so each load instruction reads four 256-byte rows (the B
    // operand's order, key lc's vectors 4 kb + lg, would read sixteen half rows
    // per instruction: ~4 us slower at the OPT layer's prompts)
    const uint4* kp = reinterpret_cast<const uint4*>(a.k) + (size_t)h * kRowVecs + lc;
    auto fetch = [&](int x, uint4 (&r)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = min(key0 + 16 * x + 4 * i + lg, P - 1);
            r[i] = stream_load(kp + (size_t)(off + key) * a.Hkv * kRowVecs);
        }
    };
    // then through the wave's LDS tile into B-operand order: element (key 4 i + lg,
    // vector lc) is k-step lc / 4 of lane (lc % 4, 4 i + lg), i.e. slot
    // 16 lc + 4 i + lg; each 16-slot block's slots are XOR-ed with the block
    // number, so that both the writes (16 lanes of one lg, one slot of each
    // block) and the reads (16 consecutive slots) touch 16 different banks
    uint4* const kw = &ktr[wv][0];
    auto swz = [](int sl) { return sl ^ ((sl >> 4) & 15); };
    auto put_k = [&](const uint4 (&r)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) kw[swz(16 * lc + 4 * i + lg)] = r[i];
    };
    auto get_b = [&](bf16x8 (&bt)[4]) {
        wave_lds_sync();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) bt[kb] = as_bf16x8(kw[swz(64 * kb + lane)]);
        wave_lds_sync();  // the next tile's writes after these reads
    };
    uint4 kt0[4], kt1[4];  // two tiles in flight per wave
    if (nt > 0) fetch(0, kt0);
    if (nt > 1) fetch(1, kt1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int v = qv[i], ln = v & 63;
        const bool lo_part = (ln & 1) != 0;
        const float x[8] = {qx[2 * i].x, qx[2 * i].y, qx[2 * i].z, qx[2 * i].w,
                            qx[2 * i + 1].x, qx[2 * i + 1].y, qx[2 * i + 1].z, qx[2 * i + 1].w};
        bf16x8 o;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = split_part(x[j] * a.qscale, lo_part);
        (&qsm[0][0][0])[v] = as_u4(o);
    }
    lds_barrier();

    // logits: s[x][tq][r] = row lo + 8 tq + 2 lg + r against key key0 + 16 x + lc,
    // kMaskLogit after the row (causal), past P, or on a tile past P
    float s[kFKT][kFQT][2];
#pragma unroll
    for (int x = 0; x < kFKT; ++x) {
        uint4(&cur)[4] = (x & 1) ? kt1 : kt0;
        if (x < nt) {
            bf16x8 bt[4];
            put_k(cur);
            if (x + 2 < nt) fetch(x + 2, cur);
            get_b(bt);
            const int key = key0 + 16 * x + lc;
            // only a tile reaching past the window's first row holds keys after
            // some row (keys past P are after every row below P); rows past P
            // are dropped later (their 1 / sum is 0)
            const bool diag = key0 + 16 * x + 15 > lo;
#pragma unroll
            for (int tq = 0; tq < kFQT; ++tq) {
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) c = mma(as_bf16x8(qsm[tq][kb][lane]), bt[kb], c);
                const int pos0 = lo + 8 * tq + 2 * lg;
                s[x][tq][0] = c[0] + c[1];
                s[x][tq][1] = c[2] + c[3];
                if (diag) {
                    s[x][tq][0] = key <= pos0 ? s[x][tq][0] : kMaskLogit;
                    s[x][tq][1] = key <= pos0 + 1 ? s[x][tq][1] : kMaskLogit;
                }
            }
        } else {
#pragma unroll
            for (int tq = 0; tq < kFQT; ++tq) s[x][tq][0] = s[x][tq][1] = kMaskLogit;
        }
    }

    // each row's maximum over the wave's keys (the lane's 8, then the 16 key
    // lanes by DPP), the weights relative to it (kept in s), their sum, then
    // the row's maximum and sum over the waves in LDS
    float m16[kFQT][2], l16[kFQT * 2];  // l16[2 tq + r]
#pragma unroll
    for (int tq = 0; tq < kFQT; ++tq)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            float m = s[0][tq][r];
#pragma unroll
            for (int x = 1; x < kFKT; ++x) m = fmaxf(m, s[x][tq][r]);
            m16[tq][r] = max16(m);
        }
#pragma unroll
    for (int tq = 0; tq < kFQT; ++tq)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            float l = 0.f;
#pragma unroll
            for (int x = 0; x < kFKT; ++x) {
                s[x][tq][r] = fast_exp2(s[x][tq][r] - m16[tq][r]);
                l += s[x][tq][r];
            }
            l16[2 * tq + r] = l;
        }
    sum16_n<kFQT * 2>(l16);
    if (lc == 0) {
#pragma unroll
        for (int tq = 0; tq < kFQT; ++tq)
#pragma unroll
            for (int r = 0; r < 2; ++r) wml[wv][8 * tq + 2 * lg + r] = make_float2(m16[tq][r], l16[2 * tq + r]);
    }
    lds_barrier();
    if (tid < kFQT * 8) {
        float M = wml[0][tid].x;
#pragma unroll
        for (int v = 1; v < kFNT / 64; ++v) M = fmaxf(M, wml[v][tid].x);
        float L = 0.f;
#pragma unroll
        for (int v = 0; v < kFNT / 64; ++v) L += wml[v][tid].y * fast_exp2(wml[v][tid].x - M);
        rowf[tid] = make_float2(M, lo + tid < P ? 1.0f / L : 0.f);
    }
    lds_barrier();
    // a weight is s * 2^(m16 - M) / L: one factor per (lane, row)
    float f[kFQT][2];
#pragma unroll
    for (int tq = 0; tq < kFQT; ++tq)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const float2 rf = rowf[8 * tq + 2 * lg + r];
            f[tq][r] = fast_exp2(m16[tq][r] - rf.x) * rf.y;
        }
    // votes: per key, over the lane's rows (fp32 per query tile, fp64 across
    // tiles), then over the four lane groups
#pragma unroll
    for (int x = 0; x < kFKT; ++x) {
        double acc = 0.0;
#pragma unroll
        for (int tq = 0; tq < kFQT; ++tq) acc += (double)(s[x][tq][0] * f[tq][0] + s[x][tq][1] * f[tq][1]);
        acc = xrow_add(acc, false);
        acc = xrow_add(acc, true);
        const int key = key0 + 16 * x + lc;
        if (lg == 0 && x < nt && key < P) {
            a.votes[(size_t)(off + key) * a.Hq + hq] = acc;
            if (key < lo) stage[key] = acc;
        }
    }
    lds_barrier();
    snap_head_small<kFNT, kFusedP / kFNT>(a, lo, stage, bits, s_sel);
    if (a.G == 1) {
        snap_finish<kFNT>(a, unit, P, lo, bits, s_scan);
    } else {  // the head's prefix bits; snapkv_union_kernel ORs the group's and adds the window
        unsigned* hb = a.hbits + ((size_t)unit * a.G + g) * a.bits_words;
        for (int i = tid; i < (lo + 31) / 32; i += kFNT) hb[i] = bits[i];
    }
}

// Scratch of h2o_snapkv_select_noalloc, for callers that cannot allocate:
// every device the library runs on holds its own copy of this array until the
// process ends.  In host code its name is only a stand-in for the symbol; the
// device address of the current device's copy comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

}  // namespace

hipError_t noalloc_scratch(char** ptr)
{
    static std::mutex mu;
    static char* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {  // first call on this device, with it current
        void* p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        addr[dev] = static_cast<char*>(p);
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// G > 1: the union of each unit's per-head bitmaps (hbits), the window and the
// kept list (snapkv_union_kernel; dynamic LDS: the bitmap).
static hipError_t launch_snap_union(const SnapArgs& a, hipStream_t st)
{
    static DynLdsLimit lim;
    const size_t dyn = (size_t)a.bits_words * 4;
    hipError_t e = lim.allow((const void*)snapkv_union_kernel, dyn);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(snapkv_union_kernel, dim3((unsigned)(a.B * a.Hkv)), dim3(kSNT), dyn, st, a);
    return hipGetLastError();
}

hipError_t launch_snapkv(const SnapArgs& a, int max_p, hipStream_t st)
{
    if (max_p <= 0) return hipSuccess;
    hipError_t e = hipSuccess;
    int max_pp = 0;
    for (int i = 0; i < a.B; ++i) max_pp = std::max(max_pp, a.seq_p[i] - a.seq_w[i]);
    // prefixes up to kSnapStage are pooled inside the selection; the pooling
    // kernel serves the longer ones
    if (max_pp > kSnapStage) {
        const long long cells = (long long)max_p * a.Hq;
        hipLaunchKernelGGL(snapkv_pool_kernel, dim3((unsigned)((cells + 255) / 256), a.B), dim3(256), 0, st, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // LDS: the bitmap (a.bits_words words), then the staged votes of prefixes up to kSnapStage
    SnapArgs b = a;
    b.stage_n = std::min(max_pp, kSnapStage);
    const size_t dyn = (size_t)b.bits_words * 4 + (size_t)b.stage_n * 8;
    // above the default 48 KB of dynamic LDS the kernel's limit is raised on
    // the current device first (only prompts beyond ~130k positions need it)
    static DynLdsLimit lim_sel, lim_head;
    const unsigned units = (unsigned)(a.B * a.Hkv);
    if (a.G == 1) {
        if ((e = lim_sel.allow((const void*)snapkv_select_kernel, dyn)) != hipSuccess) return e;
        hipLaunchKernelGGL(snapkv_select_kernel, dim3(units), dim3(kSNT), dyn, st, b);
        return hipGetLastError();
    }
    if ((e = lim_head.allow((const void*)snapkv_head_kernel, dyn)) != hipSuccess) return e;
    hipLaunchKernelGGL(snapkv_head_kernel, dim3(units, (unsigned)a.G), dim3(kSNT), dyn, st, b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_snap_union(b, st);
}

bool snapkv_fused_fits(const SnapArgs& a)
{
    if (a.G < 1 || a.B < 1 || a.B > kMaxArgBatch) return false;
    for (int b = 0; b < a.B; ++b)
        if (a.seq_p[b] > kFusedP || a.seq_w[b] > kFQT * 8) return false;
    return true;
}

hipError_t launch_snapkv_fused(const ColsumArgs& ca, const SnapArgs& sa, double* votes, hipStream_t st)
{
    if (!snapkv_fused_fits(sa) || ca.G != sa.G || ca.B != sa.B || !votes || (sa.G > 1 && !sa.hbits))
        return hipErrorInvalidValue;
    SnapFusedArgs f{};
    f.q = ca.q;
    f.k = ca.k;
    f.qscale = ca.qscale;
    f.Hq = sa.Hq;
    f.Hkv = sa.Hkv;
    f.G = sa.G;
    f.units = sa.B * sa.Hkv;
    f.pool_r = sa.pool_r;
    f.keep = sa.keep;
    f.cap = sa.cap;
    f.votes = votes;
    f.kept = sa.kept;
    f.count = sa.count;
    f.hbits = sa.hbits;
    f.bits_words = sa.bits_words;
    for (int b = 0; b < sa.B; ++b) {
        f.seq_p[b] = sa.seq_p[b];
        f.seq_w[b] = sa.seq_w[b];
        f.seq_off[b] = sa.seq_off[b];
    }
    // G = 1: groups of 64 units; else groups of 8 units, each 8 G workgroups
    const unsigned wgs = sa.G == 1 ? (unsigned)((f.units + 63) / 64) * 64u
                                   : (unsigned)((f.units + 7) / 8) * 8u * (unsigned)sa.G;
    hipLaunchKernelGGL(snapkv_fused_kernel, dim3(wgs), dim3(kFNT), 0, st, f);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || sa.G == 1) return e;
    return launch_snap_union(sa, st);
}

hipError_t launch_colsum(const ColsumArgs& a, int max_p, hipStream_t st)
{
    if (max_p <= 0) return hipSuccess;
    switch (a.G) {
    case 1: return launch_colsum_g<1>(a, max_p, st);
    case 2: return launch_colsum_g<2>(a, max_p, st);
    case 4: return launch_colsum_g<4>(a, max_p, st);
    case 8: return launch_colsum_g<8>(a, max_p, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace h2o
