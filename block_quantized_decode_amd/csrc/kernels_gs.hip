// kernels_gs.hip -- the split-K decode matvec for the 4-bit exported formats
// whose scale covers several 32-element units (gfx950):
//   * 128-element blocks with a zero point, 4-bit codes ("ONNX Runtime" page,
//     section 3 "Match real exports -- BlkLen=128 CompInt8", section 4
//     "SQ8Bit"): 4 units per scale;
//   * K-quant super-blocks of 8 sub-blocks with 6-bit sub-block scales and
//     minima ("SKaiNET-native-kernels" page, section "Proving an
//     optimization is safe before writing it"): 8 units per scale.
// What is computed is that of kernels_zp.hip and kernels_q4k.hip (the same
// integer identities, the same activation quantization, bit for bit); only
// the work layout differs.  The row-streaming kernels there read whole rows
// per lane group; this kernel reads them the way the fused Q4_0 / Q8_0
// matvec does, where that was measured faster for 4-bit codes: with 8
// wavefronts on many rows of 4096 and more elements (the Llama-7B FFN
// shapes), with 4 on fewer rows (launch rule at the end of this file).  For
// 8-bit zero-point codes the row streaming stays ahead (11.6 against 11.9 us
// on W_up 11008 x 4096) and keeps them.
//
// One workgroup of WPB wavefronts per compute unit owns a run of rw rows
// (a multiple of 4); its wavefronts split K: wavefront w owns units
// [w S, w S + S) of every row (a unit = 32 elements = 16 code bytes; S a
// multiple of the units per scale, G, so no scale block
// straddles two wavefronts).  A wavefront quantizes only its own slice of
// the activation (a half-wavefront per 128-element block, a wavefront per
// 256-element block), keeps the quants of the units it will multiply in
// registers for the whole launch, and streams passes of 4 rows: lane l takes
// row l / 16 of the pass and units l % 16 + 16 k (k < NC) of the slice, so
// 16 lanes read 16 consecutive units of a row and the G lanes of one scale
// block are adjacent.  A ring of D passes is in flight (D - 1 issued ahead
// of the one being computed; the first before the activation work).
//
// Per unit a lane forms the exact int32 dot of its codes with the activation
// quants (v_dot4 on the codes masked into low and high nibbles), the G lanes
// of the block add
// theirs by DPP (exact), and one lane of the G -- lane g of the group for
// unit k = g, the lane that loaded that block's scale -- applies the scales
// in fp32 as the oracle does:
//   zero point: sumi = P - zp * sum(q),  t = ((float)sumi * dw) * dx
//   K-quant:    S1 = sum over the 8 units of sc * dot, S2 = sum of mn * sum(q),
//               t = ((float)S1 * d - (float)S2 * dmin) * dx.
// The row's 16 lanes are added by DPP, the wavefronts' slice sums in LDS in
// wavefront order, so repeated calls give identical bits.
//
// Loads use raw buffer descriptors covering this workgroup's rows only; every
// variable part of an address is in the range-checked offset, so rows past
// r1, units past the slice and passes past the last read zeros.
#include "count.h"
#include "launch.h"
#include "rowstream.h"

namespace qmv {
namespace {

using rs::v4i;

#ifndef QMV_GS_D  // ring depth (passes in registers)
#define QMV_GS_D 4
#endif
#ifndef QMV_GS_D3_NC  // K-quant units per lane from which the ring is 3 deep
#define QMV_GS_D3_NC 2
#endif
#ifndef QMV_GS_D0  // passes issued before the activation work
#define QMV_GS_D0 1
#endif
#ifndef QMV_GS_TAIL  // 1: the last passes specialised on their count; 0: tested per pass
#define QMV_GS_TAIL 1
#endif

constexpr int kOff = 0x40000000;  // an offset beyond every range here, with room for pass strides
constexpr int kNTg = 2;           // non-temporal: weights are read once

enum { kGsZp4 = 1, kGsQ4k = 2 };

template <int FMT>
struct GsFmt {
    static constexpr int UB = 16;                        // code bytes per unit
    static constexpr int G = FMT == kGsQ4k ? 8 : 4;      // units per scale block
    static constexpr int BLK = 32 * G;                   // elements per scale block
};

// One pass of weights in a lane's registers.
template <int FMT, int NC>
struct GsPass {
    static constexpr bool KQ = FMT == kGsQ4k;
    v4i w[NC];
    int sc[KQ ? NC : 1], mn[KQ ? NC : 1];  // K-quant: this lane's units' scale and minimum
};

// The block scales of one ring turn (D passes, NC units per lane each: the
// D * NC (pass, unit) pairs p = d * NC + k of a lane's scale block).  Lane g
// of the block's G lanes holds those of pairs m * G + g (m < MR) and applies
// them itself, so one load instruction serves G pairs rather than one.
template <int FMT, int MR>
struct GsMeta {
    static constexpr bool KQ = FMT == kGsQ4k;
    float s0[MR];              // dw (zero point) or d (K-quant)
    float s1[KQ ? MR : 1];     // K-quant: dmin
    int z[KQ ? 1 : MR];        // zero point: zp
};

// Exact int32 dot of one unit's 16 code bytes with its activation quants:
// the low nibbles of dword k against xa[k], the high ones against xb[k]
// (zero point: byte i holds element 2i low and 2i + 1 high, so xa holds the
// even elements of each 8 and xb the odd ones; K-quant: byte i holds
// element i low and i + 16 high, so xa and xb are the unit's two halves --
// see the prologue).
__device__ __forceinline__ int unit_dot(v4i w, v4i xa, v4i xb) {
    int p = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int lo = w[k] & 0x0F0F0F0F, hi = (w[k] >> 4) & 0x0F0F0F0F;
        p = __builtin_amdgcn_sdot4(lo, xa[k], p, false);
        p = __builtin_amdgcn_sdot4(hi, xb[k], p, false);
    }
    return p;
}

// The Q8_0 rule (Legacy-ISA ML Inference Runtime -- Design Spec, section 4
// "Q8 quantization", section 5 rounding bullet) on a block held by L lanes
// (16 or 32, aligned), 8 elements each: amax exact (non-negative floats order
// like their bit patterns; a DPP maximum within rows of 16 lanes, then
// across the two rows of a 32-lane block), d = amax / 127 and id = 127 /
// amax correctly rounded, each element rounded by rs::q8_round; qsum = the
// block's sum of quants, in every lane of the block.
template <int L>
__device__ __forceinline__ void quant8(const float4 &a, const float4 &b, int (&q)[8], float &d, int &qsum) {
    const float m = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                          fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
    const auto imax = [](int u, int v) { return max(u, v); };
    const auto isum = [](int u, int v) { return u + v; };
    int mi = rs::row16_reduce(__float_as_int(m), imax);
    if constexpr (L == 32) mi = max(mi, __shfl_xor(mi, 16));
    const float amax = __int_as_float(mi);
    d = amax / 127.0f;
    const float id = amax != 0.0f ? 127.0f / amax : 0.0f;
    q[0] = rs::q8_round(a.x, id);
    q[1] = rs::q8_round(a.y, id);
    q[2] = rs::q8_round(a.z, id);
    q[3] = rs::q8_round(a.w, id);
    q[4] = rs::q8_round(b.x, id);
    q[5] = rs::q8_round(b.y, id);
    q[6] = rs::q8_round(b.z, id);
    q[7] = rs::q8_round(b.w, id);
    int s = rs::row16_reduce(((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7])), isum);
    if constexpr (L == 32) s += __shfl_xor(s, 16);
    qsum = s;
}

template <int G>
__device__ __forceinline__ int group_isum(int v) {
    v += rs::dppi<rs::kX1>(v);
    v += rs::dppi<rs::kX2>(v);
    if constexpr (G == 8) v += rs::dppi<rs::kM8>(v);
    return v;
}

template <int FMT, int NC, int D, int WPB>
__global__ void __launch_bounds__(64 * WPB)
k_gs(float *__restrict__ y, const uint8_t *__restrict__ wq, const float *__restrict__ ws0,
     const float *__restrict__ ws1, const uint8_t *__restrict__ wzp, const uint8_t *__restrict__ wsc,
     const uint8_t *__restrict__ wmn, int32_t zdef, int32_t rows, int32_t K, const float *__restrict__ x,
     int8_t *__restrict__ xq_out, float *__restrict__ xd_out, int32_t r0, int32_t r1, int32_t rw, int32_t S) {
    using F = GsFmt<FMT>;
    constexpr bool KQ = FMT == kGsQ4k;
    constexpr int T = 16, PASS = 4, G = F::G, UB = F::UB, BLK = F::BLK;
    constexpr int SMAX = T * NC;          // units of a slice at most
    constexpr int BMAX = SMAX / G;        // scale blocks of a slice at most
    static_assert(NC >= 1 && NC <= 4 && NC <= G, "units per lane per pass");
    __shared__ v4i s_xa[WPB][SMAX], s_xb[WPB][SMAX];  // activation quants of each unit, two halves
    __shared__ int s_qs[KQ ? WPB : 1][KQ ? SMAX : 1];  // K-quant: sum of each unit's quants
    __shared__ float s_dx[WPB][BMAX];                 // activation scale per block
    __shared__ int s_qb[WPB][BMAX];                   // zero point: sum of each block's quants
    extern __shared__ float s_red[];                  // [WPB][rw] slice sums

    const int nu = K >> 5;                // units per row
    const int nbk = K / BLK;              // scale blocks per row
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int u0 = min(wid * S, nu);
    const int ns = min(S, nu - u0);       // units of this wavefront's slice
    const int nbw = ns / G;               // its scale blocks
    const int g0 = r0 + blockIdx.x * rw;
    const int rows_here = min(r1, g0 + rw) - g0;
    const int npass = (rows_here + PASS - 1) / PASS;
    const int row_bytes = nu * UB;

    // 1. the activation loads of this slice: round i, lane l holds elements
    //    8 (l % LPB) .. + 7 of block BPR i + l / LPB (LPB = 16 lanes per
    //    128-element block, 32 per 256-element block; BPR blocks per round,
    //    NC rounds cover the largest slice)
    constexpr int LPB = BLK / 8, BPR = 64 / LPB;
    const __amdgpu_buffer_rsrc_t rx = rs::rsrc(x, (int64_t)K * 4);
    float4 xv[NC][2];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int bl = BPR * i + lane / LPB;
        const int o = bl < nbw ? (u0 * 32 + bl * BLK + 8 * (lane % LPB)) * 4 : kOff;
        xv[i][0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 0));
        xv[i][1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rx, o + 16, 0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);  // the activation requests go out first

    // 2. weight offsets of pass 0 and the first pass in flight
    const int prow = lane / T;
    const int gl = lane % G;              // position in the scale block (the lane of its pairs g = gl)
    const int64_t rb = (int64_t)g0;
    const __amdgpu_buffer_rsrc_t rq = rs::rsrc(wq + rb * row_bytes, (int64_t)rows_here * row_bytes);
    const __amdgpu_buffer_rsrc_t r0s = rs::rsrc(ws0 + rb * nbk, (int64_t)rows_here * nbk * 4);
    const __amdgpu_buffer_rsrc_t r1s = rs::rsrc(KQ ? ws1 + rb * nbk : ws0, KQ ? (int64_t)rows_here * nbk * 4 : 0);
    const __amdgpu_buffer_rsrc_t rz = rs::rsrc(!KQ && wzp != nullptr ? wzp + rb * nbk : wq,
                                               !KQ && wzp != nullptr ? (int64_t)rows_here * nbk : 0);
    const __amdgpu_buffer_rsrc_t rsc = rs::rsrc(KQ ? wsc + rb * nu : wq, KQ ? (int64_t)rows_here * nu : 0);
    const __amdgpu_buffer_rsrc_t rmn = rs::rsrc(KQ ? wmn + rb * nu : wq, KQ ? (int64_t)rows_here * nu : 0);
    int oq[NC], ou[NC];
#pragma unroll
    for (int k = 0; k < NC; ++k) {
        const int c = lane % T + T * k;
        const bool ok = c < ns;
        oq[k] = ok ? prow * row_bytes + (u0 + c) * UB : kOff;
        ou[k] = ok ? prow * nu + u0 + c : kOff;
    }
    const int pq = PASS * row_bytes, pu = PASS * nu;  // strides of one pass
    const int zbase = wzp != nullptr ? 0 : zdef;
    auto load = [&](GsPass<FMT, NC> &p, int j) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int a = oq[k] + j * pq;
            p.w[k] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rq, a, 0, kNTg));
            if constexpr (KQ) {
                p.sc[k] = (int)__builtin_amdgcn_raw_buffer_load_b8(rsc, ou[k] + j * pu, 0, 0);
                p.mn[k] = (int)__builtin_amdgcn_raw_buffer_load_b8(rmn, ou[k] + j * pu, 0, 0);
            }
        }
    };
    // scales of ring turn `it` (passes it * D .. it * D + D - 1): pair
    // p = m * G + gl is pass d = p / NC, unit k = p % NC; its block is the
    // group's unit base plus 16 k
    constexpr int MR = (D * NC + G - 1) / G;
    auto load_meta = [&](GsMeta<FMT, MR> &mt, int it) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const int pr = m * G + gl, d = pr / NC, k = pr % NC;
            const int c = lane % T - gl + T * k;  // the block's first unit in the slice
            const int row = (it * D + d) * PASS + prow;
            const int mi = row * nbk + (u0 + c) / G;  // rows past the range fall outside it
            const bool ok = pr < D * NC && c < ns;
            mt.s0[m] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r0s, ok ? 4 * mi : kOff, 0, 0));
            if constexpr (KQ) {
                mt.s1[m] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r1s, ok ? 4 * mi : kOff, 0, 0));
            } else {
                // (issued and used unconditionally -- without zero points the
                // range is 0, the load reads 0 and zbase is the default -- so
                // that no branch blurs the compiler's count of loads in flight)
                mt.z[m] = (int)__builtin_amdgcn_raw_buffer_load_b8(rz, ok ? mi : kOff, 0, 0) + zbase;
            }
        }
    };
    constexpr int D0 = QMV_GS_D0 < D - 1 ? QMV_GS_D0 : D - 1;
    GsPass<FMT, NC> ring[D];
    GsMeta<FMT, MR> mcur, mnxt;
    load_meta(mnxt, 0);
#pragma unroll
    for (int d = 0; d < D0; ++d) load(ring[d], d);
    __builtin_amdgcn_sched_barrier(0);

    // 3. quantize the slice (the Q8_0 rule per block) into this wavefront's
    //    LDS region: unit-major, 32 bytes per unit -- natural order, except
    //    for 4-bit zero-point codes: bytes 0..15 hold the even elements of
    //    each 8 (elements 8 k, 8 k + 2, 8 k + 4, 8 k + 6 in dword k), bytes
    //    16..31 the odd ones, so that a weight dword's low and high nibbles
    //    meet theirs in one v_dot4 each
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int bl = BPR * i + lane / LPB;
        const int e = 8 * (lane % LPB);  // element in the block
        int q[8], qs;
        float d;
        quant8<LPB>(xv[i][0], xv[i][1], q, d, qs);
        if (bl < nbw) {
            const int ul = bl * G + (e >> 5);   // unit in the slice
            const int pos = e & 31;             // element in the unit: 0, 8, 16 or 24
            int8_t *ua = reinterpret_cast<int8_t *>(&s_xa[wid][ul]);
            int8_t *ub = reinterpret_cast<int8_t *>(&s_xb[wid][ul]);
            const int lo = (q[0] & 0xFF) | ((q[1] & 0xFF) << 8) | ((q[2] & 0xFF) << 16) | (q[3] << 24);
            const int hi = (q[4] & 0xFF) | ((q[5] & 0xFF) << 8) | ((q[6] & 0xFF) << 16) | (q[7] << 24);
            if constexpr (FMT == kGsZp4) {
                const int ev = (q[0] & 0xFF) | ((q[2] & 0xFF) << 8) | ((q[4] & 0xFF) << 16) | (q[6] << 24);
                const int od = (q[1] & 0xFF) | ((q[3] & 0xFF) << 8) | ((q[5] & 0xFF) << 16) | (q[7] << 24);
                reinterpret_cast<int *>(ua)[pos >> 3] = ev;
                reinterpret_cast<int *>(ub)[pos >> 3] = od;
            } else {
                *reinterpret_cast<int2 *>(pos < 16 ? ua + pos : ub + pos - 16) = make_int2(lo, hi);
            }
            if constexpr (KQ) {  // the unit's sum of quants: its 4 lanes
                int us = ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
                us += rs::dppi<rs::kX1>(us);
                us += rs::dppi<rs::kX2>(us);
                if ((lane & 3) == 0) s_qs[wid][ul] = us;
            }
            const bool lead = lane % LPB == 0;
            if (lead) {
                s_dx[wid][bl] = d;
                s_qb[wid][bl] = qs;
            }
            if (xq_out != nullptr && blockIdx.x == 0) {  // optional copy of the quantized activation
                const int ge = u0 * 32 + bl * BLK + e;
                *reinterpret_cast<int2 *>(xq_out + ge) = make_int2(lo, hi);
                if (lead) xd_out[ge / BLK] = d;
            }
        }
    }
    // LDS operations of one wavefront complete in order
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    v4i xa[NC], xb[NC];
    int qsu[KQ ? NC : 1];
#pragma unroll
    for (int k = 0; k < NC; ++k) {
        const int c = lane % T + T * k;
        const bool ok = c < ns;
        const int cc = ok ? c : 0;
        xa[k] = ok ? s_xa[wid][cc] : (v4i){0, 0, 0, 0};
        xb[k] = ok ? s_xb[wid][cc] : (v4i){0, 0, 0, 0};
        if constexpr (KQ) qsu[k] = ok ? s_qs[wid][cc] : 0;
    }
    float dxm[NC];  // the activation scale and quant sum of each unit's scale block
    int qbm[NC];
#pragma unroll
    for (int k = 0; k < NC; ++k) {
        const int c = lane % T + T * k;
        const bool ok = c < ns;
        dxm[k] = ok ? s_dx[wid][ok ? c / G : 0] : 0.0f;
        qbm[k] = ok ? s_qb[wid][ok ? c / G : 0] : 0;
    }

    // the rest of the first D - 1 passes
#pragma unroll
    for (int d = D0; d < D - 1; ++d) load(ring[d], d);

    // 4. passes: the loads of pass j + D - 1 in flight while pass j is computed.
    //    Turns whose loads all fall inside the range run unguarded (so the
    //    compiler's waits stay exact); the last one or two turns load and
    //    compute only passes that exist (measured: loads past the range,
    //    though they read nothing, cost time at the end of the launch).
    auto compute = [&](const GsPass<FMT, NC> &p, const GsMeta<FMT, MR> &mt, int j, int d)
        __attribute__((always_inline)) {
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int pr = d * NC + k, m = pr / G;  // this pair's scales: lane pr % G, slot m
            const int dot = unit_dot(p.w[k], xa[k], xb[k]);
            if constexpr (KQ) {
                const int s1 = group_isum<G>(dot * p.sc[k]);
                const int s2 = group_isum<G>(p.mn[k] * qsu[k]);
                if (gl == pr % G) {
#pragma clang fp contract(off)
                    float t = (float)s1 * mt.s0[m] - (float)s2 * mt.s1[m];
                    acc = acc + t * dxm[k];
                }
            } else {
                const int ps = group_isum<G>(dot);
                if (gl == pr % G) {
#pragma clang fp contract(off)
                    const int sumi = ps - mt.z[m] * qbm[k];
                    float t = (float)sumi * mt.s0[m];
                    acc = acc + t * dxm[k];
                }
            }
        }
        const float t = rs::group_sum<T>(acc);
        const int r = j * PASS + prow;
        if (lane % T == 0 && r < rows_here) s_red[wid * rw + r] = t;
    };
    int it = 0;
    for (; (it + 2) * D - 2 < npass; ++it) {
        mcur = mnxt;  // (issued with the turn's first pass)
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int j = it * D + d;
            load(ring[(d + D - 1) % D], j + D - 1);
            if (d == 1) load_meta(mnxt, it + 1);  // with the next turn's first pass
            compute(ring[d], mcur, j, d);
        }
    }
    // The remaining R passes (1 .. 2 D - 2, the first D - 1 of them in the
    // ring; at most two turns' scales): as code specialised on R, which keeps
    // the waits for the ring exact, where that measured faster (8 wavefronts,
    // and 4-bit zero-point codes); else one or two turns testing each pass.
    if constexpr (QMV_GS_TAIL && (WPB >= 8 || FMT == kGsZp4)) {
        with_count<1, 2 * D - 2>(npass - it * D, [&](auto rc) __attribute__((always_inline)) {
            constexpr int R = decltype(rc)::value;
#pragma unroll
            for (int q = 0; q < R; ++q) {
                if (q % D == 0) mcur = mnxt;
                if (q + D - 1 < R) load(ring[(q + D - 1) % D], it * D + q + D - 1);
                if (q == 1 && R > D) load_meta(mnxt, it + 1);
                compute(ring[q % D], mcur, it * D + q, q % D);
            }
        });
    } else {
        for (; it * D < npass; ++it) {
            mcur = mnxt;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int j = it * D + d;
                if (j < npass) {  // (wave-uniform)
                    if (j + D - 1 < npass) load(ring[(d + D - 1) % D], j + D - 1);
                    if (d == 1 && (it + 1) * D < npass) load_meta(mnxt, it + 1);
                    compute(ring[d], mcur, j, d);
                }
            }
        }
    }

    // 5. the wavefronts' slice sums of each row, in wavefront order
    __syncthreads();
    for (int r = threadIdx.x; r < rows_here; r += 64 * WPB) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WPB; ++w) s += s_red[w * rw + r];
        y[g0 + r] = s;
    }
}

constexpr int kGsWpb = 8;
#ifndef QMV_GS_W2  // 1: rows of 257 .. 384 units on 9 .. 12 wavefronts of 2 units per lane (gs_form)
#define QMV_GS_W2 1
#endif
constexpr int kGsRwCap = 512;  // rows per workgroup: slice sums [WPB][rw] in LDS

template <int FMT, int NC, int W>
hipError_t launch_gs_t(float *y, const uint8_t *wq, const float *s0, const float *s1, const uint8_t *zp,
                       const uint8_t *sc, const uint8_t *mn, int zdef, int rows, int K, const float *x,
                       int8_t *xq_out, float *xd_out, int r0, int r1, int S, int num_cu, hipStream_t s,
                       const char **name) {
    // 3 passes in flight for K-quant slices of several units per lane (each
    // unit of a pass also loads its scale and minimum bytes), 4 otherwise:
    // measured K-quant Llama W_down 8.03 -> 7.69 us, TinyLlama W_down
    // 4.49 -> 4.37 us; 4-bit zero points kept 4 (equal or 0.4% slower with 3)
    constexpr int D = (FMT == kGsQ4k && NC >= QMV_GS_D3_NC) ? 3 : QMV_GS_D;
    auto kern = k_gs<FMT, NC, D, W>;
    static const std::string kname =
        variant_name("gs_%s_n%d_d%d_w%d", FMT == kGsZp4 ? "zp4" : "q4k", NC, D, W);
    const int nrows = r1 - r0;
    int rw = ((nrows + num_cu - 1) / num_cu + 3) / 4 * 4;
    if (rw > kGsRwCap) rw = kGsRwCap;
    const int grid = (nrows + rw - 1) / rw;
    const size_t lds = (size_t)W * rw * 4;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * W), lds, s, y, wq, s0, s1, zp, sc, mn, zdef, rows, K, x,
                       xq_out, xd_out, r0, r1, rw, S);
    *name = kname.c_str();
    return hipGetLastError();
}

// Slice of units per wavefront (a multiple of G) for W wavefronts per
// workgroup, or 0 where that form does not take the shape: fewer than 16
// units per wavefront, or slices past 64 units.
int gs_slice(int K, int G, int W) {
    const int nu = K / 32;
    const int S = (nu / G + W - 1) / W * G;
    return (nu < 16 * W || S > 64) ? 0 : S;
}

template <int FMT, int W>
hipError_t launch_gs_f(float *y, const uint8_t *wq, const float *s0, const float *s1, const uint8_t *zp,
                       const uint8_t *sc, const uint8_t *mn, int zdef, int rows, int K, const float *x,
                       int8_t *xq_out, float *xd_out, int r0, int r1, int S, int num_cu, hipStream_t s,
                       const char **name) {
    switch ((S + 15) / 16) {
        case 1: return launch_gs_t<FMT, 1, W>(y, wq, s0, s1, zp, sc, mn, zdef, rows, K, x, xq_out, xd_out, r0, r1,
                                              S, num_cu, s, name);
        case 2: return launch_gs_t<FMT, 2, W>(y, wq, s0, s1, zp, sc, mn, zdef, rows, K, x, xq_out, xd_out, r0, r1,
                                              S, num_cu, s, name);
        case 3: return launch_gs_t<FMT, 3, W>(y, wq, s0, s1, zp, sc, mn, zdef, rows, K, x, xq_out, xd_out, r0, r1,
                                              S, num_cu, s, name);
        default: return launch_gs_t<FMT, 4, W>(y, wq, s0, s1, zp, sc, mn, zdef, rows, K, x, xq_out, xd_out, r0, r1,
                                               S, num_cu, s, name);
    }
}

}  // namespace

// Which form takes a shape (measured on the MI355X, weights streamed from
// HBM): 8 wavefronts for at least 16 rows (4 passes of 4) per compute unit;
// below that, 4 wavefronts where their slices fit (K-quant 256 x 2048
// 3.35 -> 2.94 us, 2048 x 2048 3.46 -> 3.32 us, 2048 x 5632 5.57 -> 4.52 us;
// 4-bit zero point 896 x 4864 4.39 -> 3.90 us, all against the
// row-streaming kernel); otherwise the row-streaming kernels, which stay
// ahead with 8 wavefronts on fewer rows and with 4 on more (K-quant
// 5632 x 2048 4.91 against 5.07 us, Llama-7B W_up 7.3 against 7.9 us).
//
// With 8 wavefronts, rows of 257 .. 384 units take 3 units per lane; where
// nu / 32 wavefronts (9 .. 12) of 2 units per lane leave at most 5% of the
// slots empty, those are taken instead (a load instruction costs the same
// whether its lanes read or fall past the slice; the fused Q4_0 matvec
// measured the same split faster on every such K).
template <int FMT>
int gs_form(int K, int nrows, int num_cu, int *S) {
    constexpr int G = FMT == kGsZp4 ? 4 : 8;
    if (nrows >= 16 * num_cu) {
        *S = gs_slice(K, G, kGsWpb);
#if QMV_GS_W2
        const int nu = K / 32, w2 = (nu + 31) / 32;
        if (*S > 32 && w2 >= 9 && w2 <= 12 && 20 * nu >= 19 * 32 * w2 && gs_slice(K, G, w2) == 32) {
            *S = 32;
            return w2;
        }
#endif
        return *S ? kGsWpb : 0;
    }
    *S = gs_slice(K, G, 4);
    return *S ? 4 : 0;
}

hipError_t launch_gs_zp(const ZpArgs &a, int num_cu, hipStream_t s, const char **name) {
    if (a.bits != 4 || a.K % 128 != 0 || a.r1 - a.r0 < 1) return hipErrorNotSupported;
    int S = 0;
    switch (gs_form<kGsZp4>(a.K, a.r1 - a.r0, num_cu, &S)) {
        case 4:
            return launch_gs_f<kGsZp4, 4>(a.y, a.wq, a.wd, nullptr, a.wzp, nullptr, nullptr, 8, a.rows, a.K, a.x,
                                          a.xq_out, a.xd_out, a.r0, a.r1, S, num_cu, s, name);
#if QMV_GS_W2
        case 9: return launch_gs_t<kGsZp4, 2, 9>(a.y, a.wq, a.wd, nullptr, a.wzp, nullptr, nullptr, 8, a.rows, a.K, a.x, a.xq_out, a.xd_out, a.r0, a.r1, S, num_cu, s, name);
        case 10: return launch_gs_t<kGsZp4, 2, 10>(a.y, a.wq, a.wd, nullptr, a.wzp, nullptr, nullptr, 8, a.rows, a.K, a.x, a.xq_out, a.xd_out, a.r0, a.r1, S, num_cu, s, name);
        case 11: return launch_gs_t<kGsZp4, 2, 11>(a.y, a.wq, a.wd, nullptr, a.wzp, nullptr, nullptr, 8, a.rows, a.K, a.x, a.xq_out, a.xd_out, a.r0, a.r1, S, num_cu, s, name);
        case 12: return launch_gs_t<kGsZp4, 2, 12>(a.y, a.wq, a.wd, nullptr, a.wzp, nullptr, nullptr, 8, a.rows, a.K, a.x, a.xq_out, a.xd_out, a.r0, a.r1, S, num_cu, s, name);
#endif
        case kGsWpb:
            return launch_gs_f<kGsZp4, kGsWpb>(a.y, a.wq, a.wd, nullptr, a.wzp, nullptr, nullptr, 8, a.rows, a.K,
                                               a.x, a.xq_out, a.xd_out, a.r0, a.r1, S, num_cu, s, name);
        default: return hipErrorNotSupported;
    }
}

hipError_t launch_gs_q4k(const Q4kArgs &a, int num_cu, hipStream_t s, const char **name) {
    if (a.K % 256 != 0 || a.r1 - a.r0 < 1) return hipErrorNotSupported;
    int S = 0;
    switch (gs_form<kGsQ4k>(a.K, a.r1 - a.r0, num_cu, &S)) {
        case 4:
            return launch_gs_f<kGsQ4k, 4>(a.y, a.wq, a.d, a.dmin, nullptr, a.sc, a.mn, 0, a.rows, a.K, a.x,
                                          a.xq_out, a.xd_out, a.r0, a.r1, S, num_cu, s, name);
#if QMV_GS_W2
        case 9: return launch_gs_t<kGsQ4k, 2, 9>(a.y, a.wq, a.d, a.dmin, nullptr, a.sc, a.mn, 0, a.rows, a.K, a.x, a.xq_out, a.xd_out, a.r0, a.r1, S, num_cu, s, name);
        case 10: return launch_gs_t<kGsQ4k, 2, 10>(a.y, a.wq, a.d, a.dmin, nullptr, a.sc, a.mn, 0, a.rows, a.K, a.x, a.xq_out, a.xd_out, a.r0, a.r1, S, num_cu, s, name);
        case 11: return launch_gs_t<kGsQ4k, 2, 11>(a.y, a.wq, a.d, a.dmin, nullptr, a.sc, a.mn, 0, a.rows, a.K, a.x, a.xq_out, a.xd_out, a.r0, a.r1, S, num_cu, s, name);
        case 12: return launch_gs_t<kGsQ4k, 2, 12>(a.y, a.wq, a.d, a.dmin, nullptr, a.sc, a.mn, 0, a.rows, a.K, a.x, a.xq_out, a.xd_out, a.r0, a.r1, S, num_cu, s, name);
#endif
        case kGsWpb:
            return launch_gs_f<kGsQ4k, kGsWpb>(a.y, a.wq, a.d, a.dmin, nullptr, a.sc, a.mn, 0, a.rows, a.K, a.x,
                                               a.xq_out, a.xd_out, a.r0, a.r1, S, num_cu, s, name);
        default: return hipErrorNotSupported;
    }
}

}  // namespace qmv
