// kernels_fx.hip -- the split-K streaming product for a few activation rows:
// the decode matvec with the activation quantized inside the kernel (M = 1,
// float32 x; optionally normalized first, rmsnorm, or formed from the FFN
// gate silu(g) * u) and the same product on pre-quantized Q8_0 activation
// rows (M = 1 .. 4), for K / 32 <= 32 and K of 2048 .. 16384.
//
// What is computed (Legacy-ISA ML Inference Runtime -- Design Spec,
// section 4 "Q8 quantization" and "Integer dot per block", section 5
// kernel interface and rounding rule):
//   qx, dx    = Q8_0(x)                     per 32-element block (fused form)
//   y[m, r]   = sum over blocks b of sumi(m, r, b) * dw(r, b) * dx(m, b),
//   sumi      = exact int32 dot of the 32 weight quants and qx of row m,
// for r in [r0, r1); y is M x rows, row-major.
//
// Layout on the chip.  One workgroup per compute unit owns a contiguous
// range of rows; its wavefronts split K: wavefront w owns blocks
// [w S, w S + S) of every row of the range (S = ceil(K / 32 / waves)).  So a
// wavefront needs only its own slice of the activation rows: it loads that
// slice (4 lanes per block), quantizes it (fused form) or forms its quant
// sums (pre-quantized form) in registers and shares it with its own lanes
// through a private LDS region -- no workgroup barrier stands between the
// activation and the first block dot, and the activation is read once per
// workgroup.  The memory system accepts only a bounded number of
// outstanding loads per compute unit and stalls a wavefront at a load it
// cannot yet accept; so each wavefront first issues its activation loads,
// then only the first D - 1 passes of weights, prepares the activation
// while those are in flight, and then runs a software pipeline over passes:
// issue the loads of pass j + D - 1, then compute pass j, and no loads for
// passes past its last.  A wavefront stalled at a load leaves the vector ALU
// to the others.  Each weight block in registers serves all M activation
// rows.
//
// A pass is 64 / T rows: lane l takes row l / T of the pass and the blocks
// c = l % T + T k (k < NBL) of its wavefront's slice, so each group of T
// lanes reads T consecutive blocks of one row (T * 16 or T * 32 contiguous
// quant bytes).  The T lanes of a row are summed with row-shift DPP adds
// (a fixed order), the wavefronts' slice sums of a row are added in LDS in
// wavefront order, and one lane stores y[m, r]: repeated calls give
// identical bits.  With K / 32 <= 32 every wavefront holds all of K instead
// and takes every waves-th pass of rows, storing whole-row sums directly.
//
// Loads use raw buffer descriptors whose range covers only this
// workgroup's rows, and every variable part of an address is in the
// per-lane offset, which the hardware range-checks: rows past r1, blocks
// past the slice and, for wavefronts of fewer than D - 1 passes, the first
// passes' loads past the last read zeros without touching memory.
#include "count.h"
#include "device_common.h"
#include "launch.h"

namespace qmv {
namespace {

constexpr int kBufFlags = 0x00020000;  // buffer descriptor word 3: raw 32-bit data
constexpr int kNT = 2;                 // non-temporal: weights are read once
constexpr int kOOB = 0x40000000;       // an offset beyond every descriptor range used here

// Tuning (measured on the Llama-7B FFN shapes): barrier between the
// activation and weight requests, one pass of weights issued before the
// quantization, four passes in the ring, one workgroup of 8 wavefronts
// per compute unit (4 for some shapes of one activation row: launch_m;
// 9 - 12 for some longer Q4_0 rows: wide_slices).
#ifndef QMV_FX_XBAR
#define QMV_FX_XBAR 1
#endif
#ifndef QMV_FX_D0
#define QMV_FX_D0 1
#endif
#ifndef QMV_FX_WPB
#define QMV_FX_WPB 8
#endif
#ifndef QMV_FX_D
#define QMV_FX_D 4
#endif
#ifndef QMV_FX_W2  // 1: one float32 row of Q4_0 with 257 .. 384 blocks on 9 .. 12 wavefronts (launch_m_w)
#define QMV_FX_W2 1
#endif
#ifndef QMV_FX_D3_NBL  // slices of at least this many blocks per lane take a ring of 3
#define QMV_FX_D3_NBL 2
#endif
#ifndef QMV_FX_WG_PER_CU
#define QMV_FX_WG_PER_CU 1
#endif
// Weight passes issued before the activation transform of the rmsnorm form
// (its workgroup barrier and norm weights lengthen the prologue: 3 passes,
// capped at D - 1, measured 7.6 against 8.1 us for one on Llama-7B W_up)
// and of the FFN-gate form (1 pass measured best on W_down).
#ifndef QMV_FX_D0_RMS
#define QMV_FX_D0_RMS 3
#endif
#ifndef QMV_FX_D0_SILU
#define QMV_FX_D0_SILU 1
#endif
#ifndef QMV_FX_SQ  // one 16-byte scale load per lane and pass (see k_fx)
#define QMV_FX_SQ 1
#endif
#ifndef QMV_MQ_SQ  // the same in k_mq
#define QMV_MQ_SQ 1
#endif
#ifndef QMV_FX_TAIL  // 1: no loads past a wavefront's last pass (see k_fx); 0: whole ring turns
#define QMV_FX_TAIL 1
#endif


__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, kBufFlags);
}

// One pass of weights in registers: NBL blocks of one row per lane.
template <int QT, int NBL>
struct Pass {
    static constexpr int QW = (QT == 8) ? 2 : 1;  // 16-byte words per block
    v4i w[NBL][QW];
    float dw[NBL];
    v4i dq;  // the pass's weight scales, 4 consecutive blocks per lane (see k_fx)
};

// Sum over aligned groups of T lanes (T a power of two, at most 64): an
// inclusive scan by row-shift DPP adds (lanes shifted in from outside a row
// of 16 read 0), then row broadcasts for T = 32 and 64.  The total of each
// group ends up in its last lane.
template <int T>
__device__ __forceinline__ float group_sum(float a) {
    if constexpr (T >= 2) a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x111, 0xF, 0xF, false));
    if constexpr (T >= 4) a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x112, 0xF, 0xF, false));
    if constexpr (T >= 8) a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x114, 0xF, 0xF, false));
    if constexpr (T >= 16) a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x118, 0xF, 0xF, false));
    // row_bcast:15 -- the last lane of each row of 16 adds into the next row
    if constexpr (T >= 32) a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x142, 0xA, 0xF, false));
    // row_bcast:31 -- lane 31 adds into the upper half
    if constexpr (T >= 64) a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x143, 0xC, 0xF, false));
    return a;
}

// LDS rows of slice sums per workgroup: the activation regions take
// M * WPB * 64 * 40 bytes and the slice sums M * WPB * rw * 4 of the
// 160 KiB of a compute unit.
constexpr int rw_cap(int M) { return M <= 3 ? 1024 : 512; }


template <int QT, int M, int AX, int T, int NBL, int D, int D0, int WPB, bool KS, bool GU = false>
__global__ void __launch_bounds__(64 * WPB)
k_fx(float *__restrict__ y, const int8_t *__restrict__ wq, const float *__restrict__ wd, int32_t rows, int32_t K,
     const float *__restrict__ x, const int8_t *__restrict__ xq, const float *__restrict__ xd,
     const float *__restrict__ xn, float eps, int8_t *__restrict__ xq_out, float *__restrict__ xd_out, int32_t r0,
     int32_t r1, int32_t rw, float *__restrict__ ya) {
    // GU: rows = 2 F, the first F rows the FFN gate and the last F the up
    // projection; this workgroup takes pairs [g0, g1) -- gate rows g0 .. g1 - 1
    // and up rows F + g0 .. F + g1 - 1, as passes 0 .. nph - 1 and nph .. 2 nph - 1
    // -- and ends with ya[j] = silu(y[j]) * y[F + j] (the spec's silu_mul on
    // the two halves of the product) besides y itself
    constexpr bool FX = AX != kActQ8;          // float32 activation, quantized here
    static_assert(!GU || (KS && M == 1), "paired gate and up rows: split-K, one activation row");
    constexpr int PASS = 64 / T;               // rows per pass
    constexpr int QB = (QT == 8) ? 32 : 16;    // quant bytes per block
    static_assert(T * NBL <= 64 && (T * NBL) % 16 == 0, "a slice is at most 64 blocks, loaded 16 blocks at a time");
    static_assert(D0 >= 0 && D0 <= D - 1, "passes issued before the quantization");
    static_assert(!FX || M == 1, "the fused form takes one float32 activation row");
    // SQ: slices of 2 or more blocks per lane fetch a pass's weight scales
    // with one 16-byte load per lane (lane l: row l / 16 of the pass, blocks
    // 4 (l % 16) .. + 3 of the slice) instead of one 4-byte load per block,
    // and redistribute them through a private 1 KiB LDS slot: the same bytes
    // in a third of the load instructions, where the LDS allows
    constexpr int LDS0 = M * WPB * 64 * 40 + (KS ? M * WPB * rw_cap(M) * 4 : 0);
    constexpr bool SQ = QMV_FX_SQ && KS && NBL >= 2 && T == 16 && LDS0 + WPB * 1024 <= 163840;
    static_assert(LDS0 + (SQ ? WPB * 1024 : 0) <= 163840, "LDS of one compute unit");
    __shared__ v4i s_lo[M][WPB][64], s_hi[M][WPB][64];
    __shared__ float s_dx[M][WPB][64];
    __shared__ int s_sx[M][WPB][64];
    __shared__ float s_dq[SQ ? WPB : 1][SQ ? 256 : 1];  // SQ: [row of the pass][block of the slice]
    __shared__ float s_bs[AX == kActRms ? 64 * WPB : 1];  // rmsnorm: sums of squares per block
    extern __shared__ float s_red[];           // [M][WPB][rw] slice sums

    const int nb = K >> 5;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // KS: the wavefronts split K (slice of S blocks each) and share every
    // row; otherwise every wavefront holds all of K and takes every WPB-th
    // pass of rows
    const int S = KS ? (nb + WPB - 1) / WPB : nb;
    const int kb0 = KS ? min(wid * S, nb) : 0;
    const int ns = min(S, nb - kb0);           // blocks in this wavefront's slice
    const int g0 = r0 + blockIdx.x * rw;       // this workgroup's rows (GU: pairs) g0 .. g1 - 1
    const int g1 = min(r1, g0 + rw);
    const int F = rows >> 1;                   // GU: gate rows
    const int nph = (g1 - g0 + PASS - 1) / PASS;  // GU: passes per half
    const int nrp = GU ? 2 * nph : nph;        // passes of the workgroup
    const int npass = KS ? nrp : (nrp + WPB - 1) / WPB;  // passes of this wavefront
    const int rws = GU ? 2 * rw : rw;          // slice sums kept per wavefront
    const int pstride = KS ? 1 : WPB;          // pass j of this wavefront = workgroup pass j * pstride + pfirst
    const int pfirst = KS ? 0 : wid;

    // 1. this wavefront's activation slice, coalesced: round k covers
    //    blocks kb0 + 16 k .. kb0 + 16 k + 15, lane l holding elements
    //    8 (l % 4) .. 8 (l % 4) + 7 of block kb0 + 16 k + l / 4 (float32
    //    in the fused form, the quants and the block scale otherwise)
    constexpr int NR = T * NBL / 16;           // rounds of 16 blocks
    constexpr int MX = FX ? 1 : M;
    constexpr int NRN = (AX == kActRms || AX == kActSilu) ? NR : 1;
    float4 xa[FX ? NR : 1], xb[FX ? NR : 1], na[NRN], nb8[NRN];
    int xv0[MX][FX ? 1 : NR], xv1[MX][FX ? 1 : NR];
    float xdv[MX][FX ? 1 : NR];
    if constexpr (FX) {
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, K * 4);
        const __amdgpu_buffer_rsrc_t rn = make_rsrc(xn, (AX == kActRms || AX == kActSilu) ? K * 4 : 0);
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const int b = 16 * k + (lane >> 2);
            const int o = b < ns ? (kb0 + b) * 128 + 32 * (lane & 3) : kOOB;
            xa[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 0));
            xb[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rx, o + 16, 0, 0));
            if constexpr (AX == kActRms || AX == kActSilu) {  // norm weights, or u, of the same elements
                na[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rn, o, 0, 0));
                nb8[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rn, o + 16, 0, 0));
            }
        }
    } else {
        const __amdgpu_buffer_rsrc_t rxq = make_rsrc(xq, M * K);
        const __amdgpu_buffer_rsrc_t rxd = make_rsrc(xd, M * nb * 4);
#pragma unroll
        for (int m = 0; m < M; ++m) {
#pragma unroll
            for (int k = 0; k < NR; ++k) {
                const int b = 16 * k + (lane >> 2);
                const bool ok = b < ns;
                const int blk = m * nb + kb0 + b;
                const auto v = __builtin_amdgcn_raw_buffer_load_b64(rxq, ok ? blk * 32 + 8 * (lane & 3) : kOOB, 0, 0);
                xv0[m][k] = (int)v[0];
                xv1[m][k] = (int)v[1];
                xdv[m][k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rxd, ok ? blk * 4 : kOOB, 0, 0));
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // the activation requests go out first
#if QMV_FX_XBAR
    __builtin_amdgcn_s_barrier();       // ... before any wavefront's weight requests
    __builtin_amdgcn_sched_barrier(0);
#endif

    // 2. the first D - 1 passes of weights
    const int rows_here = g1 - g0;
    // GU: the descriptors span gate row g0 .. up row F + g1 - 1; passes of
    // the up half skip the F - PASS * nph rows between the two ranges (rows of
    // the gate half's last pass past g1 read other rows, whose sums are
    // never stored)
    const int span = GU ? F + rows_here : rows_here;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(wq + (size_t)g0 * nb * QB, span * nb * QB);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(wd + (size_t)g0 * nb, span * nb * 4);
    const int skipq = GU ? (F - PASS * nph) * nb * QB : 0, skipd = GU ? (F - PASS * nph) * nb * 4 : 0;
    const int prow = lane / T;                 // row of a pass
    int oq[NBL], od[NBL];                      // pass-0 offsets of this lane's blocks
#pragma unroll
    for (int k = 0; k < NBL; ++k) {
        const int c = lane % T + T * k;
        const bool ok = c < ns;
        oq[k] = ok ? ((pfirst * PASS + prow) * nb + kb0 + c) * QB : kOOB;
        od[k] = ok ? ((pfirst * PASS + prow) * nb + kb0 + c) * 4 : kOOB;
    }
    const int pq = pstride * PASS * nb * QB, pd = pstride * PASS * nb * 4;  // bytes per pass of this wavefront
    const int od4 = 4 * (lane % 16) < ns ? ((pfirst * PASS + prow) * nb + kb0 + 4 * (lane % 16)) * 4 : kOOB;
    auto load = [&](Pass<QT, NBL> &p, int j) __attribute__((always_inline)) {
        const bool up = GU && j >= nph;
#pragma unroll
        for (int k = 0; k < NBL; ++k) {
            // offsets of passes at or beyond npass fall outside the range
            const int a = oq[k] + j * pq + (up ? skipq : 0), b = od[k] + j * pd + (up ? skipd : 0);
            p.w[k][0] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rq, a, 0, kNT));
            if constexpr (QT == 8)
                p.w[k][1] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rq, a + 16, 0, kNT));
            if constexpr (!SQ)
                p.dw[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, b, 0, kNT));
        }
        if constexpr (SQ)  // a quad may reach past the slice: the pass loop zeroes those scales
            p.dq = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rd, od4 + j * pd + (up ? skipd : 0),
                                                                                 0, kNT));
    };
    Pass<QT, NBL> ring[D];
#pragma unroll
    for (int d = 0; d < D0; ++d) load(ring[d], d);
    __builtin_amdgcn_sched_barrier(0);

    // 3a. rmsnorm: sum of squares of every block (pairwise over its 32
    //     elements: 8 per lane, then the 4 lanes of the block), the blocks'
    //     sums pairwise over their zero-padded count, then x <- w * (inv * x)
    if constexpr (AX == kActRms) {
        float *bs = KS ? s_bs : s_bs + 64 * wid;  // split K: the workgroup's K; whole rows: this wavefront's
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const int b = 16 * k + (lane >> 2);
            float q = sumsq8(xa[k], xb[k]);
            q += __int_as_float(dpp_xor1(__float_as_int(q)));
            q += __int_as_float(dpp_xor2(__float_as_int(q)));
            if ((lane & 3) == 0 && b < ns) bs[kb0 + b] = q;
        }
        if constexpr (KS) {
            __syncthreads();
        } else {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        int P = 1;
        while (P < nb) P *= 2;                 // block count padded to a power of two (at most 512)
        const int E = P > 64 ? P / 64 : 1;     // consecutive block sums per lane
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int b = lane * E + e;
            v[e] = (e < E && b < nb) ? bs[b] : 0.0f;
        }
        // pairwise within the lane (E = 1, 2, 4 or 8 values; the rest are 0)
        float ss = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
        if (E == 1) ss = v[0];
        else if (E == 2) ss = v[0] + v[1];
        else if (E == 4) ss = (v[0] + v[1]) + (v[2] + v[3]);
        // then across lanes, aligned groups of 2, 4, ... 64 lanes: quad
        // permutes for 2 and 4, then mirrors within 8 and 16 lanes (each
        // lane of a group already holds the group's sum, so the mirrored
        // lane holds the partner group's), then 32 and 64
        ss += __int_as_float(dpp_xor1(__float_as_int(ss)));
        ss += __int_as_float(dpp_xor2(__float_as_int(ss)));
        ss += __int_as_float(dpp_mirror8(__float_as_int(ss)));
        ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x140, 0xF, 0xF, false));
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        const float inv = rms_inv(ss, K, eps);
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            xa[k] = make_float4(rms_apply(xa[k].x, na[k].x, inv), rms_apply(xa[k].y, na[k].y, inv),
                                rms_apply(xa[k].z, na[k].z, inv), rms_apply(xa[k].w, na[k].w, inv));
            xb[k] = make_float4(rms_apply(xb[k].x, nb8[k].x, inv), rms_apply(xb[k].y, nb8[k].y, inv),
                                rms_apply(xb[k].z, nb8[k].z, inv), rms_apply(xb[k].w, nb8[k].w, inv));
        }
    }

    // 3b. FFN gate: x <- silu(g) * u elementwise
    if constexpr (AX == kActSilu) {
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            xa[k] = make_float4(silu_mul1(xa[k].x, na[k].x), silu_mul1(xa[k].y, na[k].y),
                                silu_mul1(xa[k].z, na[k].z), silu_mul1(xa[k].w, na[k].w));
            xb[k] = make_float4(silu_mul1(xb[k].x, nb8[k].x), silu_mul1(xb[k].y, nb8[k].y),
                                silu_mul1(xb[k].z, nb8[k].z), silu_mul1(xb[k].w, nb8[k].w));
        }
    }

    // 3. quantize the slice (fused) or sum its quants (pre-quantized), 4
    //    lanes per block (lanes past the slice hold zeros), into the
    //    private LDS region -- no branch around the arithmetic, so that the
    //    activation loads stay ahead of the weight loads
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const int b = 16 * k + (lane >> 2), c = lane & 3;
            float d;
            int qs;
            int2 pk;
            if constexpr (FX) {
                pk = quant_q8_group4(xa[k], xb[k], d, qs);
            } else {
                pk = make_int2(xv0[m][k], xv1[m][k]);
                d = xdv[m][k];
                qs = 0;
                if constexpr (QT == 4) {
                    qs = dot4(pk.x, 0x01010101, dot4(pk.y, 0x01010101, 0));
                    qs += dpp_xor1(qs);
                    qs += dpp_xor2(qs);
                }
            }
            *reinterpret_cast<int2 *>(reinterpret_cast<int *>(c < 2 ? &s_lo[m][wid][b] : &s_hi[m][wid][b]) +
                                      2 * (c & 1)) = pk;
            if (c == 0) {
                s_dx[m][wid][b] = d;
                s_sx[m][wid][b] = -8 * qs;
            }
            if (FX && xq_out != nullptr && blockIdx.x == 0 && b < ns) {  // optional copy of the quantized activation
                reinterpret_cast<int2 *>(xq_out + (size_t)(kb0 + b) * QK)[c] = pk;
                if (c == 0) xd_out[kb0 + b] = d;
            }
        }
    }
    // LDS operations of one wavefront complete in order: once this
    // wavefront's writes are done, all of its lanes read them
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    v4i xl[M][NBL], xh[M][NBL];
    float dx[M][NBL];
    int sx[M][NBL];
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
        for (int k = 0; k < NBL; ++k) {
            const int c = lane % T + T * k;
            const bool ok = c < ns;
            const int cc = ok ? c : 0;
            xl[m][k] = s_lo[m][wid][cc];
            xh[m][k] = s_hi[m][wid][cc];
            dx[m][k] = ok ? s_dx[m][wid][cc] : 0.0f;
            sx[m][k] = s_sx[m][wid][cc];
        }
    }

    // the rest of the first D - 1 passes
#pragma unroll
    for (int d = D0; d < D - 1; ++d) load(ring[d], d);

    // 4. passes: loads of pass j + D - 1 in flight while pass j is computed
    auto step = [&](const Pass<QT, NBL> &p, int j) __attribute__((always_inline)) {
        float dwk[NBL];
        if constexpr (SQ) {
            // lane l's 4 scales go to floats 4 l .. 4 l + 3 of the slot, that is
            // row l / 16, blocks 4 (l % 16) ..; each lane then reads its own
            // (a wavefront's LDS operations run in order); scales past the
            // slice (other slices' or the next row's) are taken as 0, the
            // value the 4-byte loads' out-of-range offsets return
            *reinterpret_cast<v4i *>(&s_dq[wid][4 * lane]) = p.dq;
#pragma unroll
            for (int k = 0; k < NBL; ++k)
                dwk[k] = lane % 16 + 16 * k < ns ? s_dq[wid][64 * prow + lane % 16 + 16 * k] : 0.0f;
        } else {
#pragma unroll
            for (int k = 0; k < NBL; ++k) dwk[k] = p.dw[k];
        }
        float a[M];
#pragma unroll
        for (int m = 0; m < M; ++m) a[m] = 0.0f;
#pragma unroll
        for (int k = 0; k < NBL; ++k) {
            if constexpr (QT == 4) {
                // byte j of the 16: low nibble = element j, high nibble = element j + 16
                const unsigned mk = 0x0F0F0F0Fu;
                const v4i w = p.w[k][0];
                const int l0 = (unsigned)w.x & mk, l1 = (unsigned)w.y & mk;
                const int l2 = (unsigned)w.z & mk, l3 = (unsigned)w.w & mk;
                const int h0 = ((unsigned)w.x >> 4) & mk, h1 = ((unsigned)w.y >> 4) & mk;
                const int h2 = ((unsigned)w.z >> 4) & mk, h3 = ((unsigned)w.w >> 4) & mk;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    int s = dot4(l0, xl[m][k].x, sx[m][k]);  // starts at -8 * sum(qx)
                    s = dot4(l1, xl[m][k].y, s);
                    s = dot4(l2, xl[m][k].z, s);
                    s = dot4(l3, xl[m][k].w, s);
                    s = dot4(h0, xh[m][k].x, s);
                    s = dot4(h1, xh[m][k].y, s);
                    s = dot4(h2, xh[m][k].z, s);
                    s = dot4(h3, xh[m][k].w, s);
                    a[m] = fmaf((float)s, dwk[k] * dx[m][k], a[m]);
                }
            } else {
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    int s = dot4(p.w[k][0].x, xl[m][k].x, 0);
                    s = dot4(p.w[k][0].y, xl[m][k].y, s);
                    s = dot4(p.w[k][0].z, xl[m][k].z, s);
                    s = dot4(p.w[k][0].w, xl[m][k].w, s);
                    s = dot4(p.w[k][1].x, xh[m][k].x, s);
                    s = dot4(p.w[k][1].y, xh[m][k].y, s);
                    s = dot4(p.w[k][1].z, xh[m][k].z, s);
                    s = dot4(p.w[k][1].w, xh[m][k].w, s);
                    a[m] = fmaf((float)s, dwk[k] * dx[m][k], a[m]);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float t = group_sum<T>(a[m]);
            if constexpr (KS) {
                const int r = j * PASS + prow;
                if (lane % T == T - 1 && j < npass && r < rws) s_red[(m * WPB + wid) * rws + r] = t;
            } else {  // whole rows: store directly
                const int r = (j * pstride + pfirst) * PASS + prow;
                if (lane % T == T - 1 && j < npass && r < rows_here) y[(size_t)m * rows + g0 + r] = t;
            }
        }
    };
#if QMV_FX_TAIL
    // Ring turns whose loads all fall among the wavefront's passes run as a
    // loop; the remaining R passes (1 .. 2 D - 2, the first D - 1 of them
    // already in the ring) run as straight-line code specialised on R that
    // loads only passes that exist.  Range-checked loads past the last pass
    // read nothing but still take the per-CU address path, which the
    // multi-block slices keep full; a per-pass test instead of the
    // specialisation makes the compiler's waits for the ring inexact.
    int it = 0;
    for (; (it + 2) * D - 2 < npass; ++it) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int j = it * D + d;
            load(ring[(d + D - 1) % D], j + D - 1);
            step(ring[d], j);
        }
    }
    with_count<1, 2 * D - 2>(npass - it * D, [&](auto rc) __attribute__((always_inline)) {
        constexpr int R = decltype(rc)::value;
#pragma unroll
        for (int q = 0; q < R; ++q) {
            if (q + D - 1 < R) load(ring[(q + D - 1) % D], it * D + q + D - 1);
            step(ring[q % D], it * D + q);
        }
    });
#else
    const int nit = (npass + D - 1) / D;
    for (int it = 0; it < nit; ++it) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int j = it * D + d;
            load(ring[(d + D - 1) % D], j + D - 1);
            step(ring[d], j);
        }
    }
#endif

    if constexpr (!KS) return;
    // 5. add the wavefronts' slice sums of each row in wavefront order
    __syncthreads();
    if constexpr (GU) {
        for (int v = threadIdx.x; v < rows_here; v += 64 * WPB) {
            float sg = 0.0f, su = 0.0f;
#pragma unroll
            for (int w = 0; w < WPB; ++w) {
                sg += s_red[w * rws + v];
                su += s_red[w * rws + PASS * nph + v];
            }
            y[g0 + v] = sg;
            y[F + g0 + v] = su;
            ya[g0 + v] = silu_mul1(sg, su);
        }
        return;
    }
    for (int r = threadIdx.x; r < rows_here; r += 64 * WPB) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < WPB; ++w) s += s_red[(m * WPB + w) * rws + r];
            y[(size_t)m * rows + g0 + r] = s;
        }
    }
}

// The same split-K streaming product for 3 or 4 pre-quantized activation
// rows on the matrix cores: v_mfma_i32_4x4x4_16b_i8 computes 16 independent
// 4 x 4 tiles of 4-element dots.  Lane l = 4 t + i supplies one 4-byte
// chunk of weight row i of tile t (as the A operand) and the same chunk of
// activation row i (as the B operand); register v of lane l receives
// tile t's (weight row v, activation row i) dot.  Here tile t of a pass is
// block c = t + 16 k of the wavefront's slice for the pass's 4 weight rows,
// so eight chained instructions (the 8 chunks of a block) leave in lane
// 4 t + i the block sums of the 4 weight rows against activation row i:
// one lane per (weight row, block) loads its own weight block (16 lanes
// read 16 consecutive blocks of a row, 4 rows per load instruction) and
// its own activation row's block, straight into registers.  The Q4_0 offset
// -8 * sum(qx) seeds the accumulator.  The fp32 scaling is spread over all
// 64 lanes (4 block sums each), the 4 lanes of a tile share the weight
// scales through quad permutes, the 4 tiles of each 16-lane row are added
// with row-shift DPP adds and the 4 rows of 16 lanes with two lane
// shuffles; the wavefronts' sums are added in LDS in wavefront order, one
// (weight row, activation row) per thread.
constexpr int kMqRwCap = 256;  // rows per workgroup: slice sums [4][WPB][rw] in LDS

template <int QT, int NBL, int D, int D0, int WPB>
__global__ void __launch_bounds__(64 * WPB)
k_mq(float *__restrict__ y, const int8_t *__restrict__ wq, const float *__restrict__ wd, int32_t rows, int32_t K,
     int32_t M, const int8_t *__restrict__ xq, const float *__restrict__ xd, int32_t r0, int32_t r1, int32_t rw) {
    constexpr int QB = (QT == 8) ? 32 : 16;    // quant bytes per block
    static_assert(D0 >= 0 && D0 <= D - 1, "passes issued before the activation sums");
    // SQ: a pass's weight scales in one 16-byte load per lane, as in k_fx
    constexpr bool SQ = QMV_MQ_SQ && NBL >= 2;
    extern __shared__ float s_red[];           // [activation row][wavefront][rw] partial sums
    __shared__ float s_dq[SQ ? WPB : 1][SQ ? 256 : 1];  // SQ: [row of the pass][block of the slice]

    const int nb = K >> 5;
    const int lane = threadIdx.x & 63;
    const int t = lane >> 2, i = lane & 3;     // tile (block of the pass) and row within the tile
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = (nb + WPB - 1) / WPB;
    const int kb0 = min(wid * S, nb);
    const int ns = min(S, nb - kb0);           // blocks in this wavefront's slice
    const int g0 = r0 + blockIdx.x * rw;       // this workgroup's rows g0 .. g1 - 1
    const int g1 = min(r1, g0 + rw);
    const int rows_here = g1 - g0;
    const int npass = (rows_here + 3) >> 2;    // passes of 4 weight rows

    // 1. activation row i, blocks kb0 + t + 16 k (rows at or past M, and
    //    blocks past the slice, read zeros)
    const __amdgpu_buffer_rsrc_t rxq = make_rsrc(xq, M * K);
    const __amdgpu_buffer_rsrc_t rxd = make_rsrc(xd, M * nb * 4);
    v4i xlo[NBL], xhi[NBL];
    float dx[NBL];
#pragma unroll
    for (int k = 0; k < NBL; ++k) {
        const int c = t + 16 * k;
        const bool ok = c < ns && i < M;
        const int blk = i * nb + kb0 + c;
        xlo[k] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rxq, ok ? blk * 32 : kOOB, 0, 0));
        xhi[k] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rxq, ok ? blk * 32 + 16 : kOOB, 0, 0));
        dx[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rxd, ok ? blk * 4 : kOOB, 0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);  // the activation requests go out first
#if QMV_FX_XBAR
    __builtin_amdgcn_s_barrier();       // ... before any wavefront's weight requests
    __builtin_amdgcn_sched_barrier(0);
#endif

    // 2. the first D - 1 passes of weights: lane (t, i) reads row 4 j + i,
    //    block kb0 + t + 16 k
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(wq + (size_t)g0 * nb * QB, rows_here * nb * QB);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(wd + (size_t)g0 * nb, rows_here * nb * 4);
    int oq[NBL], od[NBL];
#pragma unroll
    for (int k = 0; k < NBL; ++k) {
        const int c = t + 16 * k;
        const bool ok = c < ns;
        oq[k] = ok ? (i * nb + kb0 + c) * QB : kOOB;
        od[k] = ok ? (i * nb + kb0 + c) * 4 : kOOB;
    }
    const int pq = 4 * nb * QB, pd = 4 * nb * 4;  // bytes per pass
    // SQ: lane l reads row l / 16 of the pass, blocks 4 (l % 16) .. + 3
    const int od4 = 4 * (lane % 16) < ns ? ((lane >> 4) * nb + kb0 + 4 * (lane % 16)) * 4 : kOOB;
    auto load = [&](Pass<QT, NBL> &p, int j) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < NBL; ++k) {
            const int a = oq[k] + j * pq, b = od[k] + j * pd;
            p.w[k][0] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rq, a, 0, kNT));
            if constexpr (QT == 8)
                p.w[k][1] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rq, a + 16, 0, kNT));
            if constexpr (!SQ)
                p.dw[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, b, 0, kNT));
        }
        if constexpr (SQ)
            p.dq = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rd, od4 + j * pd, 0, kNT));
    };
    Pass<QT, NBL> ring[D];
#pragma unroll
    for (int d = 0; d < D0; ++d) load(ring[d], d);
    __builtin_amdgcn_sched_barrier(0);

    // 3. the Q4_0 offset of each activation block: -8 * sum of its quants
    int sx[NBL];
#pragma unroll
    for (int k = 0; k < NBL; ++k) {
        int s = 0;
        if constexpr (QT == 4) {
            s = dot4(xlo[k].x, 0x01010101, dot4(xlo[k].y, 0x01010101, dot4(xlo[k].z, 0x01010101,
                dot4(xlo[k].w, 0x01010101, 0))));
            s = dot4(xhi[k].x, 0x01010101, dot4(xhi[k].y, 0x01010101, dot4(xhi[k].z, 0x01010101,
                dot4(xhi[k].w, 0x01010101, s))));
        }
        sx[k] = -8 * s;
    }
#pragma unroll
    for (int d = D0; d < D - 1; ++d) load(ring[d], d);

    // 4. passes: loads of pass j + D - 1 in flight while pass j is computed
    float *red = s_red + (i * WPB + wid) * rw;
    auto step = [&](const Pass<QT, NBL> &p, int j) __attribute__((always_inline)) {
        v4i acc[NBL];
#pragma unroll
        for (int k = 0; k < NBL; ++k) acc[k] = (v4i){sx[k], sx[k], sx[k], sx[k]};
#pragma unroll
        for (int h = 0; h < 8; ++h) {
#pragma unroll
            for (int k = 0; k < NBL; ++k) {
                int a;
                if constexpr (QT == 4) {
                    // byte j of the 16: low nibble = element j, high nibble = element j + 16
                    const unsigned w = (unsigned)p.w[k][0][h & 3];
                    a = (int)((h < 4 ? w : w >> 4) & 0x0F0F0F0Fu);
                } else {
                    a = p.w[k][h >> 2][h & 3];
                }
                const int b = h < 4 ? xlo[k][h] : xhi[k][h - 4];
                acc[k] = __builtin_amdgcn_mfma_i32_4x4x4i8(a, b, acc[k], 0, 0, 0);
            }
        }
        float dwk[NBL];
        if constexpr (SQ) {
            // lane l's quad goes to floats 4 l .. 4 l + 3 of the slot; lane
            // (t, i) then reads row i's scale of block t + 16 k (0 past the
            // slice, as the 4-byte loads' out-of-range offsets give)
            *reinterpret_cast<v4i *>(&s_dq[wid][4 * lane]) = p.dq;
#pragma unroll
            for (int k = 0; k < NBL; ++k) dwk[k] = t + 16 * k < ns ? s_dq[wid][64 * i + t + 16 * k] : 0.0f;
        } else {
#pragma unroll
            for (int k = 0; k < NBL; ++k) dwk[k] = p.dw[k];
        }
        float f[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < NBL; ++k) {
            const int dwi = __float_as_int(dwk[k]);
            // weight scale of row v of the tile: lane 4 t + v's (quad_perm [v, v, v, v])
            const float w0 = __int_as_float(__builtin_amdgcn_mov_dpp(dwi, 0x00, 0xF, 0xF, false));
            const float w1 = __int_as_float(__builtin_amdgcn_mov_dpp(dwi, 0x55, 0xF, 0xF, false));
            const float w2 = __int_as_float(__builtin_amdgcn_mov_dpp(dwi, 0xAA, 0xF, 0xF, false));
            const float w3 = __int_as_float(__builtin_amdgcn_mov_dpp(dwi, 0xFF, 0xF, 0xF, false));
            f[0] = fmaf((float)acc[k][0], w0 * dx[k], f[0]);
            f[1] = fmaf((float)acc[k][1], w1 * dx[k], f[1]);
            f[2] = fmaf((float)acc[k][2], w2 * dx[k], f[2]);
            f[3] = fmaf((float)acc[k][3], w3 * dx[k], f[3]);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            // tiles 4 r .. 4 r + 3 of the 16-lane row r: lanes 12 .. 15 end with the sums
            f[v] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(f[v]), 0x114, 0xF, 0xF, false));
            f[v] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(f[v]), 0x118, 0xF, 0xF, false));
            // then the four 16-lane rows: (r0 + r1) + (r2 + r3) in every row
            f[v] += __shfl_xor(f[v], 16);
            f[v] += __shfl_xor(f[v], 32);
        }
        if (lane >= 12 && lane < 16 && j < npass)
            *reinterpret_cast<float4 *>(red + 4 * j) = make_float4(f[0], f[1], f[2], f[3]);
    };
#if QMV_FX_TAIL
    // whole ring turns, then the last passes specialised on their count (as in k_fx)
    int it = 0;
    for (; (it + 2) * D - 2 < npass; ++it) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int j = it * D + d;
            load(ring[(d + D - 1) % D], j + D - 1);
            step(ring[d], j);
        }
    }
    with_count<1, 2 * D - 2>(npass - it * D, [&](auto rc) __attribute__((always_inline)) {
        constexpr int R = decltype(rc)::value;
#pragma unroll
        for (int q = 0; q < R; ++q) {
            if (q + D - 1 < R) load(ring[(q + D - 1) % D], it * D + q + D - 1);
            step(ring[q % D], it * D + q);
        }
    });
#else
    const int nit = (npass + D - 1) / D;
    for (int it = 0; it < nit; ++it) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int j = it * D + d;
            load(ring[(d + D - 1) % D], j + D - 1);
            step(ring[d], j);
        }
    }
#endif

    // 5. add the wavefronts' sums of each (activation row, weight row) in
    //    wavefront order, one pair per thread
    __syncthreads();
    for (int e = threadIdx.x; e < rows_here * M; e += 64 * WPB) {  // one (weight row, activation row) per thread
        const int r = e % rows_here, m = e / rows_here;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WPB; ++w) s += s_red[(m * WPB + w) * rw + r];
        y[(size_t)m * rows + g0 + r] = s;
    }
}

template <int QT, int NBL, int D, int WPB>
hipError_t launch_mq_t(const RowsArgs &a, hipStream_t s, const char **name) {
    static const std::string kname = variant_name("mq_q%d_n%d_d%d_w%d", QT, NBL, D, WPB);
    constexpr int D0 = QMV_FX_D0 < D - 1 ? QMV_FX_D0 : D - 1;
    auto kern = k_mq<QT, NBL, D, D0, WPB>;
    const int nrows = a.r1 - a.r0;
    const int groups = a.num_cu * QMV_FX_WG_PER_CU;
    const int rw = min(kMqRwCap, ((nrows + groups - 1) / groups + 3) / 4 * 4);
    const int grid = (nrows + rw - 1) / rw;
    const size_t lds = (size_t)4 * WPB * rw * 4;
    // the largest size any call of this kernel asks for (rw at its cap)
    hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), (size_t)4 * WPB * kMqRwCap * 4);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WPB), lds, s, a.y, a.wq, a.wd, a.rows, a.K, a.M, a.xq, a.xd,
                       a.r0, a.r1, rw);
    *name = kname.c_str();
    return hipGetLastError();
}

template <int QT>
hipError_t launch_mq(const RowsArgs &a, hipStream_t s, const char **name) {
    // ring depth as ring_depth: 4 for one block per lane, 3 for more
    constexpr int W = QMV_FX_WPB, D = QMV_FX_D, DN = QMV_FX_D3_NBL <= 2 ? 3 : D;
    const int S = (a.K / QK + W - 1) / W;
    if (S <= 16) return launch_mq_t<QT, 1, D, W>(a, s, name);
    if (S <= 32) return launch_mq_t<QT, 2, DN, W>(a, s, name);
    if (S <= 48) return launch_mq_t<QT, 3, DN, W>(a, s, name);
    return launch_mq_t<QT, 4, DN, W>(a, s, name);
}

template <int QT, int M, int AX, int T, int NBL, int D, int WPB, bool KS = true, bool GU = false>
hipError_t launch_t(const RowsArgs &a, int rw, hipStream_t s, const char **name) {
    static const std::string kname =
        AX != kActQ8 ? variant_name("fx%s_q%d_t%d_n%d_d%d_w%d%s%s", AX == kActRms ? "n" : (AX == kActSilu ? "s" : ""),
                                    QT, T, NBL, D, WPB, KS ? "" : "_rows", GU ? "_gu" : "")
                     : variant_name("px_q%d_m%d_t%d_n%d_d%d_w%d%s", QT, M, T, NBL, D, WPB, KS ? "" : "_rows");
    constexpr int D0W = AX == kActRms ? QMV_FX_D0_RMS : (AX == kActSilu ? QMV_FX_D0_SILU : QMV_FX_D0);
    constexpr int D0 = D0W < D - 1 ? D0W : D - 1;
    auto kern = k_fx<QT, M, AX, T, NBL, D, D0, WPB, KS, GU>;
    const int nrows = a.r1 - a.r0;
    const int grid = (nrows + rw - 1) / rw;
    const size_t lds = KS ? (size_t)M * WPB * (GU ? 2 : 1) * rw * 4 : 0;
    if (KS) {  // the largest size any call of this kernel asks for (rw at its cap)
        hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), (size_t)M * WPB * rw_cap(M) * 4);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WPB), lds, s, a.y, a.wq, a.wd, a.rows, a.K, a.x, a.xq, a.xd,
                       AX == kActSilu ? a.xu : a.xn, a.eps, a.xq_out, a.xd_out, a.r0, a.r1, rw, a.ya);
    *name = kname.c_str();
    return hipGetLastError();
}

// Ring depth: four passes in flight for slices of one block per lane, three
// for slices of several blocks per lane (measured faster there: Llama-7B
// W_down 9.45 -> 9.30 us, TinyLlama W_down 3.94 -> 3.73 us; each of their
// passes already carries 2 - 4 loads per lane) and where the activation
// registers of several rows leave no room for a fourth (Q8_0 with M * NBL > 6).
template <int QT, int M, int NBL>
constexpr int ring_depth() {
    return (NBL >= QMV_FX_D3_NBL || (QT == 8 && M * NBL > 6)) ? 3 : QMV_FX_D;
}

// One float32 row of Q4_0 with 257 .. 384 blocks: 2 blocks per lane over
// nb / 32 wavefronts (9 .. 12) instead of 3 over 8, where that leaves at most
// 5% of the lanes' block slots empty (returns that wavefront count, else 0).
// A load instruction costs the same whether its lanes read or fall past the
// slice.  Measured per launch (4096 rows, graphs of launches streaming from
// HBM, alternating on one box): K = 9216 6.70 - 6.74 -> 6.25 us, 10240
// 6.90 -> 6.68 - 6.69, 11008 7.58 - 7.62 -> 7.11 - 7.15, 12288 7.51 - 7.56 ->
// 7.42 - 7.46.  12 wavefronts at K = 11008 (the same 89.6% slot use as 3
// blocks over 8) were no faster than 8.
inline int wide_slices(int nb) {
    const int w2 = (nb + 31) / 32;
    return (nb > 256 && w2 <= 12 && 20 * nb >= 19 * 32 * w2) ? w2 : 0;
}

template <int QT, int M, int AX, bool GU>
hipError_t launch_w2(const RowsArgs &a, int rw, int w2, hipStream_t s, const char **name) {
    constexpr int D2 = ring_depth<QT, M, 2>();
    switch (w2) {
        case 9: return launch_t<QT, M, AX, 16, 2, D2, 9, true, GU>(a, rw, s, name);
        case 10: return launch_t<QT, M, AX, 16, 2, D2, 10, true, GU>(a, rw, s, name);
        case 11: return launch_t<QT, M, AX, 16, 2, D2, 11, true, GU>(a, rw, s, name);
        default: return launch_t<QT, M, AX, 16, 2, D2, 12, true, GU>(a, rw, s, name);
    }
}

template <int QT, int M, int AX, int W>
hipError_t launch_m_w(const RowsArgs &a, hipStream_t s, const char **name) {
    constexpr bool FX = AX != kActQ8;
    const int nb = a.K / QK;
    const int S = (nb + W - 1) / W;
    const int nrows = a.r1 - a.r0;
    const int groups = a.num_cu * QMV_FX_WG_PER_CU;
    // rows per workgroup: a whole number of passes, at most one workgroup
    // per compute unit (capped so that the slice sums fit in LDS; whole-row
    // workgroups need no slice sums)
    auto rows_per = [&](int pass, bool ks) {
        const int want = ((nrows + groups - 1) / groups + pass - 1) / pass * pass;
        return ks ? min(rw_cap(M), want) : want;
    };
    if (a.ya != nullptr) {  // paired gate and up rows: split K only, pairs per workgroup at most rw_cap / 2
        if constexpr (FX && M == 1) {
            const int want = ((nrows + groups - 1) / groups + 3) / 4 * 4;
            const int rwp = min(rw_cap(M) / 2, want);
#if QMV_FX_W2
            if constexpr (QT == 4 && W == 8) {  // the plain product's split, so that y keeps its bits
                const int w2 = wide_slices(nb);
                if (w2) return launch_w2<QT, M, AX, true>(a, rwp, w2, s, name);
            }
#endif
            if (nb >= 64 && S <= 16) return launch_t<QT, M, AX, 16, 1, ring_depth<QT, M, 1>(), W, true, true>(a, rwp, s, name);
            if (nb >= 64 && S <= 32) return launch_t<QT, M, AX, 16, 2, ring_depth<QT, M, 2>(), W, true, true>(a, rwp, s, name);
            if (nb >= 64 && S <= 48) return launch_t<QT, M, AX, 16, 3, ring_depth<QT, M, 3>(), W, true, true>(a, rwp, s, name);
            if (nb >= 64 && S <= 64) return launch_t<QT, M, AX, 16, 4, ring_depth<QT, M, 4>(), W, true, true>(a, rwp, s, name);
        }
        return hipErrorNotSupported;
    }
    if (nb <= 16) return launch_t<QT, M, AX, 16, 1, ring_depth<QT, M, 1>(), W, false>(a, rows_per(4 * W, false), s, name);
    if (nb <= 32) return launch_t<QT, M, AX, 32, 1, ring_depth<QT, M, 1>(), W, false>(a, rows_per(2 * W, false), s, name);
    // split K: the fused matvec; pre-quantized Q8_0 weights with 2 .. 4
    // activation rows; pre-quantized Q4_0 weights with 2 or 3 rows and
    // slices of more than 16 blocks (Llama-7B W_down 4096 x 11008: 9.15 ->
    // 8.33 us at 2 rows, 10.38 -> 9.29 us at 3).  Elsewhere the
    // row-streaming kernel is as fast or faster (one row; W_up 11008 x 4096
    // at 1 - 3 rows: 6.63 / 7.1 / 7.74 against 6.8 / 7.25 / 7.98 us).
    constexpr bool PX4 = !FX && QT == 4 && M >= 2;
#if QMV_FX_W2  // more wavefronts of 2 blocks per lane (wide_slices)
    if constexpr (FX && M == 1 && QT == 4 && W == 8) {
        const int w2 = wide_slices(nb);
        if (w2) return launch_w2<QT, M, AX, false>(a, rows_per(4, true), w2, s, name);
    }
#endif
    if constexpr (FX || (QT == 8 && M >= 2) || PX4) {
        if (S <= 16) {
            if constexpr (PX4) return hipErrorNotSupported;
            else return launch_t<QT, M, AX, 16, 1, ring_depth<QT, M, 1>(), W>(a, rows_per(4, true), s, name);
        }
        if (S <= 32) return launch_t<QT, M, AX, 16, 2, ring_depth<QT, M, 2>(), W>(a, rows_per(4, true), s, name);
        if (S <= 48) return launch_t<QT, M, AX, 16, 3, ring_depth<QT, M, 3>(), W>(a, rows_per(4, true), s, name);
        if constexpr (M <= 2) return launch_t<QT, M, AX, 16, 4, ring_depth<QT, M, 4>(), W>(a, rows_per(4, true), s, name);
    }
    return hipErrorNotSupported;
}

// Wavefronts per workgroup for one activation row.  Measured on the MI355X
// (fused launches, weights streamed from HBM, 4 against 8 wavefronts):
// 4 (one per SIMD) is faster for whole rows per wavefront (Q8_0 4864 x 896
// 3.58 -> 3.39 us, 151936 x 896 31.1 -> 30.5 us) and for split-K slices of
// up to 16 Q4_0 blocks (K = 2048: 0.2 - 0.4 us faster at 256 .. 11264 rows)
// or 48 Q8_0 blocks (896 x 4864 4.93 -> 4.27 us, 11008 x 4096 12.3 ->
// 11.9 us); 8 is faster for Q4_0 at K = 4096 (11008 x 4096 7.1 against
// 7.3 us) and the only split-K form for longer rows.  Q4_0 at K = 5632 and
// Q8_0 at K = 8192 measured the same either way.
template <int QT, int M, int AX>
hipError_t launch_m(const RowsArgs &a, hipStream_t s, const char **name) {
    if constexpr (M == 1) {
        const int nb = a.K / QK, S4 = (nb + 3) / 4;
        if (nb <= 32 || (nb >= 64 && S4 <= (QT == 8 ? 48 : 16)))
            return launch_m_w<QT, M, AX, 4>(a, s, name);
    }
    return launch_m_w<QT, M, AX, QMV_FX_WPB>(a, s, name);
}

template <int QT>
hipError_t launch_q(const RowsArgs &a, hipStream_t s, const char **name) {
    if (a.x != nullptr) {
        if (a.xu != nullptr) return launch_m<QT, 1, kActSilu>(a, s, name);
        return a.xn != nullptr ? launch_m<QT, 1, kActRms>(a, s, name) : launch_m<QT, 1, kActF32>(a, s, name);
    }
    // pre-quantized: the matrix-core form for 4 rows of Q4_0 (measured
    // faster than both dot-product kernels) and for 3 or 4 rows of 64-block
    // slices (beyond the dot-product form's registers)
    const int nb = a.K / QK, S = (nb + QMV_FX_WPB - 1) / QMV_FX_WPB;
    if (nb > 32 && ((QT == 4 && a.M == 4) || (a.M >= 3 && S > 48))) return launch_mq<QT>(a, s, name);
    switch (a.M) {
        case 1: return launch_m<QT, 1, kActQ8>(a, s, name);
        case 2: return launch_m<QT, 2, kActQ8>(a, s, name);
        case 3: return launch_m<QT, 3, kActQ8>(a, s, name);
        case 4: return launch_m<QT, 4, kActQ8>(a, s, name);
        default: return hipErrorNotSupported;
    }
}

}  // namespace

// Split-K product for K / 32 <= 32 (whole rows per wavefront, M = 1 .. 4)
// and 64 <= K / 32 <= 64 * waves (K split over the wavefronts): the fused
// M = 1 matvec; pre-quantized Q8_0 weights with 2 .. 4 activation rows; 4
// rows of Q4_0 and 3 or 4 rows with slices beyond 48 blocks (matrix-core
// form).  Any other shape is not handled here (hipErrorNotSupported,
// nothing launched): the row-streaming kernel takes it.
hipError_t launch_fx(const RowsArgs &a, hipStream_t s, const char **name) {
    const int nb = a.K / QK;
    if ((a.x != nullptr && a.M != 1) || a.M < 1 || a.M > 4 || (nb > 32 && nb < 64) || nb > 64 * QMV_FX_WPB)
        return hipErrorNotSupported;
    if (a.ya != nullptr && (a.x == nullptr || a.xu != nullptr)) return hipErrorNotSupported;
    return a.qtype == 4 ? launch_q<4>(a, s, name) : launch_q<8>(a, s, name);
}

}  // namespace qmv
