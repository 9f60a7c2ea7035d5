// kernels_fx.hip -- the decode matvec with the activation quantized inside
// the kernel (M = 1, float32 x), for K of 2048 .. 16384.
//
// What is computed (Legacy-ISA ML Inference Runtime -- Design Spec,
// section 4 "Q8 quantization" and "Integer dot per block", section 5
// kernel interface and rounding rule):
//   qx, dx = Q8_0(x)                       per 32-element block
//   y[r]   = sum over blocks b of sumi(r, b) * dw(r, b) * dx(b),
//   sumi   = exact int32 dot of the 32 weight quants and qx,
// for r in [r0, r1).
//
// Layout on the chip.  One workgroup per compute unit owns a contiguous
// range of rows; its wavefronts split K: wavefront w owns blocks
// [w S, w S + S) of every row of the range (S = ceil(K / 32 / waves)).  So a
// wavefront needs only its own slice of x: it loads that slice (one block
// per lane), quantizes it in registers and shares it with its own lanes
// through a private LDS region -- no workgroup barrier stands between the
// activation and the first block dot, and x is read and quantized once per
// workgroup.  The memory system accepts only a bounded number of
// outstanding loads per compute unit and stalls a wavefront at a load it
// cannot yet accept; so each wavefront first issues its activation loads,
// then only the first D - 1 passes of weights, quantizes while those are in
// flight, and then runs a software pipeline over passes: issue the loads of
// pass j + D - 1, then compute pass j.  A wavefront stalled at a load leaves
// the vector ALU to the others.
//
// A pass is 64 / T rows: lane l takes row l / T of the pass and the blocks
// c = l % T + T k (k < NBL) of its wavefront's slice, so each group of T
// lanes reads T consecutive blocks of one row (T * 16 or T * 32 contiguous
// quant bytes).  The T lanes of a row are summed with row-shift DPP adds
// (a fixed order), the wavefronts' slice sums of a row are added in LDS in
// wavefront order, and one lane stores y[r]: repeated calls give identical
// bits.
//
// Loads use raw buffer descriptors whose range covers only this
// workgroup's rows, and every variable part of an address is in the
// per-lane offset, which the hardware range-checks: rows past r1, blocks
// past the slice and passes past the last read zeros without touching
// memory.
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
// per compute unit.
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
#ifndef QMV_FX_WG_PER_CU
#define QMV_FX_WG_PER_CU 1
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

template <int QT, int T, int NBL, int D, int D0, int WPB, bool KS>
__global__ void __launch_bounds__(64 * WPB)
k_fx(float *__restrict__ y, const int8_t *__restrict__ wq, const float *__restrict__ wd, int32_t K,
     const float *__restrict__ x, int8_t *__restrict__ xq_out, float *__restrict__ xd_out, int32_t r0, int32_t r1,
     int32_t rw) {
    constexpr int PASS = 64 / T;               // rows per pass
    constexpr int QB = (QT == 8) ? 32 : 16;    // quant bytes per block
    static_assert(T * NBL <= 64 && (T * NBL) % 16 == 0, "a slice is at most 64 blocks, loaded 16 blocks at a time");
    static_assert(D0 >= 0 && D0 <= D - 1, "passes issued before the quantization");
    __shared__ v4i s_lo[WPB][64], s_hi[WPB][64];
    __shared__ float s_dx[WPB][64];
    __shared__ int s_sx[WPB][64];
    extern __shared__ float s_red[];           // [WPB][rw] slice sums

    const int nb = K >> 5;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // KS: the wavefronts split K (slice of S blocks each) and share every
    // row; otherwise every wavefront holds all of K and takes every WPB-th
    // pass of rows
    const int S = KS ? (nb + WPB - 1) / WPB : nb;
    const int kb0 = KS ? min(wid * S, nb) : 0;
    const int ns = min(S, nb - kb0);           // blocks in this wavefront's slice
    const int g0 = r0 + blockIdx.x * rw;       // this workgroup's rows g0 .. g1 - 1
    const int g1 = min(r1, g0 + rw);
    const int nrp = (g1 - g0 + PASS - 1) / PASS;  // passes of the workgroup
    const int npass = KS ? nrp : (nrp + WPB - 1) / WPB;  // passes of this wavefront
    const int pstride = KS ? 1 : WPB;          // pass j of this wavefront = workgroup pass j * pstride + pfirst
    const int pfirst = KS ? 0 : wid;

    // 1. this wavefront's activation slice, coalesced: round k covers
    //    blocks kb0 + 16 k .. kb0 + 16 k + 15, lane l holding floats
    //    8 (l % 4) .. 8 (l % 4) + 7 of block kb0 + 16 k + l / 4
    constexpr int NR = T * NBL / 16;           // rounds of 16 blocks
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, K * 4);
    float4 xa[NR], xb[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const int b = 16 * k + (lane >> 2);
        const int o = b < ns ? (kb0 + b) * 128 + 32 * (lane & 3) : kOOB;
        xa[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 0));
        xb[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rx, o + 16, 0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);  // the activation requests go out first
#if QMV_FX_XBAR
    __builtin_amdgcn_s_barrier();       // ... before any wavefront's weight requests
    __builtin_amdgcn_sched_barrier(0);
#endif

    // 2. the first D - 1 passes of weights
    const int rows_here = g1 - g0;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(wq + (size_t)g0 * nb * QB, rows_here * nb * QB);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(wd + (size_t)g0 * nb, rows_here * nb * 4);
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
    auto load = [&](Pass<QT, NBL> &p, int j) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < NBL; ++k) {
            // offsets of passes at or beyond npass fall outside the range
            const int a = oq[k] + j * pq, b = od[k] + j * pd;
            p.w[k][0] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rq, a, 0, kNT));
            if constexpr (QT == 8)
                p.w[k][1] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rq, a + 16, 0, kNT));
            p.dw[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, b, 0, kNT));
        }
    };
    Pass<QT, NBL> ring[D];
#pragma unroll
    for (int d = 0; d < D0; ++d) load(ring[d], d);
    __builtin_amdgcn_sched_barrier(0);

    // 3. quantize the slice, 4 lanes per block (lanes past the slice hold
    //    zeros), into the private LDS region -- no branch, so that the
    //    activation loads stay ahead of the weight loads
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        const int b = 16 * k + (lane >> 2), c = lane & 3;
        float d;
        int qs;
        const int2 pk = quant_q8_group4(xa[k], xb[k], d, qs);
        *reinterpret_cast<int2 *>(reinterpret_cast<int *>(c < 2 ? &s_lo[wid][b] : &s_hi[wid][b]) + 2 * (c & 1)) = pk;
        if (c == 0) {
            s_dx[wid][b] = d;
            s_sx[wid][b] = -8 * qs;
        }
        if (xq_out != nullptr && blockIdx.x == 0 && b < ns) {  // optional copy of the quantized activation
            reinterpret_cast<int2 *>(xq_out + (size_t)(kb0 + b) * QK)[c] = pk;
            if (c == 0) xd_out[kb0 + b] = d;
        }
    }
    // LDS operations of one wavefront complete in order: once this
    // wavefront's writes are done, all of its lanes read them
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    v4i xl[NBL], xh[NBL];
    float dx[NBL];
    int sx[NBL];
#pragma unroll
    for (int k = 0; k < NBL; ++k) {
        const int c = lane % T + T * k;
        const bool ok = c < ns;
        const int cc = ok ? c : 0;
        xl[k] = s_lo[wid][cc];
        xh[k] = s_hi[wid][cc];
        dx[k] = ok ? s_dx[wid][cc] : 0.0f;
        sx[k] = s_sx[wid][cc];
    }

    // the rest of the first D - 1 passes
#pragma unroll
    for (int d = D0; d < D - 1; ++d) load(ring[d], d);

    // 4. passes: loads of pass j + D - 1 in flight while pass j is computed
    float *red = s_red + wid * rw;
    const int nit = (npass + D - 1) / D;
    for (int it = 0; it < nit; ++it) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int j = it * D + d;
            load(ring[(d + D - 1) % D], j + D - 1);
            const Pass<QT, NBL> &p = ring[d];
            float a = 0.0f;
#pragma unroll
            for (int k = 0; k < NBL; ++k) {
                int s;
                if constexpr (QT == 4) {
                    const unsigned m = 0x0F0F0F0Fu;
                    const v4i w = p.w[k][0];
                    s = dot4((unsigned)w.x & m, xl[k].x, sx[k]);  // starts at -8 * sum(qx)
                    s = dot4((unsigned)w.y & m, xl[k].y, s);
                    s = dot4((unsigned)w.z & m, xl[k].z, s);
                    s = dot4((unsigned)w.w & m, xl[k].w, s);
                    s = dot4(((unsigned)w.x >> 4) & m, xh[k].x, s);
                    s = dot4(((unsigned)w.y >> 4) & m, xh[k].y, s);
                    s = dot4(((unsigned)w.z >> 4) & m, xh[k].z, s);
                    s = dot4(((unsigned)w.w >> 4) & m, xh[k].w, s);
                } else {
                    s = dot4(p.w[k][0].x, xl[k].x, 0);
                    s = dot4(p.w[k][0].y, xl[k].y, s);
                    s = dot4(p.w[k][0].z, xl[k].z, s);
                    s = dot4(p.w[k][0].w, xl[k].w, s);
                    s = dot4(p.w[k][1].x, xh[k].x, s);
                    s = dot4(p.w[k][1].y, xh[k].y, s);
                    s = dot4(p.w[k][1].z, xh[k].z, s);
                    s = dot4(p.w[k][1].w, xh[k].w, s);
                }
                a = fmaf((float)s, p.dw[k] * dx[k], a);
            }
            a = group_sum<T>(a);
            if constexpr (KS) {
                const int r = j * PASS + prow;
                if (lane % T == T - 1 && j < npass && r < rw) red[r] = a;
            } else {  // whole rows: store directly
                const int r = (j * pstride + pfirst) * PASS + prow;
                if (lane % T == T - 1 && j < npass && r < rows_here) y[g0 + r] = a;
            }
        }
    }

    if constexpr (!KS) return;
    // 5. add the wavefronts' slice sums of each row in wavefront order
    __syncthreads();
    for (int r = threadIdx.x; r < rows_here; r += 64 * WPB) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < WPB; ++w) s += s_red[w * rw + r];
        y[g0 + r] = s;
    }
}

template <int QT, int T, int NBL, int D, int WPB, bool KS = true>
hipError_t launch_t(const RowsArgs &a, int rw, hipStream_t s, const char **name) {
    static char kname[64];
    constexpr int D0 = QMV_FX_D0 < D - 1 ? QMV_FX_D0 : D - 1;
    auto kern = k_fx<QT, T, NBL, D, D0, WPB, KS>;
    const int nrows = a.r1 - a.r0;
    const int grid = (nrows + rw - 1) / rw;
    const size_t lds = KS ? (size_t)WPB * rw * 4 : 0;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WPB), lds, s, a.y, a.wq, a.wd, a.K, a.x, a.xq_out, a.xd_out,
                       a.r0, a.r1, rw);
    if (kname[0] == 0) snprintf(kname, sizeof kname, "fx_q%d_t%d_n%d_d%d_w%d%s", QT, T, NBL, D, WPB, KS ? "" : "_rows");
    *name = kname;
    return hipGetLastError();
}

template <int QT>
hipError_t launch_q(const RowsArgs &a, hipStream_t s, const char **name) {
    constexpr int W = QMV_FX_WPB, D = QMV_FX_D;
    const int nb = a.K / QK;
    const int S = (nb + W - 1) / W;
    const int nrows = a.r1 - a.r0;
    const int groups = a.num_cu * QMV_FX_WG_PER_CU;
    // rows per workgroup: a whole number of passes, at most one workgroup
    // per compute unit
    // (capped so that the slice sums fit in LDS)
    // (capped so that the slice sums fit in LDS; whole-row workgroups need no
    // slice sums)
    auto rows_per = [&](int pass) {
        const int want = ((nrows + groups - 1) / groups + pass - 1) / pass * pass;
        return pass > 4 ? want : min(1024, want);
    };
    if (nb <= 16) return launch_t<QT, 16, 1, D, W, false>(a, rows_per(4 * W), s, name);
    if (nb <= 32) return launch_t<QT, 32, 1, D, W, false>(a, rows_per(2 * W), s, name);
    if (S <= 16) return launch_t<QT, 16, 1, D, W>(a, rows_per(4), s, name);
    if (S <= 32) return launch_t<QT, 16, 2, D, W>(a, rows_per(4), s, name);
    if (S <= 48) return launch_t<QT, 16, 3, D, W>(a, rows_per(4), s, name);
    return launch_t<QT, 16, 4, D, W>(a, rows_per(4), s, name);
}

}  // namespace

// Fused M = 1 matvec for K / 32 <= 32 (whole rows per wavefront) and
// 64 <= K / 32 <= 64 * waves (K split over the wavefronts); any other shape
// is not handled here (hipErrorNotSupported, nothing launched).
hipError_t launch_fx(const RowsArgs &a, hipStream_t s, const char **name) {
    const int nb = a.K / QK;
    if (a.x == nullptr || a.M != 1 || (nb > 32 && nb < 64) || nb > 64 * QMV_FX_WPB) return hipErrorNotSupported;
    return a.qtype == 4 ? launch_q<4>(a, s, name) : launch_q<8>(a, s, name);
}

}  // namespace qmv
