// kernels_rows.hip -- weight-streaming products for a few activation rows
// (M = 1 .. 8) on gfx950: the decode matvec and the small-batch product.
//
// What is computed (Legacy-ISA ML Inference Runtime -- Design Spec,
// section 4 "Integer dot per block" and section 5 kernel interface):
//   y[m, r] = sum over blocks b of sumi(m, r, b) * dw(r, b) * dx(m, b),
//   sumi = exact int32 dot of the 32 weight and activation quants,
// for r in [r0, r1).  The spec's CPU kernels take 4 rows at a time so that
// one activation-block load serves 4 weight rows; here a wavefront takes 4
// rows at a time and each of its 64 lanes owns one block column of them.
//
// Layout of the work:
//   * the activation (M rows of K) is staged once per workgroup in LDS as
//     two 16-byte halves per block plus {dx, 8 * sum of quants}; with a
//     float32 activation (FX) the staging is the Q8_0 quantization itself,
//     8 lanes per 32-element block (coalesced 1 KiB loads per wavefront,
//     block max and quant sum by DPP within the 8 lanes), so the quantized
//     activation never leaves the chip;
//   * a wavefront walks "quads" of 4 weight rows; lane l takes blocks
//     l, l + 64, l + 128, ... of the 4 rows, so every weight load of the
//     wavefront is a contiguous 1 KiB (Q4_0) or 2 KiB (Q8_0) run per row
//     (global_load_dwordx4, non-temporal: weights are streamed once);
//   * the weight loads of the next step are issued before the current step
//     is computed (register double buffering), and the very first step's
//     loads are issued before the activation staging, so staging latency
//     hides under the first HBM round trip;
//   * int8 block dots use v_dot4_i32_i8.  Q4_0 nibbles are used as unsigned
//     bytes 0..15 (gfx950 has no mixed-sign dot4) and the -8 offset is
//     folded in exactly: sumi = dot(nibble, qx) - 8 * sum(qx);
//   * per lane, block sums are scaled and accumulated in fp32, then the
//     4 * M partial sums of a quad are reduced across the wavefront with a
//     transposing butterfly and stored by one lane each.
#include "device_common.h"
#include "launch.h"

#ifndef QMV_STAGE_FIRST
#define QMV_STAGE_FIRST 0
#endif

namespace qmv {
namespace {

template <int QT, int UJ>
struct WTile {
    static constexpr int QW = (QT == 8) ? 2 : 1;  // 16-byte words per block
    v4i w[UJ][4][QW];
    float dw[UJ][4];
};

template <int QT, int UJ>
__device__ __forceinline__ void load_tile(WTile<QT, UJ> &t, const int8_t *__restrict__ wq,
                                          const float *__restrict__ wd, int nb, int rb, int r1,
                                          int j0, int lane) {
    constexpr int QB = (QT == 8) ? 32 : 16;  // quant bytes per block
    const size_t rowbytes = (size_t)nb * QB;
#pragma unroll
    for (int u = 0; u < UJ; ++u) {
        int b = lane + 64 * (j0 + u);
        int bb = b < nb ? b : nb - 1;  // out-of-range lanes re-read a valid block; their scale is zeroed
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int row = min(rb + r, r1 - 1);  // rows past r1 re-read row r1 - 1; their result is not stored
            const v4i *p = reinterpret_cast<const v4i *>(wq + (size_t)row * rowbytes + (size_t)bb * QB);
            t.w[u][r][0] = __builtin_nontemporal_load(p);
            if constexpr (QT == 8) t.w[u][r][WTile<QT, UJ>::QW - 1] = __builtin_nontemporal_load(p + 1);
            t.dw[u][r] = __builtin_nontemporal_load(wd + (size_t)row * nb + bb);
        }
    }
}

template <int QT>
__device__ __forceinline__ int block_dot(const v4i *w, v4i xl, v4i xh, int sx8) {
    int s = 0;
    if constexpr (QT == 4) {
        // byte j of the 16: low nibble = element j, high nibble = element j + 16
        const unsigned m = 0x0F0F0F0Fu;
        s = dot4((unsigned)w[0].x & m, xl.x, s);
        s = dot4((unsigned)w[0].y & m, xl.y, s);
        s = dot4((unsigned)w[0].z & m, xl.z, s);
        s = dot4((unsigned)w[0].w & m, xl.w, s);
        s = dot4(((unsigned)w[0].x >> 4) & m, xh.x, s);
        s = dot4(((unsigned)w[0].y >> 4) & m, xh.y, s);
        s = dot4(((unsigned)w[0].z >> 4) & m, xh.z, s);
        s = dot4(((unsigned)w[0].w >> 4) & m, xh.w, s);
        s -= sx8;
    } else {
        s = dot4(w[0].x, xl.x, s);
        s = dot4(w[0].y, xl.y, s);
        s = dot4(w[0].z, xl.z, s);
        s = dot4(w[0].w, xl.w, s);
        s = dot4(w[1].x, xh.x, s);
        s = dot4(w[1].y, xh.y, s);
        s = dot4(w[1].z, xh.z, s);
        s = dot4(w[1].w, xh.w, s);
    }
    return s;
}

constexpr int next_pow2(int v) { return v <= 1 ? 1 : 2 * next_pow2((v + 1) / 2); }

// Activation staging, first half: issue the global loads of one batch of
// staging tasks into registers.  FX: a task is one float4 (8 tasks per
// 32-element block, aligned groups of 8 lanes, so a wavefront reads 1 KiB of
// contiguous activation per load).  Otherwise a task is one 16-byte half of
// a Q8_0 block (2 tasks per block).  Task indices past the end are
// redirected to the last block so that every load stays in bounds and every
// lane group stays complete; their results are not stored.
template <bool FX, int SU>
struct StageRegs {
    float4 v[FX ? SU : 1];
    v4i q[FX ? 1 : SU];
    float d[FX ? 1 : SU];
};

template <int M, bool FX, int SU>
__device__ __forceinline__ void stage_load(StageRegs<FX, SU> &st, int base, int ntask, int K,
                                           const float *__restrict__ x, const int8_t *__restrict__ xq,
                                           const float *__restrict__ xd) {
    const int nb = K >> 5;
#pragma unroll
    for (int i = 0; i < SU; ++i) {
        int e = base + i * (int)blockDim.x;
        if (FX) {
            if (e >= ntask) e = ntask - 8 + (e & 7);
            const int blk = e >> 3, c = e & 7;
            const int m = blk / nb, b = blk - m * nb;
            st.v[i] = *reinterpret_cast<const float4 *>(x + (size_t)m * K + (size_t)b * QK + 4 * c);
        } else {
            if (e >= ntask) e = ntask - 2 + (e & 1);
            const int blk = e >> 1, h = e & 1;
            const int m = blk / nb, b = blk - m * nb;
            st.q[i] = *reinterpret_cast<const v4i *>(xq + (size_t)m * K + (size_t)b * QK + 16 * h);
            st.d[i] = xd[(size_t)m * nb + b];
        }
    }
}

// Activation staging, second half: quantize (FX) or sum (pre-quantized) the
// loaded tasks and write the LDS layout.  All lanes run the cross-lane steps
// (DPP within groups of 8 or 2 lanes); only live tasks store.
template <int M, bool FX, int SU>
__device__ __forceinline__ void stage_store(const StageRegs<FX, SU> &st, int base, int ntask,
                                            v4i *xlo, v4i *xhi, float2 *meta) {
#pragma unroll
    for (int i = 0; i < SU; ++i) {
        const int e = base + i * (int)blockDim.x;
        const bool live = e < ntask;
        if (FX) {
            const int c = e & 7;
            const int blk = (live ? e : ntask - 8 + c) >> 3;
            float d;
            int s;
            const int pk = quant_q8_group8(st.v[i], d, s);
            if (live) {
                reinterpret_cast<int *>((c < 4) ? (xlo + blk) : (xhi + blk))[c & 3] = pk;
                if (c == 0) meta[blk] = make_float2(d, __int_as_float(8 * s));
            }
        } else {
            const int h = e & 1;
            const int blk = (live ? e : ntask - 2 + h) >> 1;
            const v4i v = st.q[i];
            int s = dot4(v.x, 0x01010101, dot4(v.y, 0x01010101, dot4(v.z, 0x01010101, dot4(v.w, 0x01010101, 0))));
            s += dpp_xor1(s);
            if (live) {
                (h ? xhi : xlo)[blk] = v;
                if (h == 0) meta[blk] = make_float2(st.d[i], __int_as_float(8 * s));
            }
        }
    }
}

template <int QT, int M, bool FX, int UJ, int WPB, int SU>
__global__ void __launch_bounds__(64 * WPB)
k_rows(float *__restrict__ y, const int8_t *__restrict__ wq, const float *__restrict__ wd,
       int32_t rows, int32_t K, const float *__restrict__ x, const int8_t *__restrict__ xq,
       const float *__restrict__ xd, int8_t *__restrict__ xq_out, float *__restrict__ xd_out,
       int32_t r0, int32_t r1) {
    constexpr int NV = next_pow2(4 * M);
    extern __shared__ __align__(16) unsigned char smem[];
    const int nb = K >> 5;
    v4i *xlo = reinterpret_cast<v4i *>(smem);   // [M][nb] quants 0..15 of each block
    v4i *xhi = xlo + M * nb;                    // [M][nb] quants 16..31
    float2 *meta = reinterpret_cast<float2 *>(xhi + M * nb);  // [M][nb] {dx, bits of 8 * sum(q)}

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = blockIdx.x * WPB + (tid >> 6);
    const int nwaves = gridDim.x * WPB;
    const int nquads = (r1 - r0 + 3) >> 2;
    const int nj = (nb + 63) >> 6;
    const int ntask = M * nb * (FX ? 8 : 2);

    // This wave's steps: quads wave, wave + nwaves, ...; each quad takes
    // nsq steps of UJ block columns.  The loop below is a software pipeline
    // whose every iteration issues exactly one step of weight loads with no
    // branch around them, so the compiler's wait counts stay exact (a load
    // under a branch makes the wait at the join conservative, which would
    // serialise the prefetch).
    const int nsq = (nj + UJ - 1) / UJ;
    const int myq = wave < nquads ? (nquads - 1 - wave) / nwaves + 1 : 0;
    const int T = myq * nsq;

    // Activation loads first (they hit L2 after the first workgroup touches
    // x), then the first weight step: loads return in issue order, so the
    // quantization below waits only for the activation.
    StageRegs<FX, SU> st;
    stage_load<M, FX, SU>(st, tid, ntask, K, x, xq, xd);

    WTile<QT, UJ> ta, tb;  // ping-pong weight tiles (no register copies between steps)
#if !QMV_STAGE_FIRST
    load_tile<QT, UJ>(ta, wq, wd, nb, r0 + 4 * min(wave, nquads - 1), r1, 0, lane);
    __builtin_amdgcn_sched_barrier(0);  // keep every load above ahead of the quantization below
#endif

    stage_store<M, FX, SU>(st, tid, ntask, xlo, xhi, meta);
#if QMV_STAGE_FIRST
    __builtin_amdgcn_sched_barrier(0);
    load_tile<QT, UJ>(ta, wq, wd, nb, r0 + 4 * min(wave, nquads - 1), r1, 0, lane);
#endif
    for (int base = tid + SU * 64 * WPB; base < ntask; base += SU * 64 * WPB) {  // large K: more batches
        stage_load<M, FX, SU>(st, base, ntask, K, x, xq, xd);
        stage_store<M, FX, SU>(st, base, ntask, xlo, xhi, meta);
    }
    __syncthreads();
    if (FX && xq_out != nullptr && blockIdx.x == 0) {  // optional copy of the quantized activation
        for (int blk = tid; blk < M * nb; blk += 64 * WPB) {
            const int m = blk / nb, b = blk - m * nb;
            v4i *dst = reinterpret_cast<v4i *>(xq_out + (size_t)m * K + (size_t)b * QK);
            dst[0] = xlo[blk];
            dst[1] = xhi[blk];
            xd_out[(size_t)m * nb + b] = meta[blk].x;
        }
    }
    if (T == 0) return;  // no barrier follows

    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.0f;

    auto compute = [&](const WTile<QT, UJ> &w, int j0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < UJ; ++u) {
            const int b = lane + 64 * (j0 + u);
            const bool ok = b < nb;
            const int bb = ok ? b : nb - 1;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const v4i xl = xlo[m * nb + bb];
                const v4i xh = xhi[m * nb + bb];
                const float2 mt = meta[m * nb + bb];
                const float dx = ok ? mt.x : 0.0f;
                const int sx8 = __float_as_int(mt.y);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = block_dot<QT>(w.w[u][r], xl, xh, sx8);
                    acc[m * 4 + r] = fmaf((float)s, w.dw[u][r] * dx, acc[m * 4 + r]);
                }
            }
        }
    };
    // quad finished: reduce the 4*M partial sums over the wavefront, store, reset
    auto finish_quad = [&](int q) __attribute__((always_inline)) {
        const float tot = wave_reduce_transpose<NV>(acc);
        const int idx = reduce_index<NV>(lane);
        const int m = idx >> 2, r = idx & 3;
        const int row = r0 + 4 * q + r;
        if (reduce_owner<NV>(lane) && m < M && row < r1) y[(size_t)m * rows + row] = tot;
#pragma unroll
        for (int i = 0; i < NV; ++i) acc[i] = 0.0f;
    };

    // Step t+1 is always in flight while step t is computed.  Tiles ta / tb
    // alternate, so there are no register copies (a copy of a tile whose
    // loads are still in flight would force a wait for them).
    int quad = wave, jj = 0;     // step t
    auto advance = [&](int &q, int &j) __attribute__((always_inline)) {
        j += UJ;
        if (j >= nj) {
            j = 0;
            q += nwaves;
        }
    };
    int t = 0;
    while (t + 2 < T) {
        int q1 = quad, j1 = jj;
        advance(q1, j1);
        load_tile<QT, UJ>(tb, wq, wd, nb, r0 + 4 * q1, r1, j1, lane);
        __builtin_amdgcn_sched_barrier(0);  // loads of the next step go out before this step's math
        compute(ta, jj);
        if (j1 == 0) finish_quad(quad);
        int q2 = q1, j2 = j1;
        advance(q2, j2);
        load_tile<QT, UJ>(ta, wq, wd, nb, r0 + 4 * q2, r1, j2, lane);
        __builtin_amdgcn_sched_barrier(0);
        compute(tb, j1);
        if (j2 == 0) finish_quad(q1);
        quad = q2;
        jj = j2;
        t += 2;
    }
    if (t + 1 < T) {
        int q1 = quad, j1 = jj;
        advance(q1, j1);
        load_tile<QT, UJ>(tb, wq, wd, nb, r0 + 4 * q1, r1, j1, lane);
        __builtin_amdgcn_sched_barrier(0);  // loads of the next step go out before this step's math
        compute(ta, jj);
        if (j1 == 0) finish_quad(quad);
        compute(tb, j1);
        finish_quad(q1);
    } else {
        compute(ta, jj);
        finish_quad(quad);
    }
}

template <int QT, int M, bool FX, int UJ, int WPB, int SU>
hipError_t launch_rows_t(const RowsArgs &a, hipStream_t s, const char **name) {
    static char kname[96];
    auto kern = k_rows<QT, M, FX, UJ, WPB, SU>;
    const int nb = a.K / QK;
    const size_t lds = (size_t)M * nb * 40;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int nquads = (a.r1 - a.r0 + 3) / 4;
    int grid = (nquads + WPB - 1) / WPB;
    if (grid > a.max_groups) grid = a.max_groups;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WPB), lds, s, a.y, a.wq, a.wd, a.rows, a.K, a.x, a.xq,
                       a.xd, a.xq_out, a.xd_out, a.r0, a.r1);
    if (kname[0] == 0) snprintf(kname, sizeof kname, "rows_q%d_m%d%s_u%d_w%d_s%d", QT, M, FX ? "_fx" : "", UJ, WPB, SU);
    *name = kname;
    return hipGetLastError();
}

// Staging batch size: tasks per thread per batch (one batch covers the
// whole activation of the common shapes).
template <int QT, int M, bool FX, int UJ, int WPB>
hipError_t launch_rows_s(const RowsArgs &a, hipStream_t s, const char **name) {
    const int ntask = M * (a.K / QK) * (FX ? 8 : 2);
    const int per = (ntask + 64 * WPB - 1) / (64 * WPB);
    if (per <= 1) return launch_rows_t<QT, M, FX, UJ, WPB, 1>(a, s, name);
    if (per <= 2) return launch_rows_t<QT, M, FX, UJ, WPB, 2>(a, s, name);
    if (per <= 4) return launch_rows_t<QT, M, FX, UJ, WPB, 4>(a, s, name);
    return launch_rows_t<QT, M, FX, UJ, WPB, 6>(a, s, name);
}

template <int QT, int M, bool FX>
hipError_t launch_rows_u(const RowsArgs &a, hipStream_t s, const char **name) {
    const int nj = (a.K / QK + 63) / 64;
#ifdef QMV_TUNE_WPB
    constexpr int WPB = QMV_TUNE_WPB;
#else
    constexpr int WPB = 8;
#endif
#ifdef QMV_TUNE_UJ
    if (QMV_TUNE_UJ == 2 && nj >= 2 && QT == 4) return launch_rows_s<QT, M, FX, 2, WPB>(a, s, name);
    return launch_rows_s<QT, M, FX, 1, WPB>(a, s, name);
#else
    if (nj >= 2 && QT == 4) return launch_rows_s<QT, M, FX, 2, WPB>(a, s, name);
    return launch_rows_s<QT, M, FX, 1, WPB>(a, s, name);
#endif
}

template <int QT>
hipError_t launch_rows_q(const RowsArgs &a, hipStream_t s, const char **name) {
    if (a.x != nullptr) return launch_rows_u<QT, 1, true>(a, s, name);
    switch (a.M) {
        case 1: return launch_rows_u<QT, 1, false>(a, s, name);
        case 2: return launch_rows_u<QT, 2, false>(a, s, name);
        case 3: return launch_rows_u<QT, 3, false>(a, s, name);
        case 4: return launch_rows_u<QT, 4, false>(a, s, name);
        case 5: return launch_rows_u<QT, 5, false>(a, s, name);
        case 6: return launch_rows_u<QT, 6, false>(a, s, name);
        case 7: return launch_rows_u<QT, 7, false>(a, s, name);
        case 8: return launch_rows_u<QT, 8, false>(a, s, name);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_rows(const RowsArgs &a, hipStream_t s, const char **name) {
    return a.qtype == 4 ? launch_rows_q<4>(a, s, name) : launch_rows_q<8>(a, s, name);
}

}  // namespace qmv
