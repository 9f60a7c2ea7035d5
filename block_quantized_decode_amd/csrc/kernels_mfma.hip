// kernels_mfma.hip -- the product for many activation rows on the gfx950
// int8 matrix cores.
//
// What is computed (Legacy-ISA ML Inference Runtime -- Design Spec, section
// 4, the per-block integer dot and its scaled accumulation, applied to every
// activation row):
//   Y[m, r] = sum over blocks b of sumi(m, r, b) * dw(r, b) * dx(m, b),
//   sumi(m, r, b) = exact int32 dot of the 32 quants of weight row r and
//   activation row m in block b.
//
// One matrix instruction per block and 16 x 16 tile: v_mfma_i32_16x16x32_i8
// contracts exactly one 32-element block, so its int32 result IS sumi for
// 16 weight rows x 16 activation rows, and the scales are applied in fp32
// right after it: acc += (float)sumi * (dx * dw).  Operand lane l supplies
// row l % 16 (weight row for the A operand, activation row for B) and the
// block's elements 8 g .. 8 g + 7 with g = l / 16; both operands use the
// same element choice, so the order in which the instruction walks the 32
// products does not matter.  Result register v of lane l belongs to weight
// row 4 g + v and activation row l % 16 (the gfx950 accumulator layout).
//
// Data movement.  In the operand layout consecutive lanes read different
// rows, which the vector memory path serves at a fraction of its rate, so
// nothing is loaded in that layout: every tile is loaded with 16 (or 4) bytes
// per lane such that each group of 4 consecutive lanes reads one contiguous
// span of one row, into a ring of D register stages (D - 1 stages stay in
// flight to cover memory latency), then written to a per-wavefront LDS
// stage buffer and read back in the operand layout.  The 16-byte pieces of
// each row sit in LDS under an XOR swizzle of the piece index, so that the
// operand reads of 32 lanes fall in distinct banks.
//
// Work layout: a workgroup owns 16 weight rows and all activation rows (up
// to 64 per launch); its WPB wavefronts split K into contiguous ranges of
// whole stages (4 blocks), so every weight byte is read from memory once per
// launch.  Q4_0 nibbles become signed bytes (nibble - 8) in registers.  At
// the end the wavefronts' partial tiles are summed in LDS in a fixed order
// (the result does not depend on timing) and stored with consecutive lanes
// on consecutive weight rows.
#include <stdio.h>

#include "device_common.h"
#include "launch.h"

namespace qmv {
namespace {

constexpr int kBufFlags = 0x00020000;  // buffer descriptor word 3: raw 32-bit data
constexpr int kOOB = 0x40000000;       // an offset beyond every descriptor range used here
constexpr int kNT = 2;                 // non-temporal: weights are read once
constexpr int KU = 4;                  // blocks per stage

typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, kBufFlags);
}
// The offset goes through an empty asm so that the compiler keeps one
// unconditional load (it would otherwise branch around loads whose offset
// is a select on a uniform condition, and branches cost the pipelined loop
// its precise waits).
template <int AUX>
__device__ __forceinline__ v4i load16(__amdgpu_buffer_rsrc_t r, int off) {
    asm volatile("" : "+v"(off));
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}
template <int AUX>
__device__ __forceinline__ float load4(__amdgpu_buffer_rsrc_t r, int off) {
    asm volatile("" : "+v"(off));
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX));
}

// Signed bytes nibble - 8 from 4 nibbles held one per byte (0..15): adding
// 0x78 to each byte cannot carry out of it, then flipping bit 7 subtracts
// 0x80, leaving (nibble + 0x78 - 0x80) = nibble - 8 as a signed byte.
__device__ __forceinline__ int nib_to_s8(unsigned n) { return (int)((n + 0x78787878u) ^ 0x80808080u); }

// Q4_0 operand: elements 8g .. 8g + 7 are the low nibbles (g < 2) or the
// high nibbles (g >= 2) of bytes 8 (g % 2) .. 8 (g % 2) + 7.
__device__ __forceinline__ v2i q4_operand(v2i raw, bool high) {
    const unsigned a = (unsigned)raw.x, b = (unsigned)raw.y;
    return (v2i){nib_to_s8((high ? (a >> 4) : a) & 0x0F0F0F0Fu), nib_to_s8((high ? (b >> 4) : b) & 0x0F0F0F0Fu)};
}

__device__ __forceinline__ v4i mfma16(v2i a, v2i b) {
    const v4i z = {};
    return __builtin_amdgcn_mfma_i32_16x16x32_i8(__builtin_bit_cast(long, a), __builtin_bit_cast(long, b), z, 0, 0,
                                                 0);
}

// Piece swizzles: which 16-byte piece of a row sits at position s of the
// row's LDS image.  Rows of 128 bytes: q = s ^ ((r >> 1) & 7); rows of 64
// bytes: q = s ^ ((r >> 2) & 3).  Both are involutions on the row's pieces.
__device__ __forceinline__ int swz128(int s, int r) { return s ^ ((r >> 1) & 7); }
__device__ __forceinline__ int swz64(int s, int r) { return s ^ ((r >> 2) & 3); }

// LDS stage buffer of one wavefront (bytes): weight quants (16 rows x 4
// blocks x QB), weight scales (16 x 4 floats), then per activation row tile
// quants (16 rows x 128 B) and scales (16 x 4 floats).
template <int QT, int MT>
struct Lds {
    static constexpr int QB = (QT == 8) ? 32 : 16;
    static constexpr int WQ = 16 * KU * QB;
    static constexpr int WD = WQ;                // weight scales
    static constexpr int X0 = WQ + 256;          // first activation row tile
    static constexpr int XT = 2048 + 256;        // one activation row tile
    static constexpr int WAVE = X0 + MT * XT;
};

// One stage in registers: this lane's share of the coalesced loads.
template <int QT, int MT>
struct Stage {
    v4i w[QT == 8 ? 2 : 1];
    float dw;
    v4i x[MT][2];
    float dx[MT];
};

template <int QT, int MT, int WPB, int D>
__global__ void __launch_bounds__(64 * WPB)
k_gemm_mfma(float *__restrict__ Y, const int8_t *__restrict__ wq, const float *__restrict__ wd, int32_t rows,
            int32_t K, const int8_t *__restrict__ xq, const float *__restrict__ xd, int32_t M, int32_t r0,
            int32_t r1) {
    typedef Lds<QT, MT> L;
    typedef Stage<QT, MT> St;
    constexpr int QB = L::QB;
    __shared__ __align__(16) unsigned char smem[WPB * L::WAVE];

    const int nb = K >> 5;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = r0 + blockIdx.x * 16;  // weight rows n0 .. n0 + 15
    unsigned char *const buf = smem + wid * L::WAVE;

    // descriptors cover only valid data: loads beyond them return zeros
    const int wrows = min(16, r1 - n0);
    const __amdgpu_buffer_rsrc_t rwq = make_rsrc(wq + (size_t)n0 * nb * QB, wrows * nb * QB);
    const __amdgpu_buffer_rsrc_t rwd = make_rsrc(wd + (size_t)n0 * nb, wrows * nb * 4);
    const __amdgpu_buffer_rsrc_t rxq = make_rsrc(xq, M * K);
    const __amdgpu_buffer_rsrc_t rxd = make_rsrc(xd, M * nb * 4);

    // load roles of this lane (offsets at block 0); the lane writes what it
    // loaded to byte 16 * lane (quants) or 4 * lane (scales) of its tile
    //   128-byte rows (Q8 weights, activations): row 8t + lane/8, position lane%8
    //   64-byte rows (Q4 weights): row lane/4, position lane%4
    //   scales: row lane/4, block lane%4
    const int r128 = lane >> 3;
    const int q128[2] = {swz128(lane & 7, r128), swz128(lane & 7, r128 + 8)};
    int wq_off[QT == 8 ? 2 : 1];
    if constexpr (QT == 8) {
        wq_off[0] = r128 * nb * 32 + 16 * q128[0];
        wq_off[1] = (r128 + 8) * nb * 32 + 16 * q128[1];
    } else {
        wq_off[0] = (lane >> 2) * nb * 16 + 16 * swz64(lane & 3, lane >> 2);
    }
    const int wd_off = ((lane >> 2) * nb + (lane & 3)) * 4;
    int x_off[MT][2], xd_off[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int m = mt * 16 + 8 * t + r128;
            x_off[mt][t] = m < M ? m * K + 16 * q128[t] : kOOB;
        }
        const int m = mt * 16 + (lane >> 2);
        xd_off[mt] = m < M ? (m * nb + (lane & 3)) * 4 : kOOB;
    }

#ifndef QMV_GEMM_INTERLEAVE
#define QMV_GEMM_INTERLEAVE 1
#endif
#if QMV_GEMM_INTERLEAVE
    // this wavefront's stages: wid, wid + WPB, wid + 2 WPB, ... (the
    // wavefronts of a workgroup read adjacent spans of each row together)
    const int nu = (nb + KU - 1) / KU;
    const int nst = (nu - wid + WPB - 1) / WPB;
    const int kb0 = KU * wid, kstep = KU * WPB, kb1 = nb;
#else
    // this wavefront's blocks [kb0, kb1): whole stages
    const int nu = (nb + KU - 1) / KU;
    const int kb0 = KU * ((wid * nu) / WPB);
    const int kb1 = min(nb, KU * (((wid + 1) * nu) / WPB));
    const int nst = (kb1 - kb0 + KU - 1) / KU;
    const int kstep = KU;
#endif

    // Loads of blocks outside [kb0, kb1) read zeros (per lane: each lane's
    // piece belongs to one block), so a stage past the range, or the tail of
    // a partial stage, contributes exactly 0 and the loop needs no branches.
    const int wblk = (QT == 8) ? (q128[0] >> 1) : swz64(lane & 3, lane >> 2);  // block of this lane's weight piece
    const int xblk[2] = {q128[0] >> 1, q128[1] >> 1};
    auto load = [&](St &s, int st) __attribute__((always_inline)) {
        const int kb = kb0 + kstep * st;
        const bool live = st < nst;
        if constexpr (QT == 8) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
                s.w[t] = load16<kNT>(rwq, live && kb + (q128[t] >> 1) < kb1 ? wq_off[t] + kb * QB : kOOB);
        } else {
            s.w[0] = load16<kNT>(rwq, live && kb + wblk < kb1 ? wq_off[0] + kb * QB : kOOB);
        }
        s.dw = load4<kNT>(rwd, live && kb + (lane & 3) < kb1 ? wd_off + 4 * kb : kOOB);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
                s.x[mt][t] = load16<0>(rxq, live && kb + xblk[t] < kb1 ? x_off[mt][t] + 32 * kb : kOOB);
            s.dx[mt] = load4<0>(rxd, live && kb + (lane & 3) < kb1 ? xd_off[mt] + 4 * kb : kOOB);
        }
    };
    auto stash = [&](const St &s) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < (QT == 8 ? 2 : 1); ++t) *reinterpret_cast<v4i *>(buf + 1024 * t + 16 * lane) = s.w[t];
        *reinterpret_cast<float *>(buf + L::WD + 4 * lane) = s.dw;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
                *reinterpret_cast<v4i *>(buf + L::X0 + mt * L::XT + 1024 * t + 16 * lane) = s.x[mt][t];
            *reinterpret_cast<float *>(buf + L::X0 + mt * L::XT + 2048 + 4 * lane) = s.dx[mt];
        }
    };

    // operand read offsets of this lane
    const int i = lane & 15, g = lane >> 4;
    const bool q4_high = g >= 2;
    int a_off[KU], b_off[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
        b_off[u] = 128 * i + 16 * swz128(2 * u + (g >> 1), i) + 8 * (g & 1);
        a_off[u] = (QT == 8) ? b_off[u] : 64 * i + 16 * swz64(u, i) + 8 * (g & 1);
    }

    float acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[mt][v] = 0.0f;

    auto compute = [&]() __attribute__((always_inline)) {
        v4f dw4[4], dx4[MT];
#pragma unroll
        for (int v = 0; v < 4; ++v) dw4[v] = *reinterpret_cast<const v4f *>(buf + L::WD + 16 * (4 * g + v));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            dx4[mt] = *reinterpret_cast<const v4f *>(buf + L::X0 + mt * L::XT + 2048 + 16 * i);
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            v2i a = *reinterpret_cast<const v2i *>(buf + a_off[u]);
            if constexpr (QT == 4) a = q4_operand(a, q4_high);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const v2i b = *reinterpret_cast<const v2i *>(buf + L::X0 + mt * L::XT + b_off[u]);
                const v4i c = mfma16(a, b);
                const float dx = dx4[mt][u];
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[mt][v] = fmaf((float)c[v], dx * dw4[v][u], acc[mt][v]);
            }
        }
    };

    // ring of D register stages; the loop is unrolled by D so that every
    // stage lives in fixed registers, and runs whole groups of D stages
    St ring[D];
#pragma unroll
    for (int d = 0; d < D - 1; ++d) load(ring[d], d);
    for (int st0 = 0; st0 < nst; st0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load(ring[(d + D - 1) % D], st0 + d + D - 1);
            stash(ring[d]);  // the previous stage's reads were issued before these writes
            compute();
            __builtin_amdgcn_sched_barrier(0);  // keep the stages apart: register pressure
        }
    }

    // partial tiles of the wavefronts -> each wavefront's own LDS, then a
    // fixed-order sum per output
    constexpr int PSTRIDE = L::WAVE / 4;  // floats between the wavefronts' partial tiles
    static_assert(MT * 1024 <= L::WAVE && L::WAVE % 16 == 0, "a partial tile must fit in a stage buffer");
    float *part = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) part[wid * PSTRIDE + (mt * 4 + v) * 64 + lane] = acc[mt][v];
    __syncthreads();
    for (int e = threadIdx.x; e < MT * 256; e += 64 * WPB) {
        const int nl = e & 15, ml = e >> 4;  // weight row n0 + nl, activation row ml
        const int mt = ml >> 4, l = (ml & 15) + 16 * (nl >> 2), v = nl & 3;
        float s = 0.0f;
        for (int w = 0; w < WPB; ++w) s += part[w * PSTRIDE + (mt * 4 + v) * 64 + l];
        const int n = n0 + nl;
        if (ml < M && n < r1) Y[(size_t)ml * rows + n] = s;
    }
}

template <int QT, int MT, int WPB, int D>
hipError_t launch_cfg(const GemmArgs &a, hipStream_t s, const char **name) {
    static char kname[64];
    static_assert(WPB * Lds<QT, MT>::WAVE <= 64 * 1024, "static LDS budget");
    const int grid = (a.r1 - a.r0 + 15) / 16;
    hipLaunchKernelGGL((k_gemm_mfma<QT, MT, WPB, D>), dim3(grid), dim3(64 * WPB), 0, s, a.Y, a.wq, a.wd, a.rows,
                       a.K, a.xq, a.xd, a.M, a.r0, a.r1);
    if (kname[0] == 0) snprintf(kname, sizeof kname, "gemm_mfma_q%d_mt%d_w%d_d%d", QT, MT, WPB, D);
    *name = kname;
    return hipGetLastError();
}

#ifndef QMV_GEMM_D
#define QMV_GEMM_D 3  // register stages (D - 1 in flight)
#endif
#ifndef QMV_GEMM_WPB
#define QMV_GEMM_WPB 4  // wavefronts per workgroup
#endif

template <int QT>
hipError_t launch_q(const GemmArgs &a, hipStream_t s, const char **name) {
    constexpr int D = QMV_GEMM_D, W = QMV_GEMM_WPB;
    switch ((a.M + 15) / 16) {
        case 1: return launch_cfg<QT, 1, W, D>(a, s, name);
        case 2: return launch_cfg<QT, 2, W, D>(a, s, name);
        case 3: return launch_cfg<QT, 3, W, D>(a, s, name);
        default: return launch_cfg<QT, 4, W, D>(a, s, name);
    }
}

}  // namespace

hipError_t launch_gemm_mfma(const GemmArgs &a, hipStream_t s, const char **name) {
    return a.qtype == 4 ? launch_q<4>(a, s, name) : launch_q<8>(a, s, name);
}

}  // namespace qmv
