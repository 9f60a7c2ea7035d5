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
// Work layout.  A workgroup owns 16 RG weight rows and up to 64 activation
// rows (MT tiles of 16).  Its RG x KG wavefronts are (row group rg, K group
// kg): K advances in stages of 4 blocks, group kg taking stages kg, kg + KG,
// kg + 2 KG, ... (so the groups read adjacent spans of each weight row
// together), and wavefront (rg, kg) computes the 16 x 16 MT output tiles of
// its 16 weight rows over its group's stages.  Every weight byte is read
// from memory once per launch, the activation once per workgroup: the RG
// row groups share it, which is what keeps the activation traffic (M K
// bytes per workgroup, from the L2 cache) below the weight traffic.
//
// Data movement.  In the operand layout consecutive lanes read different
// rows, which the vector memory path serves at a fraction of its rate, so
// nothing is loaded in that layout: tiles are loaded with 16 (or 4) bytes
// per lane such that each group of 4 consecutive lanes reads one contiguous
// span of one row, into a ring of D register stages per wavefront (D - 1
// stages stay in flight to cover memory latency), then written to LDS and
// read back in the operand layout.  Each wavefront stages its own weight
// rows (Q4_0 nibbles turned into signed bytes, nibble - 8, on the way) and
// the scales it needs in a private LDS buffer; the activation quants of a K
// group's stage are loaded in equal slices by the group's RG wavefronts into
// a double-buffered LDS buffer shared by the group, with one workgroup
// barrier per stage.  Every wavefront runs the same instructions (no branch
// on the wavefront's role), which keeps the compiler's waits for the
// register ring exact.  The 16-byte pieces of each 128-byte LDS row sit
// under an XOR swizzle of the piece index, so that the operand reads of 32
// lanes fall in distinct banks.  At the end the K groups' partial tiles are
// summed in LDS in a fixed order (the result does not depend on timing) and
// stored with consecutive lanes on consecutive weight rows.
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
// Loads with a per-lane offset that stays fixed across stages; the stage
// is selected by the descriptor (base advanced to the stage, range cut to
// the bytes left), which the scalar unit computes, so advancing the stage
// costs no vector instructions and every access stays range-checked (the
// scalar offset field of a buffer load is not range-checked, so it is not
// used).  The lane offset goes through an empty asm so that the compiler
// keeps one unconditional load (it would otherwise branch around loads
// whose offset is a select, and branches cost the pipelined loop its
// precise waits).
template <int AUX>
__device__ __forceinline__ v4i load16(__amdgpu_buffer_rsrc_t r, int voff) {
    asm volatile("" : "+v"(voff));
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, AUX));
}
template <int AUX>
__device__ __forceinline__ float load4(__amdgpu_buffer_rsrc_t r, int voff) {
    asm volatile("" : "+v"(voff));
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, AUX));
}

// Descriptor for the bytes [off, bytes) of a buffer (none if off >= bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sub_rsrc(const void *base, int bytes, int off) {
    const int o = __builtin_amdgcn_readfirstlane(min(off, bytes));
    return make_rsrc(static_cast<const char *>(base) + o, bytes - o);
}

__device__ __forceinline__ v4i mfma16(v2i a, v2i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x32_i8(__builtin_bit_cast(long, a), __builtin_bit_cast(long, b), c, 0, 0, 0);
}

// Q4_0 operands stay as nibbles 0..15 (one per byte); the -8 of each weight
// is folded into the matrix instruction's accumulator input: the product of
// an operand of all -8 bytes with the activation operand is -8 * (sum of the
// activation's 32 quants of the block), and the nibble product is added to
// it -- exactly sum_k (nibble_k - 8) x_k.
constexpr int kMinus8 = (int)0xF8F8F8F8;

// Position of 16-byte piece q of row r in the row's 128-byte LDS image (an
// involution on the row's 8 pieces).
__device__ __forceinline__ int swz(int q, int r) { return q ^ ((r >> 1) & 7); }

// LDS of a workgroup (bytes):
//   per K group, D shared activation stage buffers (one per stage of the
//   register ring): MT tiles x 16 rows x 128 B
//   per wavefront, a private buffer: its weight stage (16 rows x 128 B of
//   signed bytes), the weight scales (16 x 4 floats) and the activation
//   scales (MT tiles x 16 x 4 floats)
template <int MT, int RG, int KG, int D>
struct Lds {
    static constexpr int XS = MT * 2048;                // one shared activation stage
    static constexpr int PW = 2048 + 256 + MT * 256;    // one private buffer
    static constexpr int P0 = KG * D * XS;              // D shared buffers per K group
    static constexpr int TOTAL = P0 + RG * KG * PW;
    static_assert(RG * KG * MT * 1024 <= TOTAL, "partial tiles fit in the buffers");
};

// One stage in registers: this lane's share of the coalesced loads.
template <int QT, int MT, int RG>
struct Stage {
    static constexpr int NX = 2 * MT / RG;  // 1 KiB activation units per wavefront
    v4i w[QT == 8 ? 2 : 1];
    float dw;
    v4i x[NX];
    float dx[MT];
};

template <int QT, int MT, int RG, int KG, int D>
__global__ void __launch_bounds__(64 * RG * KG)
k_gemm_mfma(float *__restrict__ Y, const int8_t *__restrict__ wq, const float *__restrict__ wd, int32_t rows,
            int32_t K, const int8_t *__restrict__ xq, const float *__restrict__ xd, int32_t M, int32_t r0,
            int32_t r1) {
    typedef Lds<MT, RG, KG, D> L;
    typedef Stage<QT, MT, RG> St;
    static_assert((2 * MT) % RG == 0, "activation units split evenly over the row groups");
    constexpr int QB = (QT == 8) ? 32 : 16;
    constexpr int NX = St::NX;
    extern __shared__ __align__(16) unsigned char smem[];

    const int nb = K >> 5;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg = wid % RG, kg = wid / RG;
    const int n0 = r0 + (blockIdx.x * RG + rg) * 16;  // this wavefront's weight rows n0 .. n0 + 15
    unsigned char *const xsh = smem + kg * D * L::XS;
    unsigned char *const pbuf = smem + L::P0 + wid * L::PW;
    constexpr int PDW = 2048, PDX = 2048 + 256;

    // descriptors cover only valid data: loads beyond them return zeros
    // (a row group wholly past r1 has an empty weight range)
    // (readfirstlane: the clamp would otherwise be computed on the vector unit,
    // and a descriptor in vector registers costs every load a waterfall loop)
    const int wrows = __builtin_amdgcn_readfirstlane(max(0, min(16, r1 - n0)));
    const int wrow0 = __builtin_amdgcn_readfirstlane(min(n0, r1));
    const int8_t *const wq0 = wq + (size_t)wrow0 * nb * QB;
    const float *const wd0 = wd + (size_t)wrow0 * nb;
    const int wq_bytes = wrows * nb * QB, wd_bytes = wrows * nb * 4, xq_bytes = M * K, xd_bytes = M * nb * 4;

    // Load roles of this lane (byte offsets at block 0; the stage adds a
    // wave-uniform offset).  A stage past K reads nothing; a partial last
    // stage reads the next row's bytes for the blocks past K, which
    // contribute exactly 0: their weight scales (loaded per lane) are 0.
    //   weights, Q4_0: row lane/4, block lane%4 (16 packed bytes)
    //   weights, Q8_0 and activations: row 8t + lane/8 of a 16-row tile,
    //     16-byte piece swz(lane%8) of the row's 128 stage bytes
    //   scales: row lane/4, block lane%4
    int wq_off[QT == 8 ? 2 : 1];
    if constexpr (QT == 8) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int r = 8 * t + (lane >> 3);
            wq_off[t] = r * nb * 32 + 16 * swz(lane & 7, r);
        }
    } else {
        wq_off[0] = (lane >> 2) * nb * 16 + 16 * (lane & 3);
    }
    const int wd_off = ((lane >> 2) * nb + (lane & 3)) * 4;
    // activation units of this wavefront: un = rg + RG k, tile un / 2, rows 8 (un % 2) ..
    int x_off[NX];
#pragma unroll
    for (int k = 0; k < NX; ++k) {
        const int un = rg + RG * k;
        const int r = 8 * (un & 1) + (lane >> 3), m = (un >> 1) * 16 + r;
        x_off[k] = m < M ? m * K + 16 * swz(lane & 7, r) : kOOB;
    }
    int xd_off[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int m = t * 16 + (lane >> 2);
        xd_off[t] = m < M ? (m * nb + (lane & 3)) * 4 : kOOB;
    }

    // stages of this K group: kg, kg + KG, ...; every group runs nit
    // iterations (the barrier count must agree)
    const int nu = (nb + KU - 1) / KU;
    const int nit = (nu + KG - 1) / KG;

    auto load = [&](St &s, int it) __attribute__((always_inline)) {
        const int kb = min(KU * (it * KG + kg), nb);  // a stage past K gets empty descriptors
        const bool live = kb < nb;
        const __amdgpu_buffer_rsrc_t rwq = sub_rsrc(wq0, wq_bytes, live ? kb * QB : wq_bytes);
        const __amdgpu_buffer_rsrc_t rwd = sub_rsrc(wd0, wd_bytes, live ? kb * 4 : wd_bytes);
        const __amdgpu_buffer_rsrc_t rxq = sub_rsrc(xq, xq_bytes, live ? kb * 32 : xq_bytes);
        const __amdgpu_buffer_rsrc_t rxd = sub_rsrc(xd, xd_bytes, live ? kb * 4 : xd_bytes);
#pragma unroll
        for (int t = 0; t < (QT == 8 ? 2 : 1); ++t) s.w[t] = load16<kNT>(rwq, wq_off[t]);
        s.dw = load4<kNT>(rwd, kb + (lane & 3) < nb ? wd_off : kOOB);
#pragma unroll
        for (int k = 0; k < NX; ++k) s.x[k] = load16<0>(rxq, x_off[k]);
#pragma unroll
        for (int t = 0; t < MT; ++t) s.dx[t] = load4<0>(rxd, xd_off[t]);
    };
    auto stash = [&](const St &s, int d) __attribute__((always_inline)) {
        // weights -> private buffer in the swizzled row image: Q8_0 signed
        // bytes; Q4_0 nibbles 0..15 one per byte, elements 0..15 from the low
        // nibbles and 16..31 from the high nibbles
        if constexpr (QT == 8) {
#pragma unroll
            for (int t = 0; t < 2; ++t) *reinterpret_cast<v4i *>(pbuf + 1024 * t + 16 * lane) = s.w[t];
        } else {
            const int r = lane >> 2, u = lane & 3;
            v4i lo, hi;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const unsigned w = (unsigned)s.w[0][k];
                lo[k] = (int)(w & 0x0F0F0F0Fu);
                hi[k] = (int)((w >> 4) & 0x0F0F0F0Fu);
            }
            *reinterpret_cast<v4i *>(pbuf + 128 * r + 16 * swz(2 * u, r)) = lo;
            *reinterpret_cast<v4i *>(pbuf + 128 * r + 16 * swz(2 * u + 1, r)) = hi;
        }
        *reinterpret_cast<float *>(pbuf + PDW + 4 * lane) = s.dw;
#pragma unroll
        for (int t = 0; t < MT; ++t) *reinterpret_cast<float *>(pbuf + PDX + 256 * t + 4 * lane) = s.dx[t];
        // this wavefront's activation units -> the group's shared buffer d
        unsigned char *xb = xsh + d * L::XS;
#pragma unroll
        for (int k = 0; k < NX; ++k) *reinterpret_cast<v4i *>(xb + 1024 * (rg + RG * k) + 16 * lane) = s.x[k];
    };

    // operand read offsets of this lane (same layout for both operands)
    const int i = lane & 15, g = lane >> 4;
    int op_off[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) op_off[u] = 128 * i + 16 * swz(2 * u + (g >> 1), i) + 8 * (g & 1);

    float acc[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][v] = 0.0f;
    // All LDS operand reads of the stage first, then its 4 MT matrix
    // instructions, then their scale epilogues: independent work between
    // each read and its use, and between each MFMA and its result's use.
    auto compute = [&](int d) __attribute__((always_inline)) {
        const unsigned char *xb = xsh + d * L::XS;
        v4f dw4[4], dx4[MT];
        v2i a[KU], b[KU][MT];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            a[u] = *reinterpret_cast<const v2i *>(pbuf + op_off[u]);
#pragma unroll
            for (int t = 0; t < MT; ++t) b[u][t] = *reinterpret_cast<const v2i *>(xb + 2048 * t + op_off[u]);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) dw4[v] = *reinterpret_cast<const v4f *>(pbuf + PDW + 16 * (4 * g + v));
#pragma unroll
        for (int t = 0; t < MT; ++t) dx4[t] = *reinterpret_cast<const v4f *>(pbuf + PDX + 256 * t + 16 * i);
        v4i c[KU][MT];
        const v2i m8 = {kMinus8, kMinus8};
        const v4i z = {};
#pragma unroll
        for (int u = 0; u < KU; ++u)
#pragma unroll
            for (int t = 0; t < MT; ++t)
                c[u][t] = (QT == 4) ? mfma16(a[u], b[u][t], mfma16(m8, b[u][t], z)) : mfma16(a[u], b[u][t], z);
#pragma unroll
        for (int u = 0; u < KU; ++u)
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[t][v] = fmaf((float)c[u][t][v], dx4[t][u] * dw4[v][u], acc[t][v]);
    };

    // LDS writes of the stage done in every wavefront, then all may read
    auto barrier = []() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    // ring of D register stages; the loop is unrolled by D so that every
    // stage lives in fixed registers, and runs whole groups of D stages
    St ring[D];
#pragma unroll
    for (int d = 0; d < D - 1; ++d) load(ring[d], d);
    for (int it0 = 0; it0 < nit; it0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int it = it0 + d;
            load(ring[(d + D - 1) % D], it + D - 1);
            stash(ring[d], d);  // buffer d was last read D stages ago, before a barrier since
            barrier();          // every K group's activation stage is in LDS
            compute(d);
            __builtin_amdgcn_sched_barrier(0);  // keep the stages apart: register pressure
        }
    }

    // partial tiles of the K groups -> LDS, then a fixed-order sum per output
    barrier();
    float *part = reinterpret_cast<float *>(smem);  // [wavefront][MT][4][64]
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) part[((wid * MT + t) * 4 + v) * 64 + lane] = acc[t][v];
    barrier();
    for (int e = threadIdx.x; e < RG * MT * 256; e += 64 * RG * KG) {
        const int nl = e & 15, ml = (e >> 4) % (MT * 16), r = (e >> 4) / (MT * 16);  // row group r
        const int t = ml >> 4, l = (ml & 15) + 16 * (nl >> 2), v = nl & 3;
        float s = 0.0f;
        for (int k = 0; k < KG; ++k) s += part[(((k * RG + r) * MT + t) * 4 + v) * 64 + l];
        const int n = r0 + (blockIdx.x * RG + r) * 16 + nl;
        if (ml < M && n < r1) Y[(size_t)ml * rows + n] = s;
    }
}

template <int QT, int MT, int RG, int KG, int D>
hipError_t launch_cfg(const GemmArgs &a, hipStream_t s, const char **name) {
    static char kname[64];
    typedef Lds<MT, RG, KG, D> L;
    static_assert(L::TOTAL <= 160 * 1024, "LDS budget");
    static_assert(RG * KG <= 16, "at most 1024 threads");
    auto kern = k_gemm_mfma<QT, MT, RG, KG, D>;
    if (L::TOTAL > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, L::TOTAL);
        if (e != hipSuccess) return e;
    }
    const int grid = (a.r1 - a.r0 + 16 * RG - 1) / (16 * RG);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * RG * KG), L::TOTAL, s, a.Y, a.wq, a.wd, a.rows, a.K, a.xq, a.xd,
                       a.M, a.r0, a.r1);
    if (kname[0] == 0) snprintf(kname, sizeof kname, "gemm_mfma_q%d_mt%d_rg%d_kg%d_d%d", QT, MT, RG, KG, D);
    *name = kname;
    return hipGetLastError();
}

// Register stages per wavefront (D - 1 stay in flight), by activation tiles.
// Measured: deeper rings cost more in occupancy than they gain in flight.
#ifndef QMV_GEMM_D1
#define QMV_GEMM_D1 2
#endif
#ifndef QMV_GEMM_D2
#define QMV_GEMM_D2 2
#endif
#ifndef QMV_GEMM_D4
#define QMV_GEMM_D4 2
#endif
#ifndef QMV_GEMM_WAVES
#define QMV_GEMM_WAVES 8  // wavefronts per workgroup (RG x KG)
#endif
#ifndef QMV_GEMM_MIN_GROUPS
#define QMV_GEMM_MIN_GROUPS 160  // fewest workgroups a larger row-group count may leave
#endif

// Row groups per workgroup: the most (up to 4) that still leave enough
// workgroups to fill the chip.
template <int QT, int MT>
hipError_t launch_mt(const GemmArgs &a, hipStream_t s, const char **name) {
    constexpr int W = QMV_GEMM_WAVES;
    constexpr int D = MT == 1 ? QMV_GEMM_D1 : MT == 2 ? QMV_GEMM_D2 : QMV_GEMM_D4;
    // one row group loads the whole activation stage per wavefront: a
    // shallower ring keeps that case within the register file
    constexpr int D1 = (MT == 4) ? 2 : (MT == 2 && D > 4) ? 4 : D;
    const int tiles = (a.r1 - a.r0 + 15) / 16;
#ifdef QMV_GEMM_FORCE_RG
    if (MT == 1 || QMV_GEMM_FORCE_RG <= 2 * MT)
        return launch_cfg<QT, MT, QMV_GEMM_FORCE_RG, QMV_GEMM_FORCE_KG, D>(a, s, name);
#endif
    if constexpr ((2 * MT) % 4 == 0)
        if (tiles / 4 >= QMV_GEMM_MIN_GROUPS) return launch_cfg<QT, MT, 4, W / 4, D>(a, s, name);
    if (tiles / 2 >= QMV_GEMM_MIN_GROUPS) return launch_cfg<QT, MT, 2, W / 2, D>(a, s, name);
    return launch_cfg<QT, MT, 1, W, D1>(a, s, name);
}

template <int QT>
hipError_t launch_q(const GemmArgs &a, hipStream_t s, const char **name) {
    switch ((a.M + 15) / 16) {
        case 1: return launch_mt<QT, 1>(a, s, name);
        case 2: return launch_mt<QT, 2>(a, s, name);
        default: return launch_mt<QT, 4>(a, s, name);
    }
}

}  // namespace

hipError_t launch_gemm_mfma(const GemmArgs &a, hipStream_t s, const char **name) {
    return a.qtype == 4 ? launch_q<4>(a, s, name) : launch_q<8>(a, s, name);
}

}  // namespace qmv
