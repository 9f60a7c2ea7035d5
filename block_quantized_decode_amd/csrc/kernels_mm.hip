// kernels_mm.hip -- the product for 9 .. 64 activation rows on the gfx950
// int8 matrix cores, one workgroup per compute unit.
//
// What is computed (Legacy-ISA ML Inference Runtime -- Design Spec, section
// 4, the per-block integer dot and its scaled accumulation, applied to every
// activation row):
//   Y[m, r] = sum over blocks b of sumi(m, r, b) * dw(r, b) * dx(m, b),
//   sumi(m, r, b) = exact int32 dot of the 32 quants of weight row r and
//   activation row m in block b.
//
// v_mfma_i32_16x16x32_i8 contracts exactly one 32-element block, so its
// int32 result is sumi for 16 weight rows x 16 activation rows; the scales
// follow in fp32 (acc += (float)sumi * (dw * dx)).  A (lane l: weight row
// l % 16) and B (lane l: activation row l % 16) both supply elements
// 8 g .. 8 g + 7 of the block, g = l / 16; result register v of lane l is
// weight row 4 g + v, activation row l % 16.
//
// Work layout.  One workgroup per compute unit owns RT tiles of 16 weight
// rows and all activation rows (MT tiles of 16); its wavefronts split K:
// wavefront w owns stages (4 blocks each) w, w + 8, w + 16, ..., so the
// wavefronts of a workgroup read adjacent spans of each row together.  Each wavefront
// stages its own slice -- weights (Q4_0 nibbles expanded to bytes 0..15),
// activation quants and both scales -- in a private LDS region, so the
// K loop has no workgroup barrier; the activation is read from memory once
// per workgroup, the weights once.  At the end the wavefronts' partial tiles
// are added in LDS in wavefront order (the result does not depend on
// timing).
//
// Loads are coalesced (each group of 4 or 8 lanes reads a contiguous span of
// one row) into a ring of D register stages, written to LDS in a
// swizzled row image (16-byte piece q of row r at q ^ ((r / 2) % 8), so the
// operand reads of 32 lanes fall in distinct banks) and read back in the
// operand layout.  Every variable part of an address is in the
// range-checked per-lane offset of a raw buffer load whose descriptor
// covers only valid data: weight rows past r1 and activation rows past M
// read zeros; blocks past K in a partial last stage read the next row's
// bytes, and their scales are set to 0, so they contribute exactly 0.
//
// Q4_0: the nibbles enter the instruction as bytes 0..15 and the -8 of each
// weight is folded into the accumulator input: the product of an operand of
// all -8 bytes with the activation operand is -8 * (sum of the activation's
// 32 quants), computed once per activation tile and block and shared by the
// RT weight tiles.
#include <stdio.h>

#include "count.h"
#include "device_common.h"
#include "launch.h"

namespace qmv {
namespace {

constexpr int kBufFlags = 0x00020000;  // buffer descriptor word 3: raw 32-bit data
constexpr int kOOB = 0x40000000;       // an offset beyond every descriptor range used here
#ifndef QMV_MM_CTAIL  // 1: the many-stage form's last stages specialised on their count; 0: tested per stage
#define QMV_MM_CTAIL 1
#endif
#ifndef QMV_MM_PARTPAD  // 1: the partial tiles' LDS layout padded against bank conflicts (see k_mm)
#define QMV_MM_PARTPAD 1
#endif
constexpr int kNT = 2;                 // non-temporal: weights are read once
constexpr int KU = 4;                  // blocks per stage
constexpr int kMinus8 = (int)0xF8F8F8F8;

#ifndef QMV_MM_D1
#define QMV_MM_D1 2
#endif
#ifndef QMV_MM_D2
#define QMV_MM_D2 2
#endif
#ifndef QMV_MM_D4
#define QMV_MM_D4 2
#endif
#ifndef QMV_MM_W1  // wavefronts per workgroup: packed weights, one activation tile
#define QMV_MM_W1 8
#endif
#ifndef QMV_MM_RTMAX  // weight-row tiles per workgroup, at most
#define QMV_MM_RTMAX 4
#endif


typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, kBufFlags);
}
template <int AUX>
__device__ __forceinline__ v4i ld16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}
__device__ __forceinline__ v4i mfma16(v2i a, v2i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x32_i8(__builtin_bit_cast(long, a), __builtin_bit_cast(long, b), c, 0, 0, 0);
}
// byte offset of 16-byte piece q of row r in a 128-byte-per-row LDS image
__device__ __forceinline__ int img(int r, int q) { return 128 * r + 16 * (q ^ ((r >> 1) & 7)); }

// The 16 x 16 products dw(4 g + v) * dx(l % 16) for lane l = 16 g + ..., in
// the accumulator layout of v_mfma_i32_16x16x32_i8 (register v: weight row
// 4 g + v, activation row l % 16), from one v_mfma_f32_4x4x1_16b_f32: its
// 16 blocks of 4 x 4 outer products put A of lane 4 j + v times B of lane
// 4 j + i into register v of lane 4 j + i.  So lane l supplies
// dw(4 (l / 16) + l % 4) as A and dx(l % 16) as B.  One product per output
// and a zero accumulator: each value is the rounded product dw * dx.
__device__ __forceinline__ v4f scale_tile(float dw_lane, float dx_lane) {
    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_f32_4x4x1f32(dw_lane, dx_lane, z, 0, 0, 0);
}

// One stage in registers (this lane's share of the coalesced loads).
template <int QT, int MT, int RT>
struct Stage {
    static constexpr int NW = (QT == 8) ? 2 * RT : RT;  // 16-byte weight loads
    v4i w[NW];
    v4i x[2 * MT];
    v4f dw, dx;
};

// Per-wavefront LDS region (bytes): activation image, weight image (none for
// packed weights), weight scales [4][64] and activation scales [4][64].
template <int MT, int RT, bool PK>
struct Region {
    static constexpr int X = 0, W = X + MT * 16 * 128, DW = W + (PK ? 0 : RT * 16 * 128), DX = DW + 4 * 64 * 4;
    static constexpr int BYTES = DX + 4 * 64 * 4;
};

// PK: the weights come in the pack-once layout of kernels_pack.hip (units of
// 16 rows x 4 blocks, quants in the A operand's lane order, scales [row][block]);
// the quants go from the load straight into the operand, never through LDS.
// The sums are the same operations in the same order as for the row-major
// layout, so the two give the same bits.
template <int QT, int MT, int RT, int WPB, int D, bool PK, bool TAIL>
__global__ void __launch_bounds__(64 * WPB)
k_mm(float *__restrict__ Y, const int8_t *__restrict__ wq, const float *__restrict__ wd, int32_t rows, int32_t K,
     const int8_t *__restrict__ xq, const float *__restrict__ xd, int32_t M, int32_t r0, int32_t r1) {
    typedef Region<MT, RT, PK> Rg;
    typedef Stage<QT, MT, RT> St;
    constexpr int QB = (QT == 8) ? 32 : 16;
    static_assert(RT * 16 <= 64 && MT * 16 <= 64, "scale loads: one row per lane");
    extern __shared__ __align__(16) unsigned char smem[];

    const int nb = K >> 5;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    unsigned char *const reg = smem + wid * Rg::BYTES;
    const int g0 = r0 + blockIdx.x * (16 * RT);  // weight rows g0 .. g1 - 1
    const int g1 = min(r1, g0 + 16 * RT);
    const int nrow = g1 - g0;

    // stages of this wavefront: wid, wid + WPB, wid + 2 WPB, ... (the
    // wavefronts of the workgroup read adjacent spans of each row together)
    const int ns = (nb + KU - 1) / KU;
    const int nst = wid < ns ? (ns - wid + WPB - 1) / WPB : 0;
    auto stage = [&](int j) { return wid + WPB * j; };

    // packed: unit (tile T, quad s) at T nq + s, UQ bytes of quants and 256 of
    // scales; g0 is a multiple of 16 there
    const int nq = (nb + KU - 1) / KU;
    constexpr int UQ = 64 * KU * QB / 4;
    const int ntile = (nrow + 15) >> 4;
    const __amdgpu_buffer_rsrc_t rw = PK ? make_rsrc(wq + (size_t)(g0 >> 4) * nq * UQ, ntile * nq * UQ)
                                         : make_rsrc(wq + (size_t)g0 * nb * QB, nrow * nb * QB);
    const __amdgpu_buffer_rsrc_t rwd = PK ? make_rsrc(wd + (size_t)(g0 >> 4) * nq * 64, ntile * nq * 256)
                                          : make_rsrc(wd + (size_t)g0 * nb, nrow * nb * 4);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(xq, M * K);
    const __amdgpu_buffer_rsrc_t rxd = make_rsrc(xd, M * nb * 4);

    // per-lane offsets at stage 0 (a stage adds 4 blocks)
    //   weights Q4_0: row 16 i + l / 4, block l % 4 (16 bytes)
    //   weights Q8_0: row 8 i + l / 8, 16-byte piece l % 8 of the stage's 128 bytes
    //   activation: row 8 i + l / 8, piece l % 8
    //   scales: row l, the stage's 4 blocks (16 bytes)
    //   packed weights: tile i (Q4_0) or i / 2 (Q8_0, half i % 2), this lane's 16 bytes
    //   packed scales: row lane % 16 of tile lane / 16, the unit's 4 blocks
    int ow[St::NW];
#pragma unroll
    for (int i = 0; i < St::NW; ++i) {
        if constexpr (PK)
            ow[i] = (QT == 8) ? ((i >> 1) * nq * UQ + 1024 * (i & 1) + 16 * lane) : (i * nq * UQ + 16 * lane);
        else
            ow[i] = (QT == 8) ? ((8 * i + (lane >> 3)) * nb * 32 + 16 * (lane & 7))
                              : ((16 * i + (lane >> 2)) * nb * 16 + 16 * (lane & 3));
    }
    int ox[2 * MT];
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) ox[i] = (8 * i + (lane >> 3)) * K + 16 * (lane & 7);
    const int odw = lane >= 16 * RT ? kOOB : PK ? (lane >> 4) * nq * 256 + 16 * (lane & 15) : lane * nb * 4;
    const int sw = PK ? UQ : KU * QB, sd = PK ? 256 : KU * 4;  // weight and scale bytes per stage
    const int odx = lane < 16 * MT ? lane * nb * 4 : kOOB;

    auto load = [&](St &st, int j) __attribute__((always_inline)) {
        const bool live = j < nst;  // past this wavefront's stages: empty loads
        const int s = stage(j);
#pragma unroll
        for (int i = 0; i < St::NW; ++i) st.w[i] = ld16<kNT>(rw, live ? ow[i] + s * sw : kOOB);
#pragma unroll
        for (int i = 0; i < 2 * MT; ++i) st.x[i] = ld16<0>(rx, live ? ox[i] + s * KU * 32 : kOOB);
        st.dw = __builtin_bit_cast(v4f, ld16<0>(rwd, live ? odw + s * sd : kOOB));
        st.dx = __builtin_bit_cast(v4f, ld16<0>(rxd, live ? odx + s * KU * 4 : kOOB));
    };
    auto stash = [&](St &st, int j) __attribute__((always_inline)) {
        const int b0 = stage(j) * KU;  // scales of blocks past K -> 0
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (b0 + e >= nb) {
                st.dw[e] = 0.0f;
                st.dx[e] = 0.0f;
            }
        }
        if constexpr (PK) {
            // the quants stay in registers
        } else if constexpr (QT == 8) {
#pragma unroll
            for (int i = 0; i < St::NW; ++i)
                *reinterpret_cast<v4i *>(reg + Rg::W + img(8 * i + (lane >> 3), lane & 7)) = st.w[i];
        } else {
            // bytes j of the 16 hold elements j (low nibble) and j + 16 (high)
            const int u = lane & 3;
#pragma unroll
            for (int i = 0; i < St::NW; ++i) {
                const int r = 16 * i + (lane >> 2);
                v4i lo, hi;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    lo[k] = (int)((unsigned)st.w[i][k] & 0x0F0F0F0Fu);
                    hi[k] = (int)(((unsigned)st.w[i][k] >> 4) & 0x0F0F0F0Fu);
                }
                *reinterpret_cast<v4i *>(reg + Rg::W + img(r, 2 * u)) = lo;
                *reinterpret_cast<v4i *>(reg + Rg::W + img(r, 2 * u + 1)) = hi;
            }
        }
#pragma unroll
        for (int i = 0; i < 2 * MT; ++i)
            *reinterpret_cast<v4i *>(reg + Rg::X + img(8 * i + (lane >> 3), lane & 7)) = st.x[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            reinterpret_cast<float *>(reg + Rg::DW)[64 * e + lane] = st.dw[e];
            reinterpret_cast<float *>(reg + Rg::DX)[64 * e + lane] = st.dx[e];
        }
    };

    const int i16 = lane & 15, g = lane >> 4;
    // one activation tile: the 16 x 16 scale products dw * dx of a block
    // come from the matrix core (measured 4% faster at M = 16 on the
    // Llama-7B FFN matrices); four tiles keep the VALU multiply (no gain
    // there, and packed Q4_0 W_up at M = 64 was 3% slower)
    constexpr bool SMF = MT == 1;
    float acc[RT][MT][4];
#pragma unroll
    for (int a = 0; a < RT; ++a)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[a][t][v] = 0.0f;

    auto compute = [&](const St &st) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int q = 2 * u + (g >> 1), h = 8 * (g & 1);  // piece and half of elements 8 g .. 8 g + 7
            v2i b[MT];
            float dxv[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                b[t] = *reinterpret_cast<const v2i *>(reg + Rg::X + img(16 * t + i16, q) + h);
                dxv[t] = reinterpret_cast<const float *>(reg + Rg::DX)[64 * u + 16 * t + i16];
            }
            v4i c0[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const v4i z = {};
                const v2i m8 = {kMinus8, kMinus8};
                c0[t] = (QT == 4) ? mfma16(m8, b[t], z) : z;
            }
#pragma unroll
            for (int a = 0; a < RT; ++a) {
                v2i aw;
                if constexpr (PK && QT == 4) {  // nibbles of elements 8 g + j and 8 g + 4 + j in byte j
                    const unsigned w = (unsigned)st.w[a][u];
                    aw = (v2i){(int)(w & 0x0F0F0F0Fu), (int)((w >> 4) & 0x0F0F0F0Fu)};
                } else if constexpr (PK) {
                    const v4i &w = st.w[2 * a + (u >> 1)];
                    aw = (v2i){w[2 * (u & 1)], w[2 * (u & 1) + 1]};
                } else {
                    aw = *reinterpret_cast<const v2i *>(reg + Rg::W + img(16 * a + i16, q) + h);
                }
                // SMF: lane l holds the scale of weight row 4 g + l % 4 (the
                // f32 instruction's A operand); otherwise the 4 rows 4 g + v
                const float *dwp = reinterpret_cast<const float *>(reg + Rg::DW) + 64 * u + 16 * a + 4 * g;
                const float dwl = SMF ? dwp[lane & 3] : 0.0f;
                const v4f dw4 = SMF ? v4f{} : *reinterpret_cast<const v4f *>(dwp);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const v4i c = mfma16(aw, b[t], c0[t]);
                    if constexpr (SMF) {
                        const v4f sc = scale_tile(dwl, dxv[t]);
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[a][t][v] = fmaf((float)c[v], sc[v], acc[a][t][v]);
                    } else {
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[a][t][v] = fmaf((float)c[v], dw4[v] * dxv[t], acc[a][t][v]);
                    }
                }
            }
        }
    };

    // ring of D register stages, unrolled by D so that each stage lives in
    // fixed registers.  (This wavefront's reads of the previous stage are
    // done before its writes of this one: LDS operations of a wavefront
    // complete in order.)
    St ring[D];
#pragma unroll
    for (int d = 0; d < D - 1; ++d) load(ring[d], d);
    auto step = [&](int d, int j) __attribute__((always_inline)) {
        stash(ring[d], j);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        compute(ring[d]);
    };
    if constexpr (TAIL) {
        // many stages (the launcher's choice): turns whose loads all fall
        // among this wavefront's stages run unguarded (exact wait counts),
        // and the last one or two load and compute only stages that exist
        // (measured: Q4_0 W_down 4096 x 11008 at M = 16, 11 stages,
        // 14.3 -> 12.9 us), as code specialised on their count, which keeps
        // those waits exact too (12.9 -> 12.7 us; packed and M = 64 0 - 1.5%)
        int it = 0;
        for (; (it + 2) * D - 2 < nst; ++it) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int j = it * D + d;
                load(ring[(d + D - 1) % D], j + D - 1);
                step(d, j);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#if QMV_MM_CTAIL
        with_count<1, 2 * D - 2>(nst - it * D, [&](auto rc) __attribute__((always_inline)) {
            constexpr int R = decltype(rc)::value;
#pragma unroll
            for (int q = 0; q < R; ++q) {
                if (q + D - 1 < R) load(ring[(q + D - 1) % D], it * D + q + D - 1);
                step(q % D, it * D + q);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
#else
        for (; it * D < nst; ++it) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int j = it * D + d;
                if (j < nst) {  // (wave-uniform)
                    if (j + D - 1 < nst) load(ring[(d + D - 1) % D], j + D - 1);
                    step(d, j);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#endif
    } else {
        // few stages: whole turns (stages past the last load nothing and
        // compute zeros); a guarded tail would be half of the loop here and
        // measured slower (Q8_0 W_up 11008 x 4096, 4 stages: 28 -> 31 us at
        // M = 64), and so was one kernel holding both loops
        const int nit = (nst + D - 1) / D;
        for (int it = 0; it < nit; ++it) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int j = it * D + d;
                load(ring[(d + D - 1) % D], j + D - 1);
                step(d, j);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // partial tiles of the wavefronts -> LDS (over the staging regions),
    // then a fixed-order sum per output
    __syncthreads();
    // [wavefront][RT][MT] blocks of BS floats, each [4][PS]: the rows of 64
    // lanes padded to 65 floats and each block to 4 * 65 + 1, so the sum
    // below (consecutive threads on consecutive accumulator registers v, then
    // on the next weight tile) reads distinct banks: measured bank conflicts
    // of packed W_up, M = 64, 55% -> 23% -> 9% of LDS-active cycles
    constexpr int PS = QMV_MM_PARTPAD ? 65 : 64, BS = QMV_MM_PARTPAD ? 4 * 65 + 1 : 4 * 64;
    float *part = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int a = 0; a < RT; ++a)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) part[((wid * RT + a) * MT + t) * BS + v * PS + lane] = acc[a][t][v];
    __syncthreads();
    for (int e = threadIdx.x; e < 16 * RT * 16 * MT; e += 64 * WPB) {
        const int nl = e % (16 * RT), m = e / (16 * RT);  // weight row within the range, activation row
        const int a = nl >> 4, gv = nl & 15, t = m >> 4;
        const int l = 16 * (gv >> 2) + (m & 15), v = gv & 3;
        float s = 0.0f;
        for (int w = 0; w < WPB; ++w) s += part[((w * RT + a) * MT + t) * BS + v * PS + l];
        if (m < M && nl < nrow) Y[(size_t)m * rows + g0 + nl] = s;
    }
}

template <int QT, int MT, int RT, bool PK, bool TAIL>
hipError_t launch_cfg_t(const GemmArgs &a, hipStream_t s, const char **name) {
    // register stages in the ring (D - 1 in flight) by activation tiles
    // (measured: deeper rings for one tile lose more to registers than they
    // gain in flight; four tiles leave no room for a third stage)
    constexpr int WPB = (PK && MT == 1) ? QMV_MM_W1 : 8, D = MT == 1 ? QMV_MM_D1 : MT == 2 ? QMV_MM_D2 : QMV_MM_D4;
    typedef Region<MT, RT, PK> Rg;
    constexpr int lds_stage = WPB * Rg::BYTES, lds_part = WPB * RT * MT * (QMV_MM_PARTPAD ? 4 * 65 + 1 : 4 * 64) * 4;
    constexpr int lds = lds_stage > lds_part ? lds_stage : lds_part;
    static_assert(lds <= 160 * 1024, "LDS budget");
    static const std::string kname =
        variant_name("mm%s_q%d_mt%d_rt%d_w%d_d%d%s", PK ? "p" : "", QT, MT, RT, WPB, D, TAIL ? "_t" : "");
    auto kern = k_mm<QT, MT, RT, WPB, D, PK, TAIL>;
    hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), lds);
    if (e != hipSuccess) return e;
    const int grid = (a.r1 - a.r0 + 16 * RT - 1) / (16 * RT);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WPB), lds, s, a.Y, PK ? static_cast<const int8_t *>(a.pq) : a.wq,
                       PK ? a.pd : a.wd, a.rows, a.K, a.xq, a.xd, a.M, a.r0, a.r1);
    *name = kname.c_str();
    return hipGetLastError();
}

// The stage loop with a guarded tail for wavefronts of at least 3 ring turns
// of stages (every wavefront has per or per - 1 stages), whole turns below.
template <int QT, int MT, int RT, bool PK>
hipError_t launch_cfg(const GemmArgs &a, hipStream_t s, const char **name) {
    constexpr int D = MT == 1 ? QMV_MM_D1 : MT == 2 ? QMV_MM_D2 : QMV_MM_D4;
    constexpr int WPB = (PK && MT == 1) ? QMV_MM_W1 : 8;
    const int ns = (a.K / 32 + KU - 1) / KU;
    if (ns / WPB >= 3 * D) return launch_cfg_t<QT, MT, RT, PK, true>(a, s, name);
    return launch_cfg_t<QT, MT, RT, PK, false>(a, s, name);
}

template <int QT, int MT, bool PK>
hipError_t launch_mt(const GemmArgs &a, int num_cu, hipStream_t s, const char **name) {
    // weight-row tiles per workgroup: enough that one workgroup per compute
    // unit covers the range, at most 4
    const int tiles = (a.r1 - a.r0 + 15) / 16;
    const int rt = min((tiles + num_cu - 1) / num_cu, QMV_MM_RTMAX);
    if (rt <= 1) return launch_cfg<QT, MT, 1, PK>(a, s, name);
    if (rt <= 2) return launch_cfg<QT, MT, 2, PK>(a, s, name);
    if (rt <= 3) return launch_cfg<QT, MT, 3, PK>(a, s, name);
    return launch_cfg<QT, MT, 4, PK>(a, s, name);
}

template <int QT, bool PK>
hipError_t launch_q(const GemmArgs &a, int num_cu, hipStream_t s, const char **name) {
    switch ((a.M + 15) / 16) {
        case 1: return launch_mt<QT, 1, PK>(a, num_cu, s, name);
        case 2: return launch_mt<QT, 2, PK>(a, num_cu, s, name);
        default: return launch_mt<QT, 4, PK>(a, num_cu, s, name);
    }
}

}  // namespace

hipError_t launch_mm(const GemmArgs &a, int num_cu, hipStream_t s, const char **name) {
    if (a.M < 1 || a.M > kGemmMaxRows) return hipErrorNotSupported;
    if (a.pq != nullptr) {
        if (a.r0 % 16 != 0) return hipErrorInvalidValue;  // packed tiles start every 16 rows
        return a.qtype == 4 ? launch_q<4, true>(a, num_cu, s, name) : launch_q<8, true>(a, num_cu, s, name);
    }
    return a.qtype == 4 ? launch_q<4, false>(a, num_cu, s, name) : launch_q<8, false>(a, num_cu, s, name);
}

}  // namespace qmv
