// kernels_zp.hip -- the decode matvec on 128-element blocks with a zero
// point (gfx950).
//
// What is computed ("ONNX Runtime" page, section 3 "Match real exports --
// BlkLen=128 CompInt8" and section 4 "SQ8Bit"): weights are unsigned codes
// B (one byte, or one nibble: element 2i in the low nibble of byte i,
// 2i + 1 in the high nibble) with an fp32 scale dw and a zero point zp per
// 128-element block (a null zp array means 2^(bits-1)); the float
// activation is quantized to int8 per 128-element block with the Q8_0 rule
// of the Legacy-ISA ML Inference Runtime -- Design Spec (section 4 "Q8
// quantization", section 5 rounding), and
//   y[r] = sum over blocks b of sumi(r, b) * dw(r, b) * dx(b),
//   sumi = sum over the block of (B - zp) * q, exact in int32.
// gfx950 has no signed x unsigned byte dot, so sumi is evaluated through the
// page's identity: with B' = B - 128 (the code with its top bit flipped, a
// signed byte), sumi = sum B' q - (zp - 128) * sum q; 4-bit codes are
// already non-negative bytes, so sumi = sum B q - zp * sum q.  sum q is
// computed once per block when the activation is quantized.
//
// Work layout.  Workgroups of 8 wavefronts, 2 or 4 per compute unit.
//   Phase A: the workgroup quantizes the whole activation into LDS: each
//   half-wavefront one 128-element block, 4 elements per lane, maximum and
//   sum reduced by DPP within rows of 16 lanes and lane reads across rows;
//   the block scales and the block sums of the quants go to LDS as well.
//   For 4-bit weights the quants of each 8-element group are stored as
//   (x0, x2, x4, x6, x1, x3, x5, x7), so that the masked low and high
//   nibbles of a weight dword meet their activation bytes in one v_dot4
//   each.  The first weight loads are issued before this phase.
//   Phase B: groups of L lanes (L = 16, 32 or 64) stream whole weight rows:
//   lane c of a group reads 16-byte chunk c, c + L, ... of the row (J chunks
//   per window, a ring of D windows in registers, non-temporal), so the
//   LB = 8 (8-bit) or 4 (4-bit) lanes of one block are adjacent.  Their
//   partial dots are added by DPP, giving the exact block sum in every lane
//   of the block; one of those lanes, the one that loaded the block's scale
//   and zero point, scales it in fp32 and adds it to its accumulator, in
//   ascending block order.  At the end of a row the group's lanes are added
//   in a fixed order and the group's first lane writes y.  Rows too few to
//   give every wavefront work are shared by teams of P wavefronts, which
//   take interleaved windows and add their partial sums in LDS in
//   wavefront order.  The result does not depend on timing.
//
// Every variable part of an address is in the range-checked offset of a raw
// buffer load: chunks past the row, and rows past r1, read zeros and are
// not used.
#include <stdio.h>

#include "launch.h"

namespace qmv {
namespace {

typedef int v4i_zp __attribute__((ext_vector_type(4)));

#ifndef QMV_ZP_D12  // register ring depth for 1-2 chunks per lane
#define QMV_ZP_D12 4
#endif
#ifndef QMV_ZP_D34  // ... and for 3-4 chunks per lane
#define QMV_ZP_D34 3
#endif
#ifndef QMV_ZP_WG_PER_CU_SCALE  // scales the workgroups per compute unit
#define QMV_ZP_WG_PER_CU_SCALE 1
#endif
#ifndef QMV_ZP_FORCE_P  // 0: wavefronts per row chosen by shape
#define QMV_ZP_FORCE_P 0
#endif

constexpr int BLK = 128;               // elements per block
#ifndef QMV_ZP_QBATCH
#define QMV_ZP_QBATCH 2
#endif
constexpr int kQBatch = QMV_ZP_QBATCH;  // block pairs whose loads a wavefront issues together
constexpr int kWpb = 8;                // wavefronts per workgroup
constexpr int kOOBz = 0x7FFFFFF0;      // an offset beyond every descriptor range used here
constexpr int kBufFlagsZ = 0x00020000; // buffer descriptor word 3: raw 32-bit data

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
    const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, kBufFlagsZ);
}

// The Q8_0 rounding of one element (spec section 5): v = x * id,
// t = v + copysign(0.5, x), q = trunc(t), each operation rounded on its own.
__device__ __forceinline__ int q8_round(float x, float id) {
#pragma clang fp contract(off)
    float v = x * id;
    float t = v + copysignf(0.5f, x);
    int q = (int)t;
    return min(max(q, -127), 127);
}

// Reductions over each half-wavefront (lanes 0-31 and 32-63): DPP within
// rows of 16 lanes (swap neighbours, swap pairs, mirror 8, mirror 16), then
// the four row values read out and combined per half.  Max is exact and the
// integer sum is exact, so the order does not matter.
template <typename F>
__device__ __forceinline__ int half_reduce(int v, F op) {
    v = op(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
    v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
    v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));
    v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));
    const int r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const int r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    const int lane = threadIdx.x & 63;
    return lane < 32 ? op(r0, r1) : op(r2, r3);
}

// Quantize the 128-element block held by this half-wavefront (lane c of the
// half holds elements 4c .. 4c + 3): amax exact, d = amax / 127,
// id = 127 / amax (both correctly rounded divisions), then q8_round.
__device__ __forceinline__ void quant_half(float4 v, int (&q)[4], float &d, int &qsum) {
    const float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    // non-negative floats order like their bit patterns
    const float amax = __int_as_float(half_reduce(__float_as_int(m), [](int a, int b) { return max(a, b); }));
    d = amax / 127.0f;
    const float id = amax != 0.0f ? 127.0f / amax : 0.0f;
    q[0] = q8_round(v.x, id);
    q[1] = q8_round(v.y, id);
    q[2] = q8_round(v.z, id);
    q[3] = q8_round(v.w, id);
    qsum = half_reduce(q[0] + q[1] + q[2] + q[3], [](int a, int b) { return a + b; });
}

// position of element e of a block in the 4-bit activation order
__device__ __forceinline__ int perm4(int e) { return (e & ~7) + ((e & 1) << 2) + ((e & 7) >> 1); }

__device__ __forceinline__ int dpp_x1(int v) { return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_x2(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_m8(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false); }

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over an aligned group of L lanes (16, 32 or 64), the same value in
// every lane of the group, in a fixed order: DPP within each 16-lane row
// (neighbour swap, pair swap, mirror 8, mirror 16: after each step the value
// is uniform over 2, 4, 8, 16 lanes), then the rows' values read out and
// added ((r0 + r1) + (r2 + r3) for L = 64).
template <int L>
__device__ __forceinline__ float group_sum(float v) {
    v = v + dppf<0xB1>(v);
    v = v + dppf<0x4E>(v);
    v = v + dppf<0x141>(v);
    v = v + dppf<0x140>(v);
    if constexpr (L == 16) return v;
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(v), 48));
    if constexpr (L == 32) return (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
    return (r0 + r1) + (r2 + r3);
}

template <int BITS, int L, int J, int D, int P>
__global__ void __launch_bounds__(64 * kWpb)
k_zp(float *__restrict__ y, const uint8_t *__restrict__ wq, const float *__restrict__ wd,
     const uint8_t *__restrict__ wzp, int32_t rows, int32_t K, const float *__restrict__ x,
     int8_t *__restrict__ xq_out, float *__restrict__ xd_out, int32_t r0, int32_t r1, int32_t rows_wg) {
    constexpr int LB = BITS == 8 ? 8 : 4;  // lanes (16-byte chunks) per block
    constexpr int GPW = 64 / L;            // row groups per wavefront
    static_assert(L >= LB && (L & (L - 1)) == 0 && L <= 64, "group size");
    static_assert(P == 1 || (L == 64 && kWpb % P == 0), "teams of P wavefronts share rows of 64-lane groups");
    extern __shared__ __align__(16) unsigned char smem[];
    const int nb = K / BLK;
    int8_t *xs = reinterpret_cast<int8_t *>(smem);
    float *sd = reinterpret_cast<float *>(smem + K);
    int *sq = reinterpret_cast<int *>(smem + K + 4 * nb);

    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;

    // ---- phase B: rows
    //   P = 1: group g of L lanes takes rows r0 + g, r0 + g + G, ... (G groups
    //   in the grid), each row in W windows of L * J chunks, in order.
    //   P > 1: workgroup b takes rows_wg consecutive rows; its 8 / P teams of P
    //   wavefronts take every (8 / P)-th of them, and wavefront q of a team
    //   takes windows q, q + P, ... of the team's rows.  The P partial sums of
    //   a row meet in LDS and are added in wavefront order at the end.
    const int row_bytes = BITS == 8 ? K : K / 2;
    const int chunks = row_bytes >> 4;
    const int W = (chunks + L * J - 1) / (L * J);  // windows per row
    const int gl = lane & (L - 1);
    const int nrow = r1 - r0;
    constexpr int TPW = kWpb / P;                  // teams per workgroup (P > 1)
    const int tm = wid / P, pw = wid % P;
    const int rb0 = r0 + blockIdx.x * rows_wg;     // P > 1: this workgroup's rows
    const int rows_here = P > 1 ? max(0, min(rows_wg, r1 - rb0)) : 0;
    const int rows_team = P > 1 ? (rows_here - tm + TPW - 1) / TPW : 0;
    const int rows_team_max = P > 1 ? (rows_wg + TPW - 1) / TPW : 0;  // workgroup-uniform
    const int wpw = (W + P - 1) / P;                                   // windows per wavefront and row
    const int G = gridDim.x * kWpb * GPW;               // P = 1: row groups in the grid
    const int g0 = (blockIdx.x * kWpb + wid) * GPW;     // this wavefront's first group
    const int g = g0 + lane / L;
    const int rows_g = g < nrow ? (nrow - g + G - 1) / G : 0;
    const int rows_w = g0 < nrow ? (nrow - g0 + G - 1) / G : 0;  // the wavefront's first group has the most
    const int items = P > 1 ? rows_team_max * wpw : rows_w * W;   // wave-uniform loop count
    float *part = reinterpret_cast<float *>(smem + ((K + 8 * nb + 15) & ~15));  // P > 1: [rows_wg][P]

    // item t of this lane group: its row, window, and whether it starts or
    // ends the row's accumulation
    struct Item {
        int r, win, li;
        bool live, first, last;
    };
    auto item = [&](int t) __attribute__((always_inline)) {
        Item it;
        if constexpr (P == 1) {
            const int rl = t / W;
            it.win = t - rl * W;
            it.live = rl < rows_g;
            it.r = r0 + g + rl * G;
            it.li = 0;
            it.first = it.win == 0;
            it.last = it.win == W - 1;
        } else {
            const int i = t / wpw, k = t - i * wpw;
            it.win = pw + P * k;
            it.li = tm + TPW * i;
            it.live = i < rows_team && it.win < W;
            it.r = rb0 + it.li;
            it.first = k == 0;
            it.last = k == wpw - 1;
        }
        return it;
    };

    const __amdgpu_buffer_rsrc_t rq = rsrc(wq, (int64_t)rows * row_bytes);
    const __amdgpu_buffer_rsrc_t rd = rsrc(wd, (int64_t)rows * nb * 4);
    const __amdgpu_buffer_rsrc_t rz = rsrc(wzp, wzp != nullptr ? (int64_t)rows * nb : 0);
    const int zdef = 1 << (BITS - 1);
    constexpr int off = BITS == 8 ? 128 : 0;  // bias of the dotted codes

    // Scales and zero points: lane `sub` of a block's LB lanes loads those of
    // the slot's blocks at iterations sub, sub + LB, ... of the window, and
    // scales those blocks itself (one load per LB blocks instead of one per
    // block and lane).
    constexpr int JM = (J + LB - 1) / LB;
    struct Buf {
        v4i_zp w[J];
        float dw[JM];
        int zp[JM];
    };
    auto load = [&](Buf &bf, int t) __attribute__((always_inline)) {
        const Item it = item(t);
        const int r = it.r;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int c = (it.win * J + j) * L + gl;  // chunk of the row
            const bool ok = it.live && c < chunks;
            bf.w[j] = __builtin_bit_cast(
                v4i_zp, __builtin_amdgcn_raw_buffer_load_b128(rq, ok ? r * row_bytes + 16 * c : kOOBz, 0, 2));
        }
        const int sub = gl % LB;
#pragma unroll
        for (int m = 0; m < JM; ++m) {
            const int jj = sub + LB * m;  // the iteration whose block this lane scales
            const int c = (it.win * J + jj) * L + (gl - sub);
            const bool ok = it.live && jj < J && c < chunks;
            const int b = c / LB;
            bf.dw[m] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(rd, ok ? 4 * (r * nb + b) : kOOBz, 0, 0));
            if (wzp != nullptr)
                bf.zp[m] = (int)__builtin_amdgcn_raw_buffer_load_b8(rz, ok ? r * nb + b : kOOBz, 0, 0);
            else
                bf.zp[m] = zdef;
        }
    };

    float acc = 0.0f;
    auto compute = [&](const Buf &bf, int t) __attribute__((always_inline)) {
        const Item it = item(t);
        if (it.first) acc = 0.0f;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int c = (it.win * J + j) * L + gl;
            const bool ok = it.live && c < chunks;
            const int b = ok ? c / LB : 0;
            const int sub = c % LB;
            int p = 0;
            if constexpr (BITS == 8) {
                const v4i_zp xv = *reinterpret_cast<const v4i_zp *>(xs + b * BLK + 16 * sub);
#pragma unroll
                for (int k = 0; k < 4; ++k) p = __builtin_amdgcn_sdot4(bf.w[j][k] ^ (int)0x80808080, xv[k], p, false);
            } else {
                const v4i_zp xe = *reinterpret_cast<const v4i_zp *>(xs + b * BLK + 32 * sub);
                const v4i_zp xo = *reinterpret_cast<const v4i_zp *>(xs + b * BLK + 32 * sub + 16);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    // dword k covers elements 8k .. 8k + 7 of the chunk: even ones in the
                    // low nibbles, odd ones in the high nibbles
                    const int lo = bf.w[j][k] & 0x0F0F0F0F, hi = (bf.w[j][k] >> 4) & 0x0F0F0F0F;
                    const int xe_k = k < 2 ? xe[2 * k] : xo[2 * k - 4];
                    const int xo_k = k < 2 ? xe[2 * k + 1] : xo[2 * k - 3];
                    p = __builtin_amdgcn_sdot4(lo, xe_k, p, false);
                    p = __builtin_amdgcn_sdot4(hi, xo_k, p, false);
                }
            }
            // exact block sum in every lane of the block
            p += dpp_x1(p);
            p += dpp_x2(p);
            if constexpr (LB == 8) p += dpp_m8(p);
            if (ok && sub == j % LB) {
#pragma clang fp contract(off)
                const int sumi = p - (bf.zp[j / LB] - off) * sq[b];
                float tt = (float)sumi * bf.dw[j / LB];
                tt = tt * sd[b];
                acc = acc + tt;
            }
        }
        if (it.last) {
            const float s = group_sum<L>(acc);
            if constexpr (P == 1) {
                if (it.live && gl == 0) y[it.r] = s;
            } else {
                // this wavefront's share of the row (0 if it had no window of it)
                if (it.li < rows_here && gl == 0) part[it.li * P + pw] = s;
            }
        }
    };

    // ring of D register buffers, D - 1 items in flight ahead of the one
    // being computed (unrolled by D so that each buffer has fixed registers)
    Buf ring[D];
#pragma unroll
    for (int d = 0; d < D - 1; ++d) load(ring[d], d);  // the weights do not wait for the activation

    // ---- phase A: the activation, quantized into LDS.  Each half-wavefront
    // takes one block (4 elements per lane); a wavefront first issues the
    // loads of up to kQBatch block pairs, then quantizes them.
    for (int base = 2 * wid; base < nb; base += 2 * kWpb * kQBatch) {
        float4 v[kQBatch];
#pragma unroll
        for (int u = 0; u < kQBatch; ++u) {
            const int b = base + 2 * kWpb * u + (lane >> 5);
            v[u] = b < nb ? *reinterpret_cast<const float4 *>(x + (int64_t)b * BLK + 4 * (lane & 31))
                          : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
#pragma unroll
        for (int u = 0; u < kQBatch; ++u) {
            const int b0 = base + 2 * kWpb * u;
            if (b0 >= nb) break;  // wave-uniform
            const int b = b0 + (lane >> 5);
            int q[4], qs;
            float d;
            quant_half(v[u], q, d, qs);
            if (b < nb) {
                const int e = 4 * (lane & 31);
                const int pk = (q[0] & 0xFF) | ((q[1] & 0xFF) << 8) | ((q[2] & 0xFF) << 16) | (q[3] << 24);
                if constexpr (BITS == 8) {
                    *reinterpret_cast<int *>(xs + b * BLK + e) = pk;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) xs[b * BLK + perm4(e + i)] = (int8_t)q[i];
                }
                if ((lane & 31) == 0) {
                    sd[b] = d;
                    sq[b] = qs;
                }
                if (xq_out != nullptr && blockIdx.x == 0) {
                    *reinterpret_cast<int *>(xq_out + (int64_t)b * BLK + e) = pk;
                    if ((lane & 31) == 0) xd_out[b] = d;
                }
            }
        }
    }
    __syncthreads();

    for (int t0 = 0; t0 < items; t0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int t = t0 + d;
            if (t < items) {  // wave-uniform
                load(ring[(d + D - 1) % D], t + D - 1);
                compute(ring[d], t);
            }
        }
    }
    if constexpr (P > 1) {
        __syncthreads();
        for (int li = threadIdx.x; li < rows_here; li += 64 * kWpb) {
            float s = part[li * P];
#pragma unroll
            for (int q = 1; q < P; ++q) s += part[li * P + q];
            y[rb0 + li] = s;
        }
    }
}

template <int BITS, int L, int J, int P>
hipError_t launch_cfg(const ZpArgs &a, int grid, int rows_wg, size_t lds, hipStream_t s, const char **name) {
    constexpr int D = J <= 2 ? QMV_ZP_D12 : J <= 4 ? QMV_ZP_D34 : 2;
    auto kern = k_zp<BITS, L, J, D, P>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * kWpb), lds, s, a.y, a.wq, a.wd, a.wzp, a.rows, a.K, a.x,
                       a.xq_out, a.xd_out, a.r0, a.r1, rows_wg);
    static char kname[48];
    if (kname[0] == 0) snprintf(kname, sizeof kname, "zp%d_l%d_j%d_d%d_p%d", BITS, L, J, D, P);
    *name = kname;
    return hipGetLastError();
}

template <int BITS, int P>
hipError_t launch_j(const ZpArgs &a, int J, int grid, int rows_wg, size_t lds, hipStream_t s, const char **name) {
    switch (J) {
        case 1: return launch_cfg<BITS, 64, 1, P>(a, grid, rows_wg, lds, s, name);
        case 2: return launch_cfg<BITS, 64, 2, P>(a, grid, rows_wg, lds, s, name);
        case 3: return launch_cfg<BITS, 64, 3, P>(a, grid, rows_wg, lds, s, name);
        case 4: return launch_cfg<BITS, 64, 4, P>(a, grid, rows_wg, lds, s, name);
        case 5: return launch_cfg<BITS, 64, 5, P>(a, grid, rows_wg, lds, s, name);
        case 6: return launch_cfg<BITS, 64, 6, P>(a, grid, rows_wg, lds, s, name);
        case 7: return launch_cfg<BITS, 64, 7, P>(a, grid, rows_wg, lds, s, name);
        default: return launch_cfg<BITS, 64, 8, P>(a, grid, rows_wg, lds, s, name);
    }
}

// J chunks per lane per window (at most 8) for rows of `chunks` chunks split
// over P wavefronts: the windows of a row as even as possible.
int pick_j(int chunks, int P) {
    const int per = (chunks + P - 1) / P;  // chunks per wavefront and row
    const int win = (per + 64 * 8 - 1) / (64 * 8);
    return (per + 64 * win - 1) / (64 * win);
}

template <int BITS>
hipError_t launch_bits(const ZpArgs &a, int num_cu, hipStream_t s, const char **name) {
    const int chunks = (BITS == 8 ? a.K : a.K / 2) / 16;
    const size_t lds_x = ((size_t)a.K + 8 * (size_t)(a.K / BLK) + 15) & ~(size_t)15;
    const int nrow = a.r1 - a.r0;
    // lanes per row: the fewest power of two (16 .. 64) that covers a row
    int L = 64;
    if (chunks <= 16) L = 16;
    else if (chunks <= 32) L = 32;
    const int wgpc = L < 64 || pick_j(chunks, 1) == 1 ? 4 : 2;  // workgroups per compute unit
    const int waves = QMV_ZP_WG_PER_CU_SCALE * wgpc * num_cu * kWpb;
    // rows shared by a team of P wavefronts when there are fewer than two
    // rows per wavefront and each row has at least two windows' worth
    int P = 1;
    if (L == 64 && chunks >= 128) {
        while (P < kWpb && (int64_t)nrow * P < 2 * (int64_t)waves && chunks / (2 * P) >= 64) P *= 2;
    }
#if QMV_ZP_FORCE_P
    if (L == 64) P = QMV_ZP_FORCE_P;
#endif
    if (P == 1) {
        const int groups_per_wg = kWpb * (64 / L);
        int grid = (nrow + groups_per_wg - 1) / groups_per_wg;
        if (grid > waves / kWpb) grid = waves / kWpb;
        if (grid < 1) grid = 1;
        if (L == 16) return launch_cfg<BITS, 16, 1, 1>(a, grid, 0, lds_x, s, name);
        if (L == 32) return launch_cfg<BITS, 32, 1, 1>(a, grid, 0, lds_x, s, name);
        return launch_j<BITS, 1>(a, pick_j(chunks, 1), grid, 0, lds_x, s, name);
    }
    // P > 1: consecutive rows per workgroup, enough workgroups to give each
    // wavefront work, partial sums in LDS (at most 8 KiB of them)
    int grid = waves / kWpb;
    int rows_wg = (nrow + grid - 1) / grid;
    if (rows_wg < 1) rows_wg = 1;
    if (rows_wg * P > 2048) rows_wg = 2048 / P;
    grid = (nrow + rows_wg - 1) / rows_wg;
    if (grid < 1) grid = 1;
    const size_t lds = lds_x + (size_t)rows_wg * P * 4;
    const int J = pick_j(chunks, P);
    if (P == 2) return launch_j<BITS, 2>(a, J, grid, rows_wg, lds, s, name);
    if (P == 4) return launch_j<BITS, 4>(a, J, grid, rows_wg, lds, s, name);
    return launch_j<BITS, 8>(a, J, grid, rows_wg, lds, s, name);
}

__global__ void __launch_bounds__(256)
k_quant_b128(int8_t *__restrict__ q, float *__restrict__ d, const float *__restrict__ x, int64_t nblk) {
    // one block per half-wavefront, 4 elements per lane (as the matvec's
    // activation phase, hence the same bits)
    const int lane = threadIdx.x & 63;
    const int64_t h0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;  // wavefront
    const int64_t nw = ((int64_t)gridDim.x * 256) >> 6;
    for (int64_t b0 = 2 * h0; b0 < nblk; b0 += 2 * nw) {  // wave-uniform
        const int64_t b = b0 + (lane >> 5);
        const float4 v = b < nblk ? *reinterpret_cast<const float4 *>(x + b * BLK + 4 * (lane & 31))
                                  : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        int qv[4], qs;
        float dd;
        quant_half(v, qv, dd, qs);
        if (b < nblk) {
            *reinterpret_cast<int *>(q + b * BLK + 4 * (lane & 31)) =
                (qv[0] & 0xFF) | ((qv[1] & 0xFF) << 8) | ((qv[2] & 0xFF) << 16) | (qv[3] << 24);
            if ((lane & 31) == 0) d[b] = dd;
        }
    }
}

}  // namespace

size_t zp_lds_bytes(int32_t K) { return (((size_t)K + 8 * (size_t)(K / BLK) + 15) & ~(size_t)15) + 8192; }

hipError_t launch_zp(const ZpArgs &a, int num_cu, hipStream_t s, const char **name) {
    if (a.K % BLK != 0 || zp_lds_bytes(a.K) > 160 * 1024) return hipErrorNotSupported;
    return a.bits == 8 ? launch_bits<8>(a, num_cu, s, name) : launch_bits<4>(a, num_cu, s, name);
}

hipError_t launch_quant_b128(int8_t *q, float *d, const float *x, int64_t nblk, hipStream_t s, const char **name) {
    int64_t g = (nblk + 7) / 8;  // 8 blocks per workgroup of 4 wavefronts
    if (g > 4096) g = 4096;
    if (g < 1) g = 1;
    hipLaunchKernelGGL(k_quant_b128, dim3((unsigned)g), dim3(256), 0, s, q, d, x, nblk);
    *name = "quant_q8_b128";
    return hipGetLastError();
}

}  // namespace qmv
