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
// Work layout.  Workgroups of 8 wavefronts, 2 or 4 per compute unit, for
// rows of one chunk per lane; of 16 wavefronts, one per compute unit, for
// longer rows (the choice is rowstream.h's).
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
#include "count.h"
#include "rowstream.h"

namespace qmv {
namespace {

using rs::kOOB;
using rs::v4i;

#ifndef QMV_GS  // split-K kernel (kernels_gs.hip) for rows of 128 and more units
#define QMV_GS 1
#endif
#ifndef QMV_ZP_D12  // register ring depth for 1-2 chunks per lane
#define QMV_ZP_D12 3
#endif
#ifndef QMV_ZP_D34  // ... and for 3-4 chunks per lane
#define QMV_ZP_D34 2
#endif

constexpr int BLK = 128;    // elements per block
constexpr int kQBatch = 2;  // block pairs whose loads a wavefront issues together

// position of element e of a block in the 4-bit activation order
__device__ __forceinline__ int perm4(int e) { return (e & ~7) + ((e & 1) << 2) + ((e & 7) >> 1); }

template <int BITS, int L, int J, int D, int P, int WPB>
__global__ void __launch_bounds__(64 * WPB)
k_zp(float *__restrict__ y, const uint8_t *__restrict__ wq, const float *__restrict__ wd,
     const uint8_t *__restrict__ wzp, int32_t rows, int32_t K, const float *__restrict__ x,
     int8_t *__restrict__ xq_out, float *__restrict__ xd_out, int32_t r0, int32_t r1, int32_t rows_wg) {
    constexpr int LB = BITS == 8 ? 8 : 4;  // lanes (16-byte chunks) per block
    static_assert(L >= LB && (L & (L - 1)) == 0 && L <= 64, "group size");
    static_assert(P == 1 || (L == 64 && WPB % P == 0), "teams of P wavefronts share rows of 64-lane groups");
    extern __shared__ __align__(16) unsigned char smem[];
    const int nb = K / BLK;
    int8_t *xs = reinterpret_cast<int8_t *>(smem);                          // [K]
    float *sd = reinterpret_cast<float *>(smem + K);                        // [nb] block scales
    int *sq = reinterpret_cast<int *>(smem + K + 4 * nb);                   // [nb] sums of the quants
    float *part = reinterpret_cast<float *>(smem + ((K + 8 * nb + 15) & ~15));  // P > 1: [rows_wg][P]

    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int row_bytes = BITS == 8 ? K : K / 2;
    const int chunks = row_bytes >> 4;
    const int gl = lane & (L - 1);
    const rs::RowMap<L, P, WPB> map(chunks, J, r0, r1, rows_wg);

    const __amdgpu_buffer_rsrc_t rq = rs::rsrc(wq, (int64_t)rows * row_bytes);
    const __amdgpu_buffer_rsrc_t rd = rs::rsrc(wd, (int64_t)rows * nb * 4);
    const __amdgpu_buffer_rsrc_t rz = rs::rsrc(wzp, wzp != nullptr ? (int64_t)rows * nb : 0);
    const int zdef = 1 << (BITS - 1);
    constexpr int off = BITS == 8 ? 128 : 0;  // bias of the dotted codes

    // Scales and zero points: lane `sub` of a block's LB lanes loads those of
    // the slot's blocks at iterations sub, sub + LB, ... of the window, and
    // scales those blocks itself (one load per LB blocks instead of one per
    // block and lane).
    constexpr int JM = (J + LB - 1) / LB;
    struct Buf {
        v4i w[J];
        float dw[JM];
        int zp[JM];
    };
    // When a block's LB lanes outnumber the J * D (item, iteration) pairs of
    // a ring turn, the turn shares one load instead: lane `sub` < J * D of the
    // block's lanes loads the scale and zero point of iteration sub % J of
    // item t0 + sub / J (the turn starting at item t0), and scales that
    // block sum itself.
    constexpr bool IB = J * D <= LB;
    struct Sc {
        float dw;
        int zp;
    };
    auto load_sc = [&](int tb) __attribute__((always_inline)) {
        Sc sc;
        const int sub = gl % LB, di = sub / J, jj = sub % J;
        const rs::Item it = map.item(tb + (di < D ? di : 0));
        const int c = (it.win * J + jj) * L + (gl - sub);  // the first chunk of that block
        const bool ok = di < D && it.live && c < chunks;
        const int b = c / LB;
        sc.dw = __builtin_bit_cast(float,
                                   __builtin_amdgcn_raw_buffer_load_b32(rd, ok ? 4 * (it.r * nb + b) : kOOB, 0, 0));
        sc.zp = wzp != nullptr ? (int)__builtin_amdgcn_raw_buffer_load_b8(rz, ok ? it.r * nb + b : kOOB, 0, 0) : zdef;
        return sc;
    };
    auto load = [&](Buf &bf, int t) __attribute__((always_inline)) {
        const rs::Item it = map.item(t);
        const int r = it.r;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int c = (it.win * J + j) * L + gl;  // chunk of the row
            const bool ok = it.live && c < chunks;
            bf.w[j] = __builtin_bit_cast(
                v4i, __builtin_amdgcn_raw_buffer_load_b128(rq, ok ? r * row_bytes + 16 * c : kOOB, 0, 2));
        }
        const int sub = gl % LB;
#pragma unroll
        for (int m = 0; m < (IB ? 0 : JM); ++m) {
            const int jj = sub + LB * m;  // the iteration whose block this lane scales
            const int c = (it.win * J + jj) * L + (gl - sub);
            const bool ok = it.live && jj < J && c < chunks;
            const int b = c / LB;
            bf.dw[m] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(rd, ok ? 4 * (r * nb + b) : kOOB, 0, 0));
            if (wzp != nullptr)
                bf.zp[m] = (int)__builtin_amdgcn_raw_buffer_load_b8(rz, ok ? r * nb + b : kOOB, 0, 0);
            else
                bf.zp[m] = zdef;
        }
    };

    float acc = 0.0f;
    auto compute = [&](const Buf &bf, int t, const Sc &sc, int dpos) __attribute__((always_inline)) {
        const rs::Item it = map.item(t);
        if (it.first) acc = 0.0f;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int c = (it.win * J + j) * L + gl;
            const bool ok = it.live && c < chunks;
            const int b = ok ? c / LB : 0;
            const int sub = c % LB;
            int p = 0;
            if constexpr (BITS == 8) {
                const v4i xv = *reinterpret_cast<const v4i *>(xs + b * BLK + 16 * sub);
#pragma unroll
                for (int k = 0; k < 4; ++k) p = __builtin_amdgcn_sdot4(bf.w[j][k] ^ (int)0x80808080, xv[k], p, false);
            } else {
                const v4i xe = *reinterpret_cast<const v4i *>(xs + b * BLK + 32 * sub);
                const v4i xo = *reinterpret_cast<const v4i *>(xs + b * BLK + 32 * sub + 16);
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
            p += rs::dppi<rs::kX1>(p);
            p += rs::dppi<rs::kX2>(p);
            if constexpr (LB == 8) p += rs::dppi<rs::kM8>(p);
            if (ok && sub == (IB ? dpos * J + j : j % LB)) {
#pragma clang fp contract(off)
                const int sumi = p - ((IB ? sc.zp : bf.zp[j / LB]) - off) * sq[b];
                float tt = (float)sumi * (IB ? sc.dw : bf.dw[j / LB]);
                tt = tt * sd[b];
                acc = acc + tt;
            }
        }
        if (it.last) {
            const float s = rs::group_sum<L>(acc);
            if constexpr (P == 1) {
                if (it.live && gl == 0) y[it.r] = s;
            } else {
                // this wavefront's share of the row (0 if it had no window of it)
                if (it.li < map.rows_here && gl == 0) part[it.li * P + map.pw] = s;
            }
        }
    };

    // ---- phase A: the activation, quantized into LDS.  Each half-wavefront
    // takes one block (4 elements per lane); a wavefront issues the loads of
    // up to kQBatch block pairs, then quantizes them.  The first batch is
    // requested before the first weights: loads return in order, so the
    // activation does not wait behind the weight stream.
    float4 v[kQBatch];
    auto load_x = [&](int base) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kQBatch; ++u) {
            const int b = base + 2 * WPB * u + (lane >> 5);
            v[u] = b < nb ? *reinterpret_cast<const float4 *>(x + (int64_t)b * BLK + 4 * (lane & 31))
                          : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    };
    load_x(2 * wid);
    // ring of D register buffers, D - 1 items in flight ahead of the one
    // being computed (unrolled by D so that each buffer has fixed registers)
    Sc cur = {}, nxt = {};
    if constexpr (IB) nxt = load_sc(0);  // (measured: ahead of the weights is faster here)
    Buf ring[D];
#pragma unroll
    for (int d = 0; d < D - 1; ++d) load(ring[d], d);  // the weights do not wait for the activation

    for (int base = 2 * wid; base < nb; base += 2 * WPB * kQBatch) {
        if (base != 2 * wid) load_x(base);  // later batches (wave-uniform)
#pragma unroll
        for (int u = 0; u < kQBatch; ++u) {
            const int b0 = base + 2 * WPB * u;
            if (b0 >= nb) break;  // wave-uniform
            const int b = b0 + (lane >> 5);
            int q[4], qs;
            float d;
            rs::quant_half(v[u], q, d, qs);
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

    // ---- phase B: the rows
    const int items = map.items;
#if QMV_RS_TAIL
    // whole ring turns while every load of the turn is one of this
    // wavefront's items, then the remaining R items (1 .. 2 D - 2) as code
    // specialised on R: no loads past the last item, exact waits
    int t0 = 0;
    for (; t0 + 2 * D - 2 < items; t0 += D) {
        if constexpr (IB) {
            cur = nxt;
            nxt = load_sc(t0 + D);
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load(ring[(d + D - 1) % D], t0 + d + D - 1);
            compute(ring[d], t0 + d, cur, d);
        }
    }
    with_count<1, 2 * D - 2>(items - t0, [&](auto rc) __attribute__((always_inline)) {
        constexpr int R = decltype(rc)::value;
#pragma unroll
        for (int q = 0; q < R; ++q) {
            if constexpr (IB) {
                if (q % D == 0) {
                    cur = nxt;
                    if (q + D < R) nxt = load_sc(t0 + q + D);
                }
            }
            if (q + D - 1 < R) load(ring[(q + D - 1) % D], t0 + q + D - 1);
            compute(ring[q % D], t0 + q, cur, q % D);
        }
    });
#else
    for (int t0 = 0; t0 < items; t0 += D) {
        if constexpr (IB) {
            cur = nxt;
            nxt = load_sc(t0 + D);
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int t = t0 + d;
            if (t < items) {  // wave-uniform
                load(ring[(d + D - 1) % D], t + D - 1);
                compute(ring[d], t, cur, d);
            }
        }
    }
#endif
    if constexpr (P > 1) {
        __syncthreads();
        for (int li = threadIdx.x; li < map.rows_here; li += 64 * WPB) {
            float s = part[li * P];
#pragma unroll
            for (int q = 1; q < P; ++q) s += part[li * P + q];
            y[map.rb0 + li] = s;
        }
    }
}

// Register ring depth: 3 stages for one chunk per lane (and two of 8-bit
// codes), measured faster than 4 once no loads past the last item are
// issued (8-bit Qwen W_down 4.54 -> 4.37 us, 4-bit lm_head 18.7 -> 17.6 us);
// 2 stages wherever a deeper ring would take the ring turn past one scale
// load (J * D > LB), measured faster on every such shape.
constexpr int ring_depth(int bits, int J) {
    return (J == 1 || (J == 2 && bits == 8)) ? QMV_ZP_D12 : J <= 4 ? QMV_ZP_D34 : 2;
}

template <int BITS, int L, int J, int P, int WPB>
hipError_t launch_cfg(const ZpArgs &a, int grid, int rows_wg, size_t lds, hipStream_t s, const char **name) {
    constexpr int D = ring_depth(BITS, J);
    auto kern = k_zp<BITS, L, J, D, P, WPB>;
    static const std::string kname = variant_name("zp%d_l%d_j%d_d%d_p%d_w%d", BITS, L, J, D, P, WPB);
    hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WPB), lds, s, a.y, a.wq, a.wd, a.wzp, a.rows, a.K, a.x,
                       a.xq_out, a.xd_out, a.r0, a.r1, rows_wg);
    *name = kname.c_str();
    return hipGetLastError();
}

// 64-lane groups in workgroups of 16 wavefronts (rows of two or more chunks
// per lane, or shared by teams)
template <int BITS, int P>
hipError_t launch_j(const ZpArgs &a, int J, int grid, int rows_wg, size_t lds, hipStream_t s, const char **name) {
    switch (J) {
        case 1: return launch_cfg<BITS, 64, 1, P, 16>(a, grid, rows_wg, lds, s, name);
        case 2: return launch_cfg<BITS, 64, 2, P, 16>(a, grid, rows_wg, lds, s, name);
        case 3: return launch_cfg<BITS, 64, 3, P, 16>(a, grid, rows_wg, lds, s, name);
        case 4: return launch_cfg<BITS, 64, 4, P, 16>(a, grid, rows_wg, lds, s, name);
        case 5: return launch_cfg<BITS, 64, 5, P, 16>(a, grid, rows_wg, lds, s, name);
        case 6: return launch_cfg<BITS, 64, 6, P, 16>(a, grid, rows_wg, lds, s, name);
        case 7: return launch_cfg<BITS, 64, 7, P, 16>(a, grid, rows_wg, lds, s, name);
        default: return launch_cfg<BITS, 64, 8, P, 16>(a, grid, rows_wg, lds, s, name);
    }
}

template <int BITS>
hipError_t launch_bits(const ZpArgs &a, int num_cu, hipStream_t s, const char **name) {
    const int chunks = (BITS == 8 ? a.K : a.K / 2) / 16;
    const size_t lds_x = ((size_t)a.K + 8 * (size_t)(a.K / BLK) + 15) & ~(size_t)15;
    const int nrow = a.r1 - a.r0;
    rs::Shape sh = rs::pick_shape(chunks, nrow, num_cu, BITS == 8 ? 8 : 4, 8, BITS == 8 ? 64 : 32);
    // rows already shared by teams: more wavefronts per row until a ring
    // turn takes one scale load (J * D <= LB); measured faster on the
    // Llama-7B W_down shape (8-bit P = 2 -> 4: 13.3 -> 11.8 us)
    while (sh.P > 1 && sh.P < 8 && sh.J * ring_depth(BITS, sh.J) > (BITS == 8 ? 8 : 4)) {
        sh.P *= 2;
        sh.J = rs::pick_j(chunks, sh.P);
    }
    const int waves = sh.wgpc * num_cu * sh.wpb;
    if (sh.P == 1) {
        const int groups_per_wg = sh.wpb * (64 / sh.L);
        int grid = (nrow + groups_per_wg - 1) / groups_per_wg;
        if (grid > waves / sh.wpb) grid = waves / sh.wpb;
        if (grid < 1) grid = 1;
        if (sh.L == 16) return launch_cfg<BITS, 16, 1, 1, 8>(a, grid, 0, lds_x, s, name);
        if (sh.L == 32) return launch_cfg<BITS, 32, 1, 1, 8>(a, grid, 0, lds_x, s, name);
        if (sh.wpb == 8) return launch_cfg<BITS, 64, 1, 1, 8>(a, grid, 0, lds_x, s, name);
        return launch_j<BITS, 1>(a, sh.J, grid, 0, lds_x, s, name);
    }
    // P > 1: consecutive rows per workgroup, enough workgroups to give each
    // wavefront work, partial sums in LDS (at most 8 KiB of them)
    int grid = waves / sh.wpb;
    int rows_wg = (nrow + grid - 1) / grid;
    if (rows_wg < 1) rows_wg = 1;
    if (rows_wg * sh.P > 2048) rows_wg = 2048 / sh.P;
    grid = (nrow + rows_wg - 1) / rows_wg;
    if (grid < 1) grid = 1;
    const size_t lds = lds_x + (size_t)rows_wg * sh.P * 4;
    if (sh.P == 2) return launch_j<BITS, 2>(a, sh.J, grid, rows_wg, lds, s, name);
    if (sh.P == 4) return launch_j<BITS, 4>(a, sh.J, grid, rows_wg, lds, s, name);
    return launch_j<BITS, 8>(a, sh.J, grid, rows_wg, lds, s, name);
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
        rs::quant_half(v, qv, dd, qs);
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
#if QMV_GS
    const hipError_t e = launch_gs_zp(a, num_cu, s, name);  // the split-K form where it takes the shape
    if (e != hipErrorNotSupported) return e;
#endif
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
