// kernels_q4k.hip -- the decode matvec on K-quant super-blocks with the
// sub-block scales folded in the integer domain (gfx950).
//
// What is computed ("SKaiNET-native-kernels" page, section "Proving an
// optimization is safe before writing it"; the value and storage are this
// library's reading, the page giving neither): a weight element of
// sub-block b (32 elements) of super-block k (8 sub-blocks) has the value
// d[k] * sc[b] * w - dmin[k] * mn[b], with 4-bit w (the spec's Q4_0 nibble
// layout within each sub-block, stored as is), 6-bit scale sc and minimum mn
// per sub-block, fp32 d and dmin per super-block.  The float activation is
// quantized to int8 per 256-element block with the Q8_0 rule of the
// Legacy-ISA ML Inference Runtime -- Design Spec (section 4 "Q8
// quantization", section 5 rounding), and per super-block
//   S1 = sum_b sc[b] * (sum_i w_i * q_i)   (the page's integer fold, exact:
//                                            |S1| <= 8*63*32*127*15)
//   S2 = sum_b mn[b] * (sum_i q_i),
//   y[r] = sum over super-blocks of ((float)S1 * d - (float)S2 * dmin) * dx.
//
// Work layout (the row streaming of rowstream.h).  Phase A: the workgroup
// quantizes the activation into LDS, one wavefront per 256-element block (4
// elements per lane), keeping the block scales and the sums of the quants of
// each 32-element sub-block.  Phase B: each lane's 16-byte chunk is one
// sub-block: two masks and 8 v_dot4 give its integer dot, the lane
// multiplies it by its scale and the sub-block's quant sum by its minimum,
// and DPP over the super-block's 8 lanes gives S1 and S2 exactly; the lane
// that loaded the super-block's d and dmin applies them and dx in fp32.  The
// first weight loads are issued before phase A.  The result does not depend
// on timing.
//
// Every variable part of an address is in the range-checked offset of a raw
// buffer load: chunks past the row, and rows past r1, read zeros and are
// not used.
#include <stdio.h>

#include "launch.h"
#include "count.h"
#include "rowstream.h"

#ifndef QMV_GS  // split-K kernel (kernels_gs.hip) for rows of 128 and more sub-blocks
#define QMV_GS 1
#endif

#ifndef QMV_Q4K_D12  // register ring depth for 1-2 chunks per lane
#define QMV_Q4K_D12 3
#endif

namespace qmv {
namespace {

using rs::kOOB;
using rs::v4i;

constexpr int SB = 256;     // elements per super-block
constexpr int SUB = 32;     // elements per sub-block (one 16-byte chunk)
constexpr int LB = SB / SUB;  // chunks (lanes) per super-block
constexpr int kQBatch = 2;  // blocks whose loads a wavefront issues together

template <int L, int J, int D, int P, int WPB>
__global__ void __launch_bounds__(64 * WPB)
k_q4k(float *__restrict__ y, const uint8_t *__restrict__ wq, const uint8_t *__restrict__ wsc,
      const uint8_t *__restrict__ wmn, const float *__restrict__ wd, const float *__restrict__ wdm, int32_t rows,
      int32_t K, const float *__restrict__ x, int8_t *__restrict__ xq_out, float *__restrict__ xd_out, int32_t r0,
      int32_t r1, int32_t rows_wg) {
    static_assert(L >= LB && (L & (L - 1)) == 0 && L <= 64, "group size");
    static_assert(P == 1 || (L == 64 && WPB % P == 0), "teams of P wavefronts share rows of 64-lane groups");
    extern __shared__ __align__(16) unsigned char smem[];
    const int nk = K / SB, nsub = K / SUB;
    int8_t *xs = reinterpret_cast<int8_t *>(smem);                   // [K]
    float *sd = reinterpret_cast<float *>(smem + K);                 // [nk] block scales
    int *sqs = reinterpret_cast<int *>(smem + K + 4 * nk);           // [nsub] sums of the quants per sub-block
    float *part = reinterpret_cast<float *>(smem + ((K + 4 * nk + 4 * nsub + 15) & ~15));  // P > 1: [rows_wg][P]

    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int chunks = nsub;  // 16 bytes of nibbles per sub-block
    const int row_bytes = K / 2;
    const int gl = lane & (L - 1);
    const rs::RowMap<L, P, WPB> map(chunks, J, r0, r1, rows_wg);

    const __amdgpu_buffer_rsrc_t rq = rs::rsrc(wq, (int64_t)rows * row_bytes);
    const __amdgpu_buffer_rsrc_t rsc = rs::rsrc(wsc, (int64_t)rows * nsub);
    const __amdgpu_buffer_rsrc_t rmn = rs::rsrc(wmn, (int64_t)rows * nsub);
    const __amdgpu_buffer_rsrc_t rd = rs::rsrc(wd, (int64_t)rows * nk * 4);
    const __amdgpu_buffer_rsrc_t rdm = rs::rsrc(wdm, (int64_t)rows * nk * 4);

    // d and dmin: lane `sub` of a super-block's 8 lanes loads those of the
    // slot's super-blocks at iterations sub, sub + 8, ... and applies them.
    constexpr int JM = (J + LB - 1) / LB;
    struct Buf {
        v4i w[J];
        int sc[J], mn[J];
        float d[JM], dm[JM];
    };
    // When a super-block's 8 lanes outnumber the J * D (item, iteration)
    // pairs of a ring turn, the turn shares one load instead: lane `sub` <
    // J * D of the super-block's lanes loads d and dmin of iteration sub % J
    // of item t0 + sub / J (the turn starting at item t0), and applies them
    // to that S1 and S2 itself.
    constexpr bool IB = J * D <= LB;
    struct Sc {
        float d, dm;
    };
    auto load_sc = [&](int tb) __attribute__((always_inline)) {
        Sc sc;
        const int sub = gl % LB, di = sub / J, jj = sub % J;
        const rs::Item it = map.item(tb + (di < D ? di : 0));
        const int c = (it.win * J + jj) * L + (gl - sub);  // the first sub-block of that super-block
        const bool ok = di < D && it.live && c < chunks;
        const int k = c / LB;
        sc.d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, ok ? 4 * (it.r * nk + k) : kOOB, 0, 0));
        sc.dm = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdm, ok ? 4 * (it.r * nk + k) : kOOB, 0, 0));
        return sc;
    };
    auto load = [&](Buf &bf, int t) __attribute__((always_inline)) {
        const rs::Item it = map.item(t);
        const int r = it.r;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int c = (it.win * J + j) * L + gl;  // sub-block of the row
            const bool ok = it.live && c < chunks;
            bf.w[j] = __builtin_bit_cast(
                v4i, __builtin_amdgcn_raw_buffer_load_b128(rq, ok ? r * row_bytes + 16 * c : kOOB, 0, 2));
            bf.sc[j] = (int)__builtin_amdgcn_raw_buffer_load_b8(rsc, ok ? r * nsub + c : kOOB, 0, 0);
            bf.mn[j] = (int)__builtin_amdgcn_raw_buffer_load_b8(rmn, ok ? r * nsub + c : kOOB, 0, 0);
        }
        const int sub = gl % LB;
#pragma unroll
        for (int m = 0; m < (IB ? 0 : JM); ++m) {
            const int jj = sub + LB * m;
            const int c = (it.win * J + jj) * L + (gl - sub);
            const bool ok = it.live && jj < J && c < chunks;
            const int k = c / LB;
            bf.d[m] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, ok ? 4 * (r * nk + k) : kOOB, 0, 0));
            bf.dm[m] =
                __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdm, ok ? 4 * (r * nk + k) : kOOB, 0, 0));
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
            const int cc = ok ? c : 0;
            const int sub = c % LB;
            // byte j of the chunk holds elements j (low nibble) and j + 16 (high)
            const v4i xa = *reinterpret_cast<const v4i *>(xs + SUB * cc);
            const v4i xb = *reinterpret_cast<const v4i *>(xs + SUB * cc + 16);
            int p = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                p = __builtin_amdgcn_sdot4(bf.w[j][k] & 0x0F0F0F0F, xa[k], p, false);
                p = __builtin_amdgcn_sdot4((bf.w[j][k] >> 4) & 0x0F0F0F0F, xb[k], p, false);
            }
            int s1 = bf.sc[j] * p, s2 = bf.mn[j] * sqs[cc];
            // the super-block's S1 and S2, exact, in every lane of it
            s1 += rs::dppi<rs::kX1>(s1);
            s2 += rs::dppi<rs::kX1>(s2);
            s1 += rs::dppi<rs::kX2>(s1);
            s2 += rs::dppi<rs::kX2>(s2);
            s1 += rs::dppi<rs::kM8>(s1);
            s2 += rs::dppi<rs::kM8>(s2);
            if (ok && sub == (IB ? dpos * J + j : j % LB)) {
#pragma clang fp contract(off)
                const float tt = (float)s1 * (IB ? sc.d : bf.d[j / LB]);
                const float uu = (float)s2 * (IB ? sc.dm : bf.dm[j / LB]);
                float v = tt - uu;
                v = v * sd[cc / LB];
                acc = acc + v;
            }
        }
        if (it.last) {
            const float s = rs::group_sum<L>(acc);
            if constexpr (P == 1) {
                if (it.live && gl == 0) y[it.r] = s;
            } else {
                if (it.li < map.rows_here && gl == 0) part[it.li * P + map.pw] = s;
            }
        }
    };

    // ---- phase A: the activation, quantized into LDS, one wavefront per
    // 256-element block; a wavefront issues the loads of up to kQBatch
    // blocks, then quantizes them.  The first batch is requested before the
    // first weights: loads return in order, so the activation does not wait
    // behind the weight stream.
    float4 v[kQBatch];
    auto load_x = [&](int base) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kQBatch; ++u) {
            const int b = base + WPB * u;
            v[u] = b < nk ? *reinterpret_cast<const float4 *>(x + (int64_t)b * SB + 4 * lane)
                          : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    };
    load_x(wid);
    Buf ring[D];
#pragma unroll
    for (int d = 0; d < D - 1; ++d) load(ring[d], d);  // the weights do not wait for the activation
    Sc cur = {}, nxt = {};
    if constexpr (IB) nxt = load_sc(0);  // (measured: after the first weights is faster here)

    for (int base = wid; base < nk; base += WPB * kQBatch) {
        if (base != wid) load_x(base);  // later batches (wave-uniform)
#pragma unroll
        for (int u = 0; u < kQBatch; ++u) {
            const int b = base + WPB * u;
            if (b >= nk) break;  // wave-uniform
            int q[4], subsum;
            float d;
            rs::quant_block256(v[u], q, d, subsum);
            const int pk = (q[0] & 0xFF) | ((q[1] & 0xFF) << 8) | ((q[2] & 0xFF) << 16) | (q[3] << 24);
            *reinterpret_cast<int *>(xs + b * SB + 4 * lane) = pk;
            if ((lane & 7) == 0) sqs[b * LB + (lane >> 3)] = subsum;
            if (lane == 0) sd[b] = d;
            if (xq_out != nullptr && blockIdx.x == 0) {
                *reinterpret_cast<int *>(xq_out + (int64_t)b * SB + 4 * lane) = pk;
                if (lane == 0) xd_out[b] = d;
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

template <int L, int J, int P, int WPB>
hipError_t launch_cfg(const Q4kArgs &a, int grid, int rows_wg, size_t lds, hipStream_t s, const char **name) {
    constexpr int D = J <= 2 ? QMV_Q4K_D12 : 2;  // (3: TinyLlama W_gate 4.71 -> 4.44 us against 4)
    auto kern = k_q4k<L, J, D, P, WPB>;
    static const std::string kname = variant_name("q4k_l%d_j%d_d%d_p%d_w%d", L, J, D, P, WPB);
    hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WPB), lds, s, a.y, a.wq, a.sc, a.mn, a.d, a.dmin, a.rows, a.K,
                       a.x, a.xq_out, a.xd_out, a.r0, a.r1, rows_wg);
    *name = kname.c_str();
    return hipGetLastError();
}

// 64-lane groups in workgroups of 16 wavefronts (rows of two or more chunks
// per lane, or shared by teams)
template <int P>
hipError_t launch_j(const Q4kArgs &a, int J, int grid, int rows_wg, size_t lds, hipStream_t s, const char **name) {
    switch (J) {
        case 1: return launch_cfg<64, 1, P, 16>(a, grid, rows_wg, lds, s, name);
        case 2: return launch_cfg<64, 2, P, 16>(a, grid, rows_wg, lds, s, name);
        case 3: return launch_cfg<64, 3, P, 16>(a, grid, rows_wg, lds, s, name);
        case 4: return launch_cfg<64, 4, P, 16>(a, grid, rows_wg, lds, s, name);
        case 5: return launch_cfg<64, 5, P, 16>(a, grid, rows_wg, lds, s, name);
        default: return launch_cfg<64, 6, P, 16>(a, grid, rows_wg, lds, s, name);
    }
}

size_t lds_x_bytes(int32_t K) { return ((size_t)K + 4 * (size_t)(K / SB) + 4 * (size_t)(K / SUB) + 15) & ~(size_t)15; }

__global__ void __launch_bounds__(256)
k_quant_b256(int8_t *__restrict__ q, float *__restrict__ d, const float *__restrict__ x, int64_t nblk) {
    // one block per wavefront (as the matvec's activation phase, hence the same bits)
    const int lane = threadIdx.x & 63;
    const int64_t w0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const int64_t nw = ((int64_t)gridDim.x * 256) >> 6;
    for (int64_t b = w0; b < nblk; b += nw) {  // wave-uniform
        const float4 v = *reinterpret_cast<const float4 *>(x + b * SB + 4 * lane);
        int qv[4], subsum;
        float dd;
        rs::quant_block256(v, qv, dd, subsum);
        *reinterpret_cast<int *>(q + b * SB + 4 * lane) =
            (qv[0] & 0xFF) | ((qv[1] & 0xFF) << 8) | ((qv[2] & 0xFF) << 16) | (qv[3] << 24);
        if (lane == 0) d[b] = dd;
    }
}

}  // namespace

size_t q4k_lds_bytes(int32_t K) { return lds_x_bytes(K) + 8192; }

hipError_t launch_q4k(const Q4kArgs &a, int num_cu, hipStream_t s, const char **name) {
    if (a.K % SB != 0 || q4k_lds_bytes(a.K) > 160 * 1024) return hipErrorNotSupported;
#if QMV_GS
    const hipError_t e = launch_gs_q4k(a, num_cu, s, name);  // the split-K form where it takes the shape
    if (e != hipErrorNotSupported) return e;
#endif
    const int chunks = a.K / SUB;
    const int nrow = a.r1 - a.r0;
    const size_t lds_x = lds_x_bytes(a.K);
    const rs::Shape sh = rs::pick_shape(chunks, nrow, num_cu, LB, 6, 32);  // 7 or 8 chunks per lane spill
    const int waves = sh.wgpc * num_cu * sh.wpb;
    if (sh.P == 1) {
        const int groups_per_wg = sh.wpb * (64 / sh.L);
        int grid = (nrow + groups_per_wg - 1) / groups_per_wg;
        if (grid > waves / sh.wpb) grid = waves / sh.wpb;
        if (grid < 1) grid = 1;
        if (sh.L == 16) return launch_cfg<16, 1, 1, 8>(a, grid, 0, lds_x, s, name);
        if (sh.L == 32) return launch_cfg<32, 1, 1, 8>(a, grid, 0, lds_x, s, name);
        if (sh.wpb == 8) return launch_cfg<64, 1, 1, 8>(a, grid, 0, lds_x, s, name);
        return launch_j<1>(a, sh.J, grid, 0, lds_x, s, name);
    }
    int grid = waves / sh.wpb;
    int rows_wg = (nrow + grid - 1) / grid;
    if (rows_wg < 1) rows_wg = 1;
    if (rows_wg * sh.P > 2048) rows_wg = 2048 / sh.P;
    grid = (nrow + rows_wg - 1) / rows_wg;
    if (grid < 1) grid = 1;
    const size_t lds = lds_x + (size_t)rows_wg * sh.P * 4;
    if (sh.P == 2) return launch_j<2>(a, sh.J, grid, rows_wg, lds, s, name);
    if (sh.P == 4) return launch_j<4>(a, sh.J, grid, rows_wg, lds, s, name);
    return launch_j<8>(a, sh.J, grid, rows_wg, lds, s, name);
}

hipError_t launch_quant_b256(int8_t *q, float *d, const float *x, int64_t nblk, hipStream_t s, const char **name) {
    int64_t g = (nblk + 3) / 4;  // 4 blocks per workgroup of 4 wavefronts
    if (g > 4096) g = 4096;
    if (g < 1) g = 1;
    hipLaunchKernelGGL(k_quant_b256, dim3((unsigned)g), dim3(256), 0, s, q, d, x, nblk);
    *name = "quant_q8_b256";
    return hipGetLastError();
}

}  // namespace qmv
