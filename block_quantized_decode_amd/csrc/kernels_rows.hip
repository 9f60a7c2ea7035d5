// kernels_rows.hip -- weight-streaming products for a few activation rows
// (M = 1 .. 8) on gfx950: the decode matvec and the small-batch product.
//
// What is computed (Legacy-ISA ML Inference Runtime -- Design Spec,
// section 4 "Integer dot per block" and section 5 kernel interface):
//   y[m, r] = sum over blocks b of sumi(m, r, b) * dw(r, b) * dx(m, b),
//   sumi = exact int32 dot of the 32 weight and activation quants,
// for r in [r0, r1).  The spec's CPU kernels take 4 rows at a time so that
// one activation-block load serves 4 weight rows; here a wavefront takes 4
// rows at a time (or 2 or 1 for matrices with few rows) and each of its 64
// lanes owns block columns l, l + 64, l + 128, ... of them.
//
// How the work is laid out on the chip:
//   * one wavefront per unit of R rows (R = 4, 2 or 1, picked so that every
//     CU gets 8 - 16 wavefronts), and the grid covers all units: every
//     weight byte a wavefront needs (its rows, whole length, up to 8 column
//     groups = K 16384) is requested at once, so the memory system sees the
//     whole matrix at the start and streams it at full rate; a CU holds its
//     ~1/256 share of a 28 MB matrix in registers with room to spare;
//   * weights are read with raw buffer loads: base and byte range live in a
//     wave-uniform descriptor covering only the rows below r1, so rows past
//     r1 and blocks past the row end read zeros without touching memory,
//     and no load sits under a branch;
//   * the activation is brought into LDS first, with direct-to-LDS buffer
//     loads (1 KiB of contiguous float32 per wavefront instruction, no
//     registers), so its requests go out ahead of the weight stream;
//   * the workgroup then quantizes it in LDS (FX: Q8_0, one lane per
//     32-element block, reading the block in a lane-rotated chunk order
//     that avoids LDS bank conflicts) into two 16-byte halves
//     per block plus dx and 8 * sum(q) per block; pre-quantized activations
//     are copied the same way and only their quant sums are formed;
//   * int8 block dots use v_dot4_i32_i8.  Q4_0 nibbles are used as unsigned
//     bytes 0..15 (gfx950 has no mixed-sign dot4) and the -8 offset is
//     folded in exactly: sumi = dot(nibble, qx) - 8 * sum(qx);
//   * per lane, block sums are scaled and accumulated in fp32; the R * M
//     partial sums of the unit are reduced across the wavefront with a
//     transposing butterfly and stored by one lane each.
#include "device_common.h"
#include "launch.h"


namespace qmv {
namespace {

constexpr int kBufFlags = 0x00020000;  // buffer descriptor word 3, gfx9-family raw buffers
constexpr int kNT = 2;                 // cache policy: non-temporal (weights are streamed once)
constexpr int kOOB = 0x40000000;       // an offset beyond every descriptor range used here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, kBufFlags);
}

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS: lane i of the
// wavefront lands at lds + 16 i (the instruction is issued by the whole
// wavefront; lds must be wave-uniform).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, void *lds, int voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voffset, 0, 0, 0);
}

// 4 bytes per lane from global memory straight into LDS (lane i at lds + 4 i).
__device__ __forceinline__ void load_lds4(__amdgpu_buffer_rsrc_t r, void *lds, int voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 4, voffset, 0, 0, 0);
}

template <int QT, int J, int R>
struct WTile {
    static constexpr int QW = (QT == 8) ? 2 : 1;  // 16-byte words per block
    v4i w[J][R][QW];
    float dw[J][R];
};

// All weight loads of one unit chunk: rows rb .. rb+R-1 (those below r1),
// block columns j0 .. j0+J-1 (lane l takes block l + 64 j).
template <int QT, int J, int R>
__device__ __forceinline__ void load_tile(WTile<QT, J, R> &t, const int8_t *__restrict__ wq,
                                          const float *__restrict__ wd, int nb, int rb, int r1, int j0,
                                          int lane) {
    constexpr int QB = (QT == 8) ? 32 : 16;  // quant bytes per block
    const int rows_here = max(0, min(R, r1 - rb));
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(wq + (size_t)rb * nb * QB, rows_here * nb * QB);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(wd + (size_t)rb * nb, rows_here * nb * 4);
#pragma unroll
    for (int u = 0; u < J; ++u) {
        const int b = lane + 64 * (j0 + u);
        const int oq = b < nb ? b * QB : kOOB;
        const int od = b < nb ? b * 4 : kOOB;
        // the row offset goes into the per-lane offset, which the hardware
        // range-checks (the scalar offset field is not): rows past r1 read
        // zeros
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int rq_off = oq + r * nb * QB, rd_off = od + r * nb * 4;
            t.w[u][r][0] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rq, rq_off, 0, kNT));
            if constexpr (QT == 8)
                t.w[u][r][1] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rq, rq_off + 16, 0, kNT));
            t.dw[u][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, rd_off, 0, kNT));
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

// LDS layout for M activation rows of nb blocks each:
//   xlo [M*nb] 16 B  quants 0..15 of each block
//   xhi [M*nb] 16 B  quants 16..31
//   xdx [M*nb] 4 B   block scale dx
//   xsx [M*nb] 4 B   8 * sum of the block's quants (for the Q4_0 offset)
//   raw [M*K]  4 B   float32 activation as loaded (FX only), rounded up to
//                    whole 1 KiB chunks
// (the pre-quantized arrays are rounded up to whole 64-block chunks, the
// granularity of their direct loads).
__host__ __device__ constexpr size_t lds_bytes(int M, int K, bool fx, bool rms = false) {
    return (size_t)((M * (K / 32) + 63) / 64 * 64) * 40 + (fx ? ((size_t)M * K * 4 + 1023) / 1024 * 1024 : 0) +
           (rms ? (size_t)next_pow2(K / 32) * 4 : 0);
}

template <int QT, int M, int AX, int J, int R, int WPB>
__global__ void __launch_bounds__(64 * WPB)
k_rows(float *__restrict__ y, const int8_t *__restrict__ wq, const float *__restrict__ wd,
       int32_t rows, int32_t K, const float *__restrict__ x, const int8_t *__restrict__ xq,
       const float *__restrict__ xd, const float *__restrict__ xn, float eps, int8_t *__restrict__ xq_out,
       float *__restrict__ xd_out, int32_t r0, int32_t r1) {
    constexpr bool FX = AX != kActQ8;
    static_assert(AX <= kActF32 || M == 1, "the neighbour forms take one float32 activation row");
    constexpr int NV = next_pow2(R * M);
    extern __shared__ __align__(16) unsigned char smem[];
    const int nb = K >> 5;
    const int nblk = M * nb;               // activation blocks
    const int nblk64 = (nblk + 63) / 64 * 64;
    v4i *xlo = reinterpret_cast<v4i *>(smem);
    v4i *xhi = xlo + nblk64;
    float *xdx = reinterpret_cast<float *>(xhi + nblk64);
    int *xsx = reinterpret_cast<int *>(xdx + nblk64);
    float *raw = reinterpret_cast<float *>(xsx + nblk64);
    // rmsnorm: the block sums of squares, padded to a power of two, after raw
    float *bs = raw + (M * K + 255) / 256 * 256;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave within the workgroup
    const int unit = blockIdx.x * WPB + wid;                    // this wavefront's R rows
    const int nunits = (r1 - r0 + R - 1) / R;
    const bool busy = unit < nunits;
    const int rb = r0 + R * unit;
    const int nchunk = (nb + 64 * J - 1) / (64 * J);  // column chunks per row

    // 1. activation into LDS: direct loads, issued before any weight load
    if constexpr (FX) {
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, M * K * 4);
        const int nkb = (M * K * 4 + 1023) >> 10;  // 1 KiB chunks; the tail of the last reads zeros
        for (int c = wid; c < nkb; c += WPB) load_lds16(rx, raw + 256 * c, 1024 * c + 16 * lane);
    } else {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(xq, M * K);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(xd, M * nb * 4);
        for (int c = wid; c < nblk64 / 64; c += WPB) {  // 64 blocks per instruction
            const int b = 64 * c + lane;
            const int o = b < nblk ? 32 * b : kOOB;
            load_lds16(rq, xlo + 64 * c, o);
            load_lds16(rq, xhi + 64 * c, o + 16);
            load_lds4(rd, xdx + 64 * c, b < nblk ? 4 * b : kOOB);
        }
    }

    // 2. this unit's weights (first column chunk), all of it in flight at
    //    once; an idle wavefront's descriptor has an empty range
    WTile<QT, J, R> t;
    load_tile<QT, J, R>(t, wq, wd, nb, rb, busy ? r1 : rb, 0, lane);
    __builtin_amdgcn_sched_barrier(0);

    // 3. once the activation has landed, quantize / sum it in LDS
    __syncthreads();
    if constexpr (FX) {
        float inv = 0.0f;
        if constexpr (AX == kActRms) {
            // rmsnorm: each block's squares summed pairwise (8-element sums,
            // then pairs of those), then the block sums pairwise over their
            // count padded to a power of two (an in-LDS tree adding
            // neighbours at every level) -- the order of the fused split-K
            // form and of the standalone kernel, hence the same bits
            int P = 1;
            while (P < nb) P *= 2;
            for (int b = tid; b < P; b += 64 * WPB) {
                float s = 0.0f;
                if (b < nb) {
                    const float4 *src = reinterpret_cast<const float4 *>(raw + 32 * b);
                    float q[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) q[k] = sumsq8(src[2 * k], src[2 * k + 1]);
                    s = block_sumsq(q);
                }
                bs[b] = s;
            }
            for (int h = 1; h < P; h *= 2) {
                __syncthreads();
                for (int i = tid; i < P / (2 * h); i += 64 * WPB) bs[2 * h * i] = pair_add(bs[2 * h * i], bs[2 * h * i + h]);
            }
            __syncthreads();
            inv = rms_inv(bs[0], K, eps);
        }
        // one lane per 32-element block: the two divisions once per block,
        // no cross-lane steps.  Lane b reads its block's eight 16-byte
        // chunks in the rotated order (k + b) mod 8, which keeps the 64
        // lanes' LDS reads at most 2-way bank conflicted; every chunk's 4
        // quants are written back to their own place in the block, so the
        // order of the reads changes nothing in the result.
        for (int blk = tid; blk < nblk; blk += 64 * WPB) {
            const int rot = blk & 7;
            const float4 *src = reinterpret_cast<const float4 *>(raw + 32 * blk);
            float4 v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = src[(k + rot) & 7];
            if constexpr (AX == kActRms || AX == kActSilu) {
                // the norm weights (rmsnorm) or u (gate) of the same elements
                const float4 *nsrc = reinterpret_cast<const float4 *>(xn + 32 * (size_t)blk);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float4 nv = nsrc[(k + rot) & 7];
                    if constexpr (AX == kActRms)
                        v[k] = make_float4(rms_apply(v[k].x, nv.x, inv), rms_apply(v[k].y, nv.y, inv),
                                           rms_apply(v[k].z, nv.z, inv), rms_apply(v[k].w, nv.w, inv));
                    else
                        v[k] = make_float4(silu_mul1(v[k].x, nv.x), silu_mul1(v[k].y, nv.y), silu_mul1(v[k].z, nv.z),
                                           silu_mul1(v[k].w, nv.w));
                }
            }
            float amax = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k)
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[k].x), fabsf(v[k].y)), fmaxf(fabsf(v[k].z), fabsf(v[k].w))));
            const float d = amax / 127.0f;
            const float id = (amax != 0.0f) ? 127.0f / amax : 0.0f;
            int sum = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int c = (k + rot) & 7;  // chunk held in v[k]
                const int pk = pack4(quant_round(v[k].x, id, -127, 127), quant_round(v[k].y, id, -127, 127),
                                     quant_round(v[k].z, id, -127, 127), quant_round(v[k].w, id, -127, 127));
                reinterpret_cast<int *>((c < 4) ? (xlo + blk) : (xhi + blk))[c & 3] = pk;
                sum = dot4(pk, 0x01010101, sum);
            }
            xdx[blk] = d;
            xsx[blk] = 8 * sum;
        }
    } else {
        for (int e = tid; e < nblk * 2; e += 64 * WPB) {  // 2 lanes per block
            const int blk = e >> 1, h = e & 1;
            const v4i v = h ? xhi[blk] : xlo[blk];
            int s = dot4(v.x, 0x01010101, dot4(v.y, 0x01010101, dot4(v.z, 0x01010101, dot4(v.w, 0x01010101, 0))));
            s += dpp_xor1(s);
            if (h == 0) xsx[blk] = 8 * s;
        }
    }
    __syncthreads();
    if (FX && xq_out != nullptr && blockIdx.x == 0) {  // optional copy of the quantized activation
        for (int blk = tid; blk < nblk; blk += 64 * WPB) {
            const int m = blk / nb, b = blk - m * nb;
            v4i *dst = reinterpret_cast<v4i *>(xq_out + (size_t)m * K + (size_t)b * QK);
            dst[0] = xlo[blk];
            dst[1] = xhi[blk];
            xd_out[(size_t)m * nb + b] = xdx[blk];
        }
    }
    if (!busy) return;  // no barrier follows

    // 4. block dots, scales, fp32 accumulation
    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.0f;
    for (int ch = 0; ch < nchunk; ++ch) {
        if (ch > 0) load_tile<QT, J, R>(t, wq, wd, nb, rb, r1, ch * J, lane);  // K beyond 2048 J only
#pragma unroll
        for (int u = 0; u < J; ++u) {
            const int b = lane + 64 * (ch * J + u);
            const bool ok = b < nb;
            const int bb = ok ? b : nb - 1;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const v4i xl = xlo[m * nb + bb];
                const v4i xh = xhi[m * nb + bb];
                const float dx = ok ? xdx[m * nb + bb] : 0.0f;
                const int sx8 = xsx[m * nb + bb];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int s = block_dot<QT>(t.w[u][r], xl, xh, sx8);
                    acc[m * R + r] = fmaf((float)s, t.dw[u][r] * dx, acc[m * R + r]);
                }
            }
        }
    }

    // 5. reduce the R*M partial sums over the wavefront and store
    const float tot = wave_reduce_transpose<NV>(acc);
    const int idx = reduce_index<NV>(lane);
    const int m = idx / R, r = idx % R;
    const int row = rb + r;
    if (reduce_owner<NV>(lane) && m < M && row < r1) y[(size_t)m * rows + row] = tot;
}

template <int QT, int M, int AX, int J, int R, int WPB>
hipError_t launch_rows_t(const RowsArgs &a, hipStream_t s, const char **name) {
    static const std::string kname =
        variant_name("rows_q%d_m%d%s_j%d_r%d_w%d", QT, M,
                     AX == kActQ8 ? "" : AX == kActF32 ? "_fx" : AX == kActRms ? "_fxn" : "_fxs", J, R, WPB);
    auto kern = k_rows<QT, M, AX, J, R, WPB>;
    const size_t lds = lds_bytes(M, a.K, AX != kActQ8, AX == kActRms);
    hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), lds);
    if (e != hipSuccess) return e;
    const int nunits = (a.r1 - a.r0 + R - 1) / R;
    const int grid = (nunits + WPB - 1) / WPB;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WPB), lds, s, a.y, a.wq, a.wd, a.rows, a.K, a.x, a.xq,
                       a.xd, AX == kActSilu ? a.xu : a.xn, a.eps, a.xq_out, a.xd_out, a.r0, a.r1);
    *name = kname.c_str();
    return hipGetLastError();
}

// Column groups held per lane at once: the whole row when it fits
// (K <= 2048 J), else chunks of J.  J is capped so that the weight
// registers plus the R * M accumulators stay within the 256-VGPR file
// without spilling: Q4_0 8 / 6 / 2 and Q8_0 4 / 2 column groups for
// M <= 2 / M <= 4 / larger M.
template <int QT, int M>
constexpr int jmax() {
    return QT == 4 ? (M <= 2 ? 8 : (M <= 4 ? 6 : 2)) : (M <= 4 ? 4 : 2);
}

// Rows per wavefront R and wavefronts per workgroup (16 / R): 4 rows per
// wavefront when that still gives every CU at least 8 wavefronts,
// otherwise 2 or 1, so that a matrix with few rows (4096 x 11008) still
// spreads over 8 - 16 wavefronts per CU and each workgroup's activation
// quantization is shared by that many wavefronts.  Several activation rows
// always use R = 4.
template <int QT, int M, int AX, int J>
hipError_t launch_rows_r(const RowsArgs &a, hipStream_t s, const char **name) {
    constexpr int JJ = J < jmax<QT, M>() ? J : jmax<QT, M>();
    if constexpr (M > 1) {
        return launch_rows_t<QT, M, AX, JJ, 4, 4>(a, s, name);
    } else {
        const int nrows = a.r1 - a.r0;
        const int per_cu = 8 * a.num_cu;
        if (nrows / 4 >= per_cu) return launch_rows_t<QT, M, AX, JJ, 4, 4>(a, s, name);
        if (nrows / 2 >= per_cu) return launch_rows_t<QT, M, AX, JJ, 2, 8>(a, s, name);
        return launch_rows_t<QT, M, AX, JJ, 1, 16>(a, s, name);
    }
}

template <int QT, int M, int AX>
hipError_t launch_rows_j(const RowsArgs &a, hipStream_t s, const char **name) {
    const int nj = (a.K / QK + 63) / 64;
    if (nj <= 1) return launch_rows_r<QT, M, AX, 1>(a, s, name);
    if (nj <= 2) return launch_rows_r<QT, M, AX, 2>(a, s, name);
    if (nj <= 3) return launch_rows_r<QT, M, AX, 3>(a, s, name);
    if (nj <= 4) return launch_rows_r<QT, M, AX, 4>(a, s, name);
    if (nj <= 6) return launch_rows_r<QT, M, AX, 6>(a, s, name);
    return launch_rows_r<QT, M, AX, 8>(a, s, name);
}

template <int QT>
hipError_t launch_rows_q(const RowsArgs &a, hipStream_t s, const char **name) {
    if (a.x != nullptr) {
        if (a.xu != nullptr) return launch_rows_j<QT, 1, kActSilu>(a, s, name);
        if (a.xn != nullptr) return launch_rows_j<QT, 1, kActRms>(a, s, name);
        return launch_rows_j<QT, 1, kActF32>(a, s, name);
    }
    switch (a.M) {
        case 1: return launch_rows_j<QT, 1, kActQ8>(a, s, name);
        case 2: return launch_rows_j<QT, 2, kActQ8>(a, s, name);
        case 3: return launch_rows_j<QT, 3, kActQ8>(a, s, name);
        case 4: return launch_rows_j<QT, 4, kActQ8>(a, s, name);
        case 5: return launch_rows_j<QT, 5, kActQ8>(a, s, name);
        case 6: return launch_rows_j<QT, 6, kActQ8>(a, s, name);
        case 7: return launch_rows_j<QT, 7, kActQ8>(a, s, name);
        case 8: return launch_rows_j<QT, 8, kActQ8>(a, s, name);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t rows_lds_bytes(int M, int K, bool fx, bool rms) { return lds_bytes(M, K, fx, rms); }

hipError_t launch_rows(const RowsArgs &a, hipStream_t s, const char **name) {
    return a.qtype == 4 ? launch_rows_q<4>(a, s, name) : launch_rows_q<8>(a, s, name);
}

}  // namespace qmv
