// rowstream.h -- pieces shared by the row-streaming matvecs of the exported
// formats (kernels_zp.hip: 128-element blocks with a zero point;
// kernels_q4k.hip: K-quant super-blocks): buffer descriptors, the Q8_0
// rounding of one element, DPP reductions, and the map from a lane group's
// work items to rows and windows.
//
// The row/window map.  A weight row is a run of 16-byte chunks.  Groups of L
// lanes (L = 16, 32 or 64) read whole rows, lane c of a group taking chunks
// c, c + L, ... in windows of L * J chunks.
//   P = 1: group g of the grid takes rows r0 + g, r0 + g + G, ... (G groups
//   in the grid), each row in W windows, in order.
//   P > 1: workgroup b takes rows_wg consecutive rows; its WPB / P teams of
//   P wavefronts take every (WPB / P)-th of them, and wavefront q of a team
//   takes windows q, q + P, ... of the team's rows.  The P partial sums of a
//   row meet in LDS and are added in wavefront order at the end.
// Every wavefront runs the same number of items; items past a group's rows
// or windows are marked dead (their loads are out of range and read zeros).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef QMV_RS_TAIL  // 1: the last items specialised on their count; 0: whole ring turns, tested per item
#define QMV_RS_TAIL 1
#endif

namespace qmv {
namespace rs {

typedef int v4i __attribute__((ext_vector_type(4)));


constexpr int kOOB = 0x7FFFFFF0;        // an offset beyond every descriptor range used here
constexpr int kBufFlags = 0x00020000;   // buffer descriptor word 3: raw 32-bit data

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
    const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, kBufFlags);
}

// The Q8_0 rounding of one element (Legacy-ISA ML Inference Runtime --
// Design Spec, section 5 rounding bullet): v = x * id, t = v + copysign(0.5,
// x), q = trunc(t), each operation rounded on its own, clamped to +-127.
__device__ __forceinline__ int q8_round(float x, float id) {
#pragma clang fp contract(off)
    float v = x * id;
    float t = v + copysignf(0.5f, x);
    int q = (int)t;
    return min(max(q, -127), 127);
}

template <int CTRL>
__device__ __forceinline__ int dppi(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// DPP controls: swap neighbours, swap pairs, mirror 8 lanes, mirror 16 lanes.
constexpr int kX1 = 0xB1, kX2 = 0x4E, kM8 = 0x141, kM16 = 0x140;

// Integer reduction over each row of 16 lanes by `op` (exact: max or sum),
// the result in every lane of the row.
template <typename F>
__device__ __forceinline__ int row16_reduce(int v, F op) {
    v = op(v, dppi<kX1>(v));
    v = op(v, dppi<kX2>(v));
    v = op(v, dppi<kM8>(v));
    return op(v, dppi<kM16>(v));
}

// The four row values of a wavefront after row16_reduce.
__device__ __forceinline__ void row_values(int v, int &r0, int &r1, int &r2, int &r3) {
    r0 = __builtin_amdgcn_readlane(v, 0);
    r1 = __builtin_amdgcn_readlane(v, 16);
    r2 = __builtin_amdgcn_readlane(v, 32);
    r3 = __builtin_amdgcn_readlane(v, 48);
}

// Sum over an aligned group of L lanes (16, 32 or 64), the same value in
// every lane of the group, in a fixed order: DPP within each 16-lane row
// (after each step the value is uniform over 2, 4, 8, 16 lanes), then the
// rows' values read out and added ((r0 + r1) + (r2 + r3) for L = 64).
template <int L>
__device__ __forceinline__ float group_sum(float v) {
    v = v + dppf<kX1>(v);
    v = v + dppf<kX2>(v);
    v = v + dppf<kM8>(v);
    v = v + dppf<kM16>(v);
    if constexpr (L == 16) return v;
    int a, b, c, d;
    row_values(__float_as_int(v), a, b, c, d);
    const float r0 = __int_as_float(a), r1 = __int_as_float(b), r2 = __int_as_float(c), r3 = __int_as_float(d);
    if constexpr (L == 32) return (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
    return (r0 + r1) + (r2 + r3);
}

// Quantize the 128-element block held by this half-wavefront (lane c of the
// half holds elements 4c .. 4c + 3): amax exact (maximum over the half by
// DPP within rows and lane reads across them; non-negative floats order like
// their bit patterns), d = amax / 127, id = 127 / amax (correctly rounded
// divisions), then the spec's rounding; qsum = the sum of the 128 quants.
__device__ __forceinline__ void quant_half(float4 v, int (&q)[4], float &d, int &qsum) {
    const float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    const auto imax = [](int a, int b) { return max(a, b); };
    const auto isum = [](int a, int b) { return a + b; };
    int r0, r1, r2, r3;
    row_values(row16_reduce(__float_as_int(m), imax), r0, r1, r2, r3);
    const bool hi = (threadIdx.x & 32) != 0;
    const float amax = __int_as_float(hi ? max(r2, r3) : max(r0, r1));
    d = amax / 127.0f;
    const float id = amax != 0.0f ? 127.0f / amax : 0.0f;
    q[0] = q8_round(v.x, id);
    q[1] = q8_round(v.y, id);
    q[2] = q8_round(v.z, id);
    q[3] = q8_round(v.w, id);
    row_values(row16_reduce(q[0] + q[1] + q[2] + q[3], isum), r0, r1, r2, r3);
    qsum = hi ? r2 + r3 : r0 + r1;
}

// Quantize the 256-element block held by this wavefront (lane c holds
// elements 4c .. 4c + 3): amax exact, d = amax / 127, id = 127 / amax, the
// spec's rounding; sub = the sum of the quants of this lane's 32-element
// sub-block (lanes 8j .. 8j + 7), in every lane of it.
__device__ __forceinline__ void quant_block256(float4 v, int (&q)[4], float &d, int &sub) {
    const float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    int r0, r1, r2, r3;
    row_values(row16_reduce(__float_as_int(m), [](int a, int b) { return max(a, b); }), r0, r1, r2, r3);
    const float amax = __int_as_float(max(max(r0, r1), max(r2, r3)));  // non-negative floats order like ints
    d = amax / 127.0f;
    const float id = amax != 0.0f ? 127.0f / amax : 0.0f;
    q[0] = q8_round(v.x, id);
    q[1] = q8_round(v.y, id);
    q[2] = q8_round(v.z, id);
    q[3] = q8_round(v.w, id);
    int s = q[0] + q[1] + q[2] + q[3];
    s += dppi<kX1>(s);
    s += dppi<kX2>(s);
    sub = s + dppi<kM8>(s);
}

// Work item t of a lane group: its row, window, and whether it starts or
// ends the row's accumulation.
struct Item {
    int r, win, li;
    bool live, first, last;
};

template <int L, int P, int WPB>
struct RowMap {
    static constexpr int GPW = 64 / L;         // row groups per wavefront
    static constexpr int TPW = WPB / P;        // teams per workgroup (P > 1)
    int W, r0, g, G, rows_g, rb0, rows_here, rows_team, wpw, tm, pw, items;

    __device__ __forceinline__ RowMap(int chunks, int J, int r0_, int r1, int rows_wg) {
        const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
        W = (chunks + L * J - 1) / (L * J);
        r0 = r0_;
        const int nrow = r1 - r0;
        tm = wid / P;
        pw = wid % P;
        rb0 = r0 + blockIdx.x * rows_wg;
        rows_here = P > 1 ? max(0, min(rows_wg, r1 - rb0)) : 0;
        rows_team = P > 1 ? (rows_here - tm + TPW - 1) / TPW : 0;
        const int rows_team_max = P > 1 ? (rows_wg + TPW - 1) / TPW : 0;  // workgroup-uniform
        wpw = (W + P - 1) / P;
        G = gridDim.x * WPB * GPW;
        const int g0 = (blockIdx.x * WPB + wid) * GPW;
        g = g0 + lane / L;
        rows_g = g < nrow ? (nrow - g + G - 1) / G : 0;
        const int rows_w = g0 < nrow ? (nrow - g0 + G - 1) / G : 0;  // the wavefront's first group has the most
        items = P > 1 ? rows_team_max * wpw : rows_w * W;             // wave-uniform
    }

    __device__ __forceinline__ Item item(int t) const {
        Item it;
        // (W and wpw are wave-uniform; one window per row is the common case
        // of short rows, and skips an integer division per item)
        if constexpr (P == 1) {
            const int rl = W == 1 ? t : t / W;
            it.win = t - rl * W;
            it.live = rl < rows_g;
            it.r = r0 + g + rl * G;
            it.li = 0;
            it.first = it.win == 0;
            it.last = it.win == W - 1;
        } else {
            const int i = wpw == 1 ? t : t / wpw, k = t - i * wpw;
            it.win = pw + P * k;
            it.li = tm + TPW * i;
            it.live = i < rows_team && it.win < W;
            it.r = rb0 + it.li;
            it.first = k == 0;
            it.last = k == wpw - 1;
        }
        return it;
    }
};

// Launch shape for rows of `chunks` chunks: lanes per row L, windows of J
// chunks per lane, teams of P wavefronts, wavefronts per workgroup WPB and
// workgroups per compute unit.
struct Shape {
    int L, J, P, wpb, wgpc;
};

// J chunks per lane per window (at most jmax) for rows split over P
// wavefronts: the windows of a row as even as possible.
inline int pick_j(int chunks, int P, int jmax = 8) {
    const int per = (chunks + P - 1) / P;
    const int win = (per + 64 * jmax - 1) / (64 * jmax);
    return (per + 64 * win - 1) / (64 * win);
}

// min_l: the smallest group allowed (the lanes of one block must fit);
// jmax: the most chunks per lane the kernel holds without spilling;
// team_min: the fewest chunks of a row a wavefront of a team may take (1024
// elements: 64 chunks of 8-bit codes, 32 of 4-bit ones).
inline Shape pick_shape(int chunks, int nrow, int num_cu, int min_l, int jmax, int team_min) {
    Shape s;
    s.L = 64;
    if (chunks <= 16 && min_l <= 16) s.L = 16;
    else if (chunks <= 32 && min_l <= 32) s.L = 32;
    // Rows of one chunk per lane: workgroups of 8 wavefronts (few registers
    // each), 2 per compute unit while that leaves at most 16 rows per
    // wavefront, 4 beyond (more rows in flight; each workgroup quantizes the
    // whole activation, so fewer workgroups spend less on it when the rows
    // are few).  Longer rows: one workgroup of 16 wavefronts per compute unit
    // (more registers per wavefront; the activation is quantized once per
    // compute unit).
    const bool short_rows = s.L < 64 || pick_j(chunks, 1) == 1;
    s.wpb = short_rows ? 8 : 16;
    s.wgpc = short_rows ? ((int64_t)nrow <= 16 * 2 * (int64_t)num_cu * 8 ? 2 : 4) : 1;
    const int waves = s.wgpc * num_cu * s.wpb;
    // rows shared by a team of P wavefronts (at most 8) when there are fewer
    // than two rows per wavefront and each wavefront keeps at least team_min
    // chunks of the row (long rows only)
    s.P = 1;
    if (s.L == 64 && chunks >= 128) {
        while (s.P < 8 && (int64_t)nrow * s.P < 2 * (int64_t)waves && chunks / (2 * s.P) >= team_min) s.P *= 2;
    }
    s.J = s.L == 64 ? pick_j(chunks, s.P, jmax) : 1;
    return s;
}

}  // namespace rs
}  // namespace qmv
