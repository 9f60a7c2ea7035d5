// device_common.h -- device helpers shared by the libqmv kernels (gfx950).
//
// Quantization rule: Legacy-ISA ML Inference Runtime -- Design Spec,
// section 4 ("Q8 quantization": d = max|x| / 127, all-zero block -> d = 0)
// and section 5 (rounding bullet: q = trunc(x * id + copysign(0.5, x)),
// id = 127 / amax, no floating-point contraction).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmv {

constexpr int QK = 32;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// One element: v = x * id, t = v + copysign(0.5, x), q = trunc(t), each
// float operation rounded on its own (contraction off in this scope), then
// clamped to [lo, hi].  fp32 division elsewhere is the IEEE correctly
// rounded sequence (hipcc default), never a reciprocal approximation.
__device__ __forceinline__ int quant_round(float x, float id, int lo, int hi) {
#pragma clang fp contract(off)
    float v = x * id;
    float t = v + copysignf(0.5f, x);
    int q = (int)t;  // float -> int conversion truncates toward zero
    return min(max(q, lo), hi);
}

// Cross-lane moves within an aligned group of 8 lanes, one DPP instruction
// each: swap neighbours (quad_perm [1,0,3,2]), swap pairs (quad_perm
// [2,3,0,1]), and mirror the 8 lanes (row_half_mirror, lane i <-> 7 - i).
// After the two quad steps every lane of a quad holds the quad's value, so
// the mirror step combines the two quads of the group.
__device__ __forceinline__ int dpp_xor1(int v) { return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_xor2(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_mirror8(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false); }
// row_shl:4 -- lane i receives lane i + 4 (within a row of 16 lanes).
__device__ __forceinline__ int dpp_down4(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0xF, false); }

__device__ __forceinline__ float group8_max(float a) {
    a = fmaxf(a, __int_as_float(dpp_xor1(__float_as_int(a))));
    a = fmaxf(a, __int_as_float(dpp_xor2(__float_as_int(a))));
    a = fmaxf(a, __int_as_float(dpp_mirror8(__float_as_int(a))));
    return a;
}

__device__ __forceinline__ int group8_sum(int s) {
    s += dpp_xor1(s);
    s += dpp_xor2(s);
    s += dpp_mirror8(s);
    return s;
}

// Largest |x| of a 32-element block spread over an aligned group of 8 lanes,
// 4 elements per lane (lane c of the group holds elements 4c..4c+3).  All 8
// lanes of the group must be active.  The maximum is exact, so its
// evaluation order does not matter.
__device__ __forceinline__ float block_amax8(float4 v) {
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    return group8_max(a);
}

__device__ __forceinline__ int pack4(int a, int b, int c, int d) {
    return (a & 0xFF) | ((b & 0xFF) << 8) | ((c & 0xFF) << 16) | ((unsigned)(d & 0xFF) << 24);
}

// Q8_0 quantization of one block held by an aligned group of 8 lanes.
// Returns this lane's 4 quants packed little-endian (element 4c in the low
// byte); d receives the block scale and qsum the sum of the block's 32
// quants (both identical in all 8 lanes).
__device__ __forceinline__ int quant_q8_group8(float4 v, float &d, int &qsum) {
    float amax = block_amax8(v);
    d = amax / 127.0f;
    float id = (amax != 0.0f) ? 127.0f / amax : 0.0f;
    int q0 = quant_round(v.x, id, -127, 127);
    int q1 = quant_round(v.y, id, -127, 127);
    int q2 = quant_round(v.z, id, -127, 127);
    int q3 = quant_round(v.w, id, -127, 127);
    qsum = group8_sum(q0 + q1 + q2 + q3);
    return pack4(q0, q1, q2, q3);
}

// Q8_0 quantization of one whole 32-element block held by one lane (the
// same arithmetic as quant_q8_group8, hence the same bits): the 32 quants
// are returned packed little-endian in lo (elements 0..15) and hi
// (elements 16..31), with the block scale d and the sum of the quants.
__device__ __forceinline__ void quant_q8_lane(const float4 (&v)[8], v4i &lo, v4i &hi, float &d, int &qsum) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    d = amax / 127.0f;
    const float id = (amax != 0.0f) ? 127.0f / amax : 0.0f;
    int w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        w[i] = pack4(quant_round(v[i].x, id, -127, 127), quant_round(v[i].y, id, -127, 127),
                     quant_round(v[i].z, id, -127, 127), quant_round(v[i].w, id, -127, 127));
    lo = (v4i){w[0], w[1], w[2], w[3]};
    hi = (v4i){w[4], w[5], w[6], w[7]};
    int s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = __builtin_amdgcn_sdot4(w[i], 0x01010101, s, false);
    qsum = s;
}

// Q8_0 quantization of one block held by an aligned group of 4 lanes, 8
// elements per lane (lane c of the group holds elements 8c..8c+7 in a and
// b).  The same arithmetic as quant_q8_group8 (the block maximum is exact
// and the two divisions and the per-element rounding are the same
// operations), hence the same bits, with half the lanes repeating the
// divisions.  Returns this lane's 8 quants packed little-endian in an int2;
// d receives the block scale and qsum the sum of the block's 32 quants (both
// identical in the 4 lanes).
__device__ __forceinline__ int2 quant_q8_group4(float4 a, float4 b, float &d, int &qsum) {
    float amax = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                       fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
    amax = fmaxf(amax, __int_as_float(dpp_xor1(__float_as_int(amax))));
    amax = fmaxf(amax, __int_as_float(dpp_xor2(__float_as_int(amax))));
    d = amax / 127.0f;
    const float id = (amax != 0.0f) ? 127.0f / amax : 0.0f;
    const int w0 = pack4(quant_round(a.x, id, -127, 127), quant_round(a.y, id, -127, 127),
                         quant_round(a.z, id, -127, 127), quant_round(a.w, id, -127, 127));
    const int w1 = pack4(quant_round(b.x, id, -127, 127), quant_round(b.y, id, -127, 127),
                         quant_round(b.z, id, -127, 127), quant_round(b.w, id, -127, 127));
    int s = __builtin_amdgcn_sdot4(w0, 0x01010101, __builtin_amdgcn_sdot4(w1, 0x01010101, 0, false), false);
    s += dpp_xor1(s);
    s += dpp_xor2(s);
    qsum = s;
    return make_int2(w0, w1);
}

// Q4_0 weight quantization of one block held by an aligned group of 8
// lanes: d = amax / 7, value = clamp(trunc(x * (7 / amax) + copysign(0.5,
// x)), -8, 7), nibble = value + 8.  Returns this lane's 4 nibbles, one per
// byte (element 4c in the low byte).
__device__ __forceinline__ int quant_q4_group8(float4 v, float &d) {
    float amax = block_amax8(v);
    d = amax / 7.0f;
    float id = (amax != 0.0f) ? 7.0f / amax : 0.0f;
    int n0 = quant_round(v.x, id, -8, 7) + 8;
    int n1 = quant_round(v.y, id, -8, 7) + 8;
    int n2 = quant_round(v.z, id, -8, 7) + 8;
    int n3 = quant_round(v.w, id, -8, 7) + 8;
    return pack4(n0, n1, n2, n3);
}

// Activation forms of the products: Q8_0 rows as given, a float32 row
// quantized in the kernel, a float32 row normalized (rmsnorm) and then
// quantized, or the FFN gate silu(g) * u of two float32 rows, then quantized.
enum { kActQ8 = 0, kActF32 = 1, kActRms = 2, kActSilu = 3 };

// ---- the decode-step neighbours of the product (Legacy-ISA ML Inference
// Runtime -- Design Spec, section 5 kernel list: ml_k_rmsnorm,
// ml_k_silu_mul; section 6 forward pass), shared by the fused activation
// forms and the standalone kernels so that both give the same bits.

// The rmsnorm scale 1 / sqrt(ss / n + eps), each operation rounded on its
// own (contraction off; the division and the square root are the correctly
// rounded ones).
__device__ __forceinline__ float rms_inv(float ss, int n, float eps) {
#pragma clang fp contract(off)
    const float mean = ss / (float)n;
    return 1.0f / sqrtf(mean + eps);
}

// w * (inv * x), two roundings.
__device__ __forceinline__ float rms_apply(float x, float w, float inv) {
#pragma clang fp contract(off)
    const float t = inv * x;
    return w * t;
}

// exp(-g) to a few ulp (the spec bounds silu's exp at 1e-6 relative) in six
// instructions: 2^t with t = -g log2(e).  The product is rounded (t_hi) and
// its rounding error recovered exactly by an FMA, the low part of log2(e)
// added to that residual r, and 2^t = 2^t_hi (v_exp_f32, 1 ulp) * (1 + r ln 2)
// with |r| < 2^-17, so the neglected (r ln 2)^2 / 2 stays below 1e-11.
// t >= 128 overflows to +inf as exp does.
__device__ __forceinline__ float exp_neg(float g) {
    const float x = -g;
    const float t = x * 1.44269502f;                     // log2(e), rounded
    float r = __builtin_fmaf(x, 1.44269502f, -t);        // x log2e_hi - t, exact
    r = __builtin_fmaf(x, 1.92596303e-8f, r);            // + x (log2(e) - log2e_hi)
    const float e = __builtin_amdgcn_exp2f(t);
    return t < 128.0f ? __builtin_fmaf(e, r * 0.693147182f, e) : e;
}

// silu(g) * u as g * (1 / (1 + exp(-g))) * u: the exp above and the
// hardware reciprocal (1 ulp), well within the spec's 1e-6; each other
// operation rounded on its own.
__device__ __forceinline__ float silu_mul1(float g, float u) {
#pragma clang fp contract(off)
    const float s = __builtin_amdgcn_rcpf(1.0f + exp_neg(g));
    const float v = g * s;
    return v * u;
}

// Pairwise (recursive-halving) sum of the squares of 8 consecutive values.
__device__ __forceinline__ float sumsq8(float4 a, float4 b) {
#pragma clang fp contract(off)
    const float s0 = a.x * a.x, s1 = a.y * a.y, s2 = a.z * a.z, s3 = a.w * a.w;
    const float s4 = b.x * b.x, s5 = b.y * b.y, s6 = b.z * b.z, s7 = b.w * b.w;
    return ((s0 + s1) + (s2 + s3)) + ((s4 + s5) + (s6 + s7));
}

// The sum of a 32-element block's squares from its four 8-element pairwise
// sums (consecutive elements), pairwise.
__device__ __forceinline__ float block_sumsq(const float (&q)[4]) {
#pragma clang fp contract(off)
    return (q[0] + q[1]) + (q[2] + q[3]);
}

// a + b rounded once (never fused with a neighbouring product).
__device__ __forceinline__ float pair_add(float a, float b) {
#pragma clang fp contract(off)
    return a + b;
}

// v_dot4_i32_i8: c + sum of the four signed byte products of a and b.
__device__ __forceinline__ int dot4(int a, int b, int c) {
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

// Transposing wave reduction of NV per-lane partial sums (NV a power of two,
// at most 64).  At each butterfly step with lane offset o, a lane keeps half
// of its values (the upper half if bit o of its lane id is set), sends the
// other half to lane ^ o and adds what it receives; once one value is left
// the remaining steps are plain butterfly sums.  On return every lane holds
// the wave-wide total of value index reduce_index<NV>(lane).
template <int NV>
__device__ __forceinline__ float wave_reduce_transpose(float (&a)[NV]) {
    static_assert(NV >= 1 && NV <= 64 && (NV & (NV - 1)) == 0, "NV must be a power of two <= 64");
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int s = 0; s < 6; ++s) {
        const int o = 32 >> s;
        const int n = NV >> s;  // values still held
        if (n > 1) {
            const bool up = (lane & o) != 0;
#pragma unroll
            for (int i = 0; i < n / 2; ++i) {
                float lo = a[i], hi = a[i + n / 2];
                // opaque to the optimizer: otherwise the selects below are
                // folded into one load from a lane-dependent address, which
                // would push the whole array out of registers into scratch
                asm volatile("" : "+v"(lo), "+v"(hi));
                float keep = up ? hi : lo;
                float send = up ? lo : hi;
                a[i] = keep + __shfl_xor(send, o);
            }
        } else {
            a[0] += __shfl_xor(a[0], o);
        }
    }
    return a[0];
}

// Value index whose total wave_reduce_transpose<NV> leaves in `lane`.
template <int NV>
__device__ __forceinline__ int reduce_index(int lane) {
    int idx = 0;
#pragma unroll
    for (int s = 0; (NV >> (s + 1)) >= 1; ++s)
        idx += ((lane >> (5 - s)) & 1) * (NV >> (s + 1));
    return idx;
}

// Lanes that hold a distinct total after wave_reduce_transpose<NV>: those
// whose lane-id bits below the top log2(NV) bits are zero.
template <int NV>
__device__ __forceinline__ bool reduce_owner(int lane) {
    return (lane & ((64 / NV) - 1)) == 0;
}

}  // namespace qmv
