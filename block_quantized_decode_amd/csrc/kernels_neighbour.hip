// kernels_neighbour.hip -- the two decode-step neighbours of the product as
// launches of their own (Legacy-ISA ML Inference Runtime -- Design Spec,
// section 5 kernel list: ml_k_rmsnorm(o, x, w, n, eps) and
// ml_k_silu_mul(g, u, n); section 6 forward pass: rmsnorm ahead of every
// quantization of a layer input, silu_mul ahead of the FFN down
// projection).  The fused activation forms of the product evaluate the same
// device functions in the same order, so a standalone step followed by the
// plain fused product gives the same bits as the fused launch.
#include "device_common.h"
#include "launch.h"

namespace qmv {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

// One workgroup of 1024 threads.  ss: the squares of each 32-element block
// summed pairwise (recursive halving: 8-element sums of consecutive
// elements, then pairs of those), the block sums summed pairwise over their
// count padded to a power of two with zeros (an in-LDS tree that adds
// neighbours at every level, the same association as recursive halving);
// then o_j = w_j * (inv * x_j), inv = 1 / sqrt(ss / n + eps), each operation
// rounded on its own.  o may be x: every read of x precedes the barrier
// ahead of the writes, and each element is then read and written by the
// same thread.
__global__ void __launch_bounds__(1024) k_rmsnorm(float *o, const float *x, const float *__restrict__ w, int32_t n,
                                                  int32_t p, float eps) {
#pragma clang fp contract(off)
    extern __shared__ float bs[];  // p block sums
    const int nb = n >> 5;
    for (int b = threadIdx.x; b < p; b += 1024) {
        float s = 0.0f;
        if (b < nb) {
            const float4 *src = reinterpret_cast<const float4 *>(x + 32 * (size_t)b);
            float q[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) q[k] = sumsq8(src[2 * k], src[2 * k + 1]);
            s = (q[0] + q[1]) + (q[2] + q[3]);
        }
        bs[b] = s;
    }
    for (int h = 1; h < p; h *= 2) {
        __syncthreads();
        for (int i = threadIdx.x; i < p / (2 * h); i += 1024) bs[2 * h * i] = bs[2 * h * i] + bs[2 * h * i + h];
    }
    __syncthreads();
    const float inv = rms_inv(bs[0], n, eps);
    for (int j = threadIdx.x; j < (n >> 2); j += 1024) {
        const float4 v = reinterpret_cast<const float4 *>(x)[j];
        const float4 g = reinterpret_cast<const float4 *>(w)[j];
        reinterpret_cast<float4 *>(o)[j] =
            make_float4(rms_apply(v.x, g.x, inv), rms_apply(v.y, g.y, inv), rms_apply(v.z, g.z, inv),
                        rms_apply(v.w, g.w, inv));
    }
}

// o_j = silu(g_j) * u_j elementwise (V4: 4 per thread where the tail
// allows, for 16-byte aligned o, g, u).
template <bool V4>
__global__ void __launch_bounds__(256) k_silu_mul(float *o, const float *g, const float *u, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t n4 = V4 ? n >> 2 : 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        const float4 a = reinterpret_cast<const float4 *>(g)[i];
        const float4 b = reinterpret_cast<const float4 *>(u)[i];
        reinterpret_cast<float4 *>(o)[i] =
            make_float4(silu_mul1(a.x, b.x), silu_mul1(a.y, b.y), silu_mul1(a.z, b.z), silu_mul1(a.w, b.w));
    }
    for (int64_t j = 4 * n4 + (int64_t)blockIdx.x * 256 + threadIdx.x; j < n; j += stride) o[j] = silu_mul1(g[j], u[j]);
}

}  // namespace

hipError_t launch_rmsnorm(float *o, const float *x, const float *w, int32_t n, float eps, hipStream_t s,
                          const char **name) {
    int32_t p = 1;
    while (p < n / 32) p *= 2;
    hipLaunchKernelGGL(k_rmsnorm, dim3(1), dim3(1024), (size_t)p * 4, s, o, x, w, n, p, eps);
    *name = "rmsnorm";
    return hipGetLastError();
}

hipError_t launch_silu_mul(float *o, const float *g, const float *u, int64_t n, hipStream_t s, const char **name) {
    const bool v4 = ((reinterpret_cast<uintptr_t>(o) | reinterpret_cast<uintptr_t>(g) |
                      reinterpret_cast<uintptr_t>(u)) & 15) == 0;
    int64_t grid = ((v4 ? n >> 2 : n) + 255) / 256;
    if (grid > 2048) grid = 2048;
    if (grid < 1) grid = 1;
    if (v4)
        hipLaunchKernelGGL(k_silu_mul<true>, dim3((unsigned)grid), dim3(256), 0, s, o, g, u, n);
    else
        hipLaunchKernelGGL(k_silu_mul<false>, dim3((unsigned)grid), dim3(256), 0, s, o, g, u, n);
    *name = v4 ? "silu_mul" : "silu_mul_scalar";
    return hipGetLastError();
}

}  // namespace qmv
