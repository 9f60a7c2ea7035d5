// kernels_quant.hip -- Q8_0 and Q4_0 quantization kernels (gfx950).
//
// Q8_0 (Legacy-ISA ML Inference Runtime -- Design Spec, section 4 "Q8
// quantization" and the section 5 rounding rule): per 32-element block
// d = amax / 127 and q = trunc(x * (127 / amax) + copysign(0.5, x)).
// Q4_0 weights: the spec fixes the storage (section 4 table: byte j holds
// element j in the low nibble and element j + 16 in the high nibble,
// value = nibble - 8) and symmetric quantization; the rule used is the Q8_0
// one with 7 in place of 127.
//
// Eight lanes take one block, one float4 each, so a wavefront reads 1 KiB of
// contiguous input per load and writes contiguous quants.  The arithmetic is
// the same __device__ code the fused matvec staging runs, so both produce
// the same bits.
#include "device_common.h"
#include "launch.h"

namespace qmv {
namespace {

__global__ void __launch_bounds__(256)
k_quant_q8(int8_t *__restrict__ q, float *__restrict__ d, const float *__restrict__ x, int64_t nblk) {
    const int64_t n = nblk * 8;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
        const int64_t blk = e >> 3;
        const int c = (int)(e & 7);
        const float4 v = *reinterpret_cast<const float4 *>(x + blk * QK + 4 * c);
        float dd;
        int s;
        const int pk = quant_q8_group8(v, dd, s);
        reinterpret_cast<int *>(q + blk * QK)[c] = pk;
        if (c == 0) d[blk] = dd;
    }
}

__global__ void __launch_bounds__(256)
k_quant_q4(int8_t *__restrict__ q, float *__restrict__ d, const float *__restrict__ x, int64_t nblk) {
    const int64_t n = nblk * 8;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
        const int64_t blk = e >> 3;
        const int c = (int)(e & 7);
        const float4 v = *reinterpret_cast<const float4 *>(x + blk * QK + 4 * c);
        float dd;
        const int nib = quant_q4_group8(v, dd);
        // lanes 0..3 hold elements 0..15 (low nibbles of bytes 0..15),
        // lanes 4..7 hold elements 16..31 (high nibbles of the same bytes)
        const int hi = dpp_down4(nib);  // lane c (c < 4) receives lane c + 4
        if (c < 4) reinterpret_cast<int *>(q + blk * (QK / 2))[c] = nib | (hi << 4);
        if (c == 0) d[blk] = dd;
    }
}

int grid_for(int64_t nblk) {
    int64_t g = (nblk * 8 + 255) / 256;
    if (g > 4096) g = 4096;
    if (g < 1) g = 1;
    return (int)g;
}

}  // namespace

hipError_t launch_quant_q8(int8_t *q, float *d, const float *x, int64_t nblk, hipStream_t s,
                           const char **name) {
    hipLaunchKernelGGL(k_quant_q8, dim3(grid_for(nblk)), dim3(256), 0, s, q, d, x, nblk);
    *name = "quant_q8";
    return hipGetLastError();
}

hipError_t launch_quant_q4(int8_t *q, float *d, const float *x, int64_t nblk, hipStream_t s,
                           const char **name) {
    hipLaunchKernelGGL(k_quant_q4, dim3(grid_for(nblk)), dim3(256), 0, s, q, d, x, nblk);
    *name = "quant_q4";
    return hipGetLastError();
}

}  // namespace qmv
