// kernels_ceiling.hip -- two measurement kernels that bound what any kernel of
// this library can reach on the chip: a plain streaming read of device
// memory (the HBM side of the roofline, as the "ONNX Runtime" page puts its
// kernel against a STREAM floor) and a loop of int8 matrix-core instructions
// with operands in registers (the arithmetic side).  Neither is on the
// product path; the bench reports each kernel's rate as a fraction of these.
#include "device_common.h"
#include "launch.h"

namespace qmv {
namespace {

// XOR of every 32-bit word of buf[0, n16 * 16).  The grid reads the buffer
// in rounds of D x (threads) 16-byte pieces: in a round thread t loads
// pieces base + d * threads + t for d < D (each load instruction of a
// wavefront covers 1 KiB contiguously), all D issued before any is used, so
// a buffer of up to D x threads pieces is requested at once.  One word per
// workgroup goes to sink (the XOR of its share), so the loads cannot be
// dropped and the result can be checked.
typedef unsigned u4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ void __launch_bounds__(1024) k_stream_read(uint32_t *__restrict__ sink, const u4 *__restrict__ buf,
                                                      int64_t n16) {
    __shared__ uint32_t s_x[16];
    const int64_t T = (int64_t)gridDim.x * blockDim.x;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (int64_t base = 0; base < n16; base += D * T) {
        u4 v[D];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int64_t i = base + d * T + t;
            v[d] = i < n16 ? __builtin_nontemporal_load(buf + i) : (u4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int d = 0; d < D; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
    if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) x ^= s_x[w];
        sink[blockIdx.x] = x;
    }
}

// CH independent accumulation chains per wavefront, each `iters` int8
// matrix-core instructions long, operands all bytes a (A) and b (B):
//   SHAPE 0: v_mfma_i32_16x16x32_i8, SHAPE 1: v_mfma_i32_16x16x64_i8,
//   SHAPE 2: v_mfma_i32_32x32x32_i8.
// Every result element ends at iters * kdepth * a * b; the sum (mod 2^32)
// of a wavefront's elements over its chains goes to sink[wavefront].
template <int SHAPE, int CH>
__global__ void __launch_bounds__(256) k_mfma_loop(uint32_t *__restrict__ sink, int32_t iters, int32_t a, int32_t b) {
    const int pa = (a & 0xFF) * 0x01010101, pb = (b & 0xFF) * 0x01010101;
    uint32_t tot = 0;
    if constexpr (SHAPE == 0) {
        const long A = (long)(((unsigned long)(unsigned)pa << 32) | (unsigned)pa);
        const long B = (long)(((unsigned long)(unsigned)pb << 32) | (unsigned)pb);
        v4i acc[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] = (v4i){0, 0, 0, 0};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, acc[c], 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int v = 0; v < 4; ++v) tot += (uint32_t)acc[c][v];
    } else if constexpr (SHAPE == 1) {
        const v4i A = {pa, pa, pa, pa}, B = {pb, pb, pb, pb};
        v4i acc[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] = (v4i){0, 0, 0, 0};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, acc[c], 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int v = 0; v < 4; ++v) tot += (uint32_t)acc[c][v];
    } else {
        const v4i A = {pa, pa, pa, pa}, B = {pb, pb, pb, pb};
        v16i acc[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[c][v] = 0;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < CH; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, acc[c], 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int v = 0; v < 16; ++v) tot += (uint32_t)acc[c][v];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) tot += (uint32_t)__shfl_xor((int)tot, o);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = tot;
}

template <int SHAPE>
hipError_t launch_mfma_shape(uint32_t *sink, int32_t iters, int32_t wgs, int32_t a, int32_t b, hipStream_t s,
                             const char **name) {
    hipLaunchKernelGGL((k_mfma_loop<SHAPE, 4>), dim3(wgs), dim3(256), 0, s, sink, iters, a, b);
    static const char *names[3] = {"ceiling_mfma_i32_16x16x32_i8", "ceiling_mfma_i32_16x16x64_i8",
                                   "ceiling_mfma_i32_32x32x32_i8"};
    *name = names[SHAPE];
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ceiling_stream(uint32_t *sink, const void *buf, int64_t bytes, int32_t wgs, int32_t depth,
                                 hipStream_t s, const char **name) {
    const int64_t n16 = bytes / 16;
    if (depth == 8) {
        hipLaunchKernelGGL(k_stream_read<8>, dim3(wgs), dim3(1024), 0, s, sink, static_cast<const u4 *>(buf), n16);
        *name = "ceiling_stream_read_d8";
    } else {
        hipLaunchKernelGGL(k_stream_read<4>, dim3(wgs), dim3(1024), 0, s, sink, static_cast<const u4 *>(buf), n16);
        *name = "ceiling_stream_read_d4";
    }
    return hipGetLastError();
}

hipError_t launch_ceiling_mfma(uint32_t *sink, int32_t shape, int32_t iters, int32_t wgs, int32_t a, int32_t b,
                               hipStream_t s, const char **name) {
    switch (shape) {
        case 0: return launch_mfma_shape<0>(sink, iters, wgs, a, b, s, name);
        case 1: return launch_mfma_shape<1>(sink, iters, wgs, a, b, s, name);
        default: return launch_mfma_shape<2>(sink, iters, wgs, a, b, s, name);
    }
}

}  // namespace qmv
