// launch.h -- internal interface between the C ABI (qmv_api.cpp) and the
// kernel translation units.  Not installed, not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <string>

namespace qmv {

// Printf-style kernel variant name.  Launchers keep the result in a
// function-local static const (initialised once per template instantiation,
// thread-safe), so the pointer handed to qmv_last_kernel stays valid and no
// thread ever writes a name another thread reads.
inline std::string variant_name(const char *fmt, ...) {
    char buf[96];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    return std::string(buf);
}

// Raises the dynamic-LDS limit of kernel `kern` on the current device to
// `bytes` if the limit granted so far is smaller (nothing to do up to the
// 64 KiB default).  hipFuncSetAttribute runs at most once per kernel,
// device and larger size; thread-safe (qmv_api.cpp).
hipError_t allow_lds(const void *kern, size_t bytes);

// Arguments of the weight-streaming product for M = 1 .. 8 activation rows.
struct RowsArgs {
    int qtype;                 // 4 or 8
    float *y;                  // M x rows, row-major
    const int8_t *wq;
    const float *wd;
    int32_t rows, K;
    int32_t M;                 // activation rows (1 when x is given)
    const float *x;            // float32 activation (fused quantization), or null
    const int8_t *xq;          // Q8_0 activation quants (when x is null)
    const float *xd;           // Q8_0 activation scales (when x is null)
    const float *xn;           // rmsnorm weights applied to x before its quantization, or null
    float eps;                 // rmsnorm epsilon (when xn is given)
    const float *xu;           // FFN gate: the activation is silu(x) * xu, or null
    int8_t *xq_out;            // optional copy of the fused quantization
    float *xd_out;
    int32_t r0, r1;            // (ya: pairs [r0, r1) of gate row r and up row rows / 2 + r)
    int num_cu;                // compute units of the device (sizes the grid)
    float *ya;                 // paired gate and up rows: ya[r] = silu(y[r]) * y[rows / 2 + r], or null
};

hipError_t launch_rows(const RowsArgs &a, hipStream_t s, const char **name);
// Split-K product (the K dimension split over the wavefronts of a
// workgroup): the fused M = 1 matvec and pre-quantized M = 1 .. 4; returns
// hipErrorNotSupported (nothing launched) for shapes it does not cover.
hipError_t launch_fx(const RowsArgs &a, hipStream_t s, const char **name);
// LDS bytes the row-streaming kernel needs for M activation rows of K
// (fused: the float32 activation is staged too; rms: plus the rmsnorm
// block sums).
size_t rows_lds_bytes(int M, int K, bool fused, bool rms = false);

// Arguments of the matrix-core product for up to 64 activation rows per launch.
struct GemmArgs {
    int qtype;                 // 4 or 8
    float *Y;                  // M x rows, row-major (row m starts at Y + m * rows)
    const int8_t *wq;
    const float *wd;
    int32_t rows, K;
    const int8_t *xq;          // Q8_0 activation quants, M x K
    const float *xd;           // Q8_0 activation scales, M x K/32
    int32_t M;                 // 1 .. 64
    int32_t r0, r1;            // packed weights: r0 a multiple of 16
    const void *pq;            // packed quants (pack-once layout), or null: wq / wd row-major
    const float *pd;           // packed scales
};

constexpr int kGemmMaxRows = 64;  // activation rows per matrix-core launch

// Matrix-core product with one workgroup per compute unit and the K
// dimension split over its wavefronts (num_cu sizes the row tiles).
hipError_t launch_mm(const GemmArgs &a, int num_cu, hipStream_t s, const char **name);

// The matvec on 128-element blocks with a zero point (kernels_zp.hip).
struct ZpArgs {
    int bits;                  // 4 or 8
    float *y;
    const uint8_t *wq;         // codes, rows x K (8 bits) or rows x K/2 (4 bits)
    const float *wd;           // rows x K/128
    const uint8_t *wzp;        // rows x K/128, or null: 2^(bits-1)
    int32_t rows, K;
    const float *x;            // float32 activation, K
    int8_t *xq_out;            // optional: the quantized activation (K) ...
    float *xd_out;             // ... and its scales (K/128)
    int32_t r0, r1;
};
size_t zp_lds_bytes(int32_t K);
// Split-K form of the zero-point and K-quant products for rows of at least
// 16 units (32 elements each) per wavefront (kernels_gs.hip); returns
// hipErrorNotSupported, launching nothing, for other shapes.
hipError_t launch_gs_zp(const ZpArgs &a, int num_cu, hipStream_t s, const char **name);
hipError_t launch_zp(const ZpArgs &a, int num_cu, hipStream_t s, const char **name);
hipError_t launch_quant_b128(int8_t *q, float *d, const float *x, int64_t nblk, hipStream_t s, const char **name);

// The matvec on K-quant super-blocks (kernels_q4k.hip).
struct Q4kArgs {
    float *y;
    const uint8_t *wq;         // nibbles, rows x K/2
    const uint8_t *sc, *mn;    // rows x K/32 sub-block scales and minima (0..63)
    const float *d, *dmin;     // rows x K/256
    int32_t rows, K;
    const float *x;            // float32 activation, K
    int8_t *xq_out;            // optional: the quantized activation (K) ...
    float *xd_out;             // ... and its scales (K/256)
    int32_t r0, r1;
};
size_t q4k_lds_bytes(int32_t K);
hipError_t launch_gs_q4k(const Q4kArgs &a, int num_cu, hipStream_t s, const char **name);
hipError_t launch_q4k(const Q4kArgs &a, int num_cu, hipStream_t s, const char **name);
hipError_t launch_quant_b256(int8_t *q, float *d, const float *x, int64_t nblk, hipStream_t s, const char **name);

// Pack-once layout of Q4_0 / Q8_0 weights for the matrix-core product (units
// of 16 rows x 4 blocks in the A operand's lane order): sizes in bytes of the
// packed quants and scales, and the packing launch (a pure permutation).
size_t pack_q_bytes(int qtype, int32_t rows, int32_t K);
size_t pack_d_bytes(int32_t rows, int32_t K);
hipError_t launch_pack(int qtype, void *pq, float *pd, const int8_t *wq, const float *wd, int32_t rows, int32_t K,
                       hipStream_t s, const char **name);

// Q8_0 quantization of nblk blocks of 32 floats (activations or weights).
hipError_t launch_quant_q8(int8_t *q, float *d, const float *x, int64_t nblk, hipStream_t s,
                           const char **name);
// Q4_0 quantization of nblk blocks of 32 floats (weights).
hipError_t launch_quant_q4(int8_t *q, float *d, const float *x, int64_t nblk, hipStream_t s,
                           const char **name);

// The neighbours as launches of their own (kernels_neighbour.hip): rmsnorm
// of n floats (one workgroup; n % 32 == 0, n <= 131072) and silu(g) * u.
hipError_t launch_rmsnorm(float *o, const float *x, const float *w, int32_t n, float eps, hipStream_t s,
                          const char **name);
hipError_t launch_silu_mul(float *o, const float *g, const float *u, int64_t n, hipStream_t s, const char **name);

// Measurement kernels (kernels_ceiling.hip): a plain streaming read of
// `bytes` (multiple of 16) with `depth` (4 or 8) 16-byte loads in flight per
// thread, and chains of int8 matrix-core instructions of one shape.
hipError_t launch_ceiling_stream(uint32_t *sink, const void *buf, int64_t bytes, int32_t wgs, int32_t depth,
                                 hipStream_t s, const char **name);
hipError_t launch_ceiling_mfma(uint32_t *sink, int32_t shape, int32_t iters, int32_t wgs, int32_t a, int32_t b,
                               hipStream_t s, const char **name);

}  // namespace qmv
