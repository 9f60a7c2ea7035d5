// kernels_pack.hip -- pack-once re-layout of Q4_0 / Q8_0 weights into the
// operand order of the int8 matrix-core product (gfx950).
//
// The spec's storage is row-major SoA (Legacy-ISA ML Inference Runtime --
// Design Spec, section 4 table: per row, the quants of each 32-element
// block, then all scales); its companion write-ups re-lay weights once into
// panels matched to the multiply instruction.  Here the unit is a tile of
// 16 rows by 4 blocks, stored in the lane order of the A operand of
// v_mfma_i32_16x16x32_i8 (lane l = 16 g + i supplies elements 8 g .. 8 g + 7
// of row i), so a wavefront reads a unit with one 16-byte load per lane
// (Q4_0; two for Q8_0), each 1 KiB contiguous:
//   quants of unit (T, Q): lane l, block u of the 4:
//     Q4_0  4 bytes at 16 l + 4 u: byte j holds element 8 g + j in its low
//           nibble and element 8 g + 4 + j in its high nibble (nibble = value
//           + 8, as stored), so two masks give the operand's 8 bytes;
//     Q8_0  8 bytes at 1024 (u / 2) + 16 l + 8 (u % 2): elements 8 g .. 8 g + 7
//           (two 1 KiB halves, blocks 0-1 and 2-3, so that each of the
//           wavefront's two 16-byte loads reads 1 KiB contiguously).
//   scales of unit (T, Q): 64 floats, row r of the tile and block u at 4 r + u.
// Units follow each other block-quad fastest: unit (T, Q) at T * nq + Q, nq =
// ceil(K / 128).  Rows past the matrix (the last tile) and blocks past K (the
// last quad) hold value 0 and scale 0.  Packing is a pure permutation of the
// stored bytes and scales: nothing is recomputed.
#include "device_common.h"
#include "launch.h"

namespace qmv {
namespace {

template <int QT>
__global__ void __launch_bounds__(256)
k_pack(uint8_t *__restrict__ pq, float *__restrict__ pd, const int8_t *__restrict__ wq, const float *__restrict__ wd,
       int32_t rows, int32_t nb, int32_t nq, int64_t units) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (unit, lane)
    if (e >= units * 64) return;
    const int64_t unit = e >> 6;
    const int l = (int)(e & 63);
    const int64_t T = unit / nq;
    const int Q = (int)(unit - T * nq);
    const int g = l >> 4, i = l & 15;
    const int64_t row = 16 * T + i;
    if constexpr (QT == 4) {
        unsigned out[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int b = 4 * Q + u;
            if (row < rows && b < nb) {
                // source bytes 8 (g & 1) .. + 7 of the block; elements 8 g .. 8 g + 7 are their
                // low nibbles (g < 2) or high nibbles (g >= 2)
                const uint2 v = *reinterpret_cast<const uint2 *>(wq + (row * nb + b) * 16 + 8 * (g & 1));
                const int sh = 4 * (g >> 1);
                out[u] = ((v.x >> sh) & 0x0F0F0F0Fu) | (((v.y >> sh) & 0x0F0F0F0Fu) << 4);
            } else {
                out[u] = 0x88888888u;  // value 0
            }
        }
        *reinterpret_cast<uint4 *>(pq + unit * 1024 + 16 * l) = make_uint4(out[0], out[1], out[2], out[3]);
    } else {
        uint2 out[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int b = 4 * Q + u;
            out[u] = (row < rows && b < nb) ? *reinterpret_cast<const uint2 *>(wq + (row * nb + b) * 32 + 8 * g)
                                            : make_uint2(0u, 0u);
        }
        *reinterpret_cast<uint4 *>(pq + unit * 2048 + 16 * l) = make_uint4(out[0].x, out[0].y, out[1].x, out[1].y);
        *reinterpret_cast<uint4 *>(pq + unit * 2048 + 1024 + 16 * l) =
            make_uint4(out[2].x, out[2].y, out[3].x, out[3].y);
    }
    // scale of tile row l / 4, block l % 4
    const int64_t srow = 16 * T + (l >> 2);
    const int sb = 4 * Q + (l & 3);
    pd[unit * 64 + l] = (srow < rows && sb < nb) ? wd[srow * nb + sb] : 0.0f;
}

}  // namespace

size_t pack_q_bytes(int qtype, int32_t rows, int32_t K) {
    const int64_t tiles = (rows + 15) / 16, nq = (K / QK + 3) / 4;
    return (size_t)(tiles * nq) * (qtype == 4 ? 1024 : 2048);
}

size_t pack_d_bytes(int32_t rows, int32_t K) {
    const int64_t tiles = (rows + 15) / 16, nq = (K / QK + 3) / 4;
    return (size_t)(tiles * nq) * 256;
}

hipError_t launch_pack(int qtype, void *pq, float *pd, const int8_t *wq, const float *wd, int32_t rows, int32_t K,
                       hipStream_t s, const char **name) {
    const int32_t nb = K / QK, nq = (nb + 3) / 4;
    const int64_t units = (int64_t)((rows + 15) / 16) * nq;
    const int64_t threads = units * 64;
    const unsigned grid = (unsigned)((threads + 255) / 256);
    if (qtype == 4)
        hipLaunchKernelGGL(k_pack<4>, dim3(grid), dim3(256), 0, s, static_cast<uint8_t *>(pq), pd, wq, wd, rows, nb,
                           nq, units);
    else
        hipLaunchKernelGGL(k_pack<8>, dim3(grid), dim3(256), 0, s, static_cast<uint8_t *>(pq), pd, wq, wd, rows, nb,
                           nq, units);
    *name = qtype == 4 ? "pack_q4" : "pack_q8";
    return hipGetLastError();
}

}  // namespace qmv
