// qmv_api.cpp -- the C ABI of libqmv (declared in include/qmv.h).
//
// Every entry point validates its arguments on the host before anything is
// enqueued (status convention of the Legacy-ISA ML Inference Runtime --
// Design Spec, section 6 "Error handling": return a status, never abort;
// shape checks of the loader such as K % 32 == 0 move to call entry), then
// checks once per device that the device is a gfx950 (the spec's
// instruction-set guard, section 6, turned into a device-architecture
// guard), then launches on the caller's stream.  There is no fallback path:
// a call either runs the gfx950 kernels or returns an error.
#include <cmath>

#include "qmv.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <utility>

#include "launch.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unchecked, 1 = gfx950, 2 = other architecture
std::atomic<int> g_arch[kMaxDevices];
std::atomic<int> g_num_cu[kMaxDevices];

thread_local const char *t_last_kernel = "";

bool diag_enabled() {
    static const bool v = [] {
        const char *e = getenv("QMV_DIAG");
        return e != nullptr && e[0] != '\0' && e[0] != '0';
    }();
    return v;
}

int num_cu(int dev) {
    const int n = (dev >= 0 && dev < kMaxDevices) ? g_num_cu[dev].load(std::memory_order_relaxed) : 0;
    return n > 0 ? n : 256;
}

qmv_status device_check(int *dev_out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return QMV_E_DEVICE;
    }
    int st = g_arch[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
            (void)hipGetLastError();
            return QMV_E_DEVICE;
        }
        st = (strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_num_cu[dev].store(p.multiProcessorCount, std::memory_order_relaxed);
        g_arch[dev].store(st, std::memory_order_release);
        if (diag_enabled())
            fprintf(stderr, "[qmv] device %d: %s, %d CUs -> %s\n", dev, p.gcnArchName, p.multiProcessorCount,
                    st == 1 ? "ok" : "QMV_E_ARCH");
    }
    if (dev_out) *dev_out = dev;
    return st == 1 ? QMV_OK : QMV_E_ARCH;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

qmv_status finish(hipError_t e, const char *name, long grid_hint) {
    if (e != hipSuccess) return QMV_E_DEVICE;
    t_last_kernel = name;
    if (diag_enabled()) fprintf(stderr, "[qmv] launch %s (%ld)\n", name, grid_hint);
    return QMV_OK;
}

// A matrix with no rows may have null data pointers: nothing is read.
qmv_status check_weight(const qmv_qtensor *W, int want_type) {
    if (W == nullptr) return QMV_E_ARG;
    if (W->rows != 0 && (W->q == nullptr || W->d == nullptr)) return QMV_E_ARG;
    if (W->type != QMV_Q4_0 && W->type != QMV_Q8_0) return QMV_E_FORMAT;
    if (want_type != 0 && W->type != want_type) return QMV_E_FORMAT;
    if (W->rows < 0 || W->cols <= 0 || (W->cols % QMV_QK) != 0) return QMV_E_SHAPE;
    return QMV_OK;
}

qmv_status check_range(const qmv_qtensor *W, int32_t r0, int32_t r1) {
    if (r0 < 0 || r1 > W->rows || r0 > r1) return QMV_E_SHAPE;
    return QMV_OK;
}

qmv_status check_weight_align(const qmv_qtensor *W) {
    if (!aligned(W->q, 16) || !aligned(W->d, 4)) return QMV_E_ARG;
    return QMV_OK;
}

qmv_status rows_common(int qtype, float *y, const qmv_qtensor *W, int32_t M, const float *x,
                       const int8_t *xq, const float *xd, qmv_qact *xq_out, int32_t r0, int32_t r1,
                       void *stream, const float *xn = nullptr, float eps = 0.0f, const float *xu = nullptr,
                       float *ya = nullptr) {
    qmv_status st = check_weight(W, qtype);
    if (st != QMV_OK) return st;
    if (y == nullptr && W->rows != 0) return QMV_E_ARG;
    if ((st = check_range(W, r0, r1)) != QMV_OK) return st;
    if (W->cols > 131072 || qmv::rows_lds_bytes(M, W->cols, x != nullptr, xn != nullptr) > (size_t)QMV_LDS_BYTES)
        return QMV_E_SHAPE;
    if ((st = check_weight_align(W)) != QMV_OK) return st;
    if (!aligned(y, 4)) return QMV_E_ARG;
    if (x != nullptr && !aligned(x, 16)) return QMV_E_ARG;
    if (xq != nullptr && (!aligned(xq, 16) || !aligned(xd, 4))) return QMV_E_ARG;
    if (xq_out != nullptr && (!aligned(xq_out->q, 16) || !aligned(xq_out->d, 4))) return QMV_E_ARG;
    int dev = -1;
    if ((st = device_check(&dev)) != QMV_OK) return st;
    if (xq_out != nullptr) xq_out->n = W->cols;
    if (r0 == r1) return QMV_OK;
    qmv::RowsArgs a = {};
    a.qtype = qtype;
    a.y = y;
    a.wq = W->q;
    a.wd = W->d;
    a.rows = W->rows;
    a.K = W->cols;
    a.M = M;
    a.x = x;
    a.xq = xq;
    a.xd = xd;
    a.xn = xn;
    a.eps = eps;
    a.xu = xu;
    a.xq_out = xq_out ? xq_out->q : nullptr;
    a.xd_out = xq_out ? xq_out->d : nullptr;
    a.r0 = r0;
    a.r1 = r1;
    a.num_cu = num_cu(dev);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const char *name = "";
    hipError_t e = hipErrorNotSupported;
    if (ya != nullptr) {  // paired gate and up rows [r0, r1) and F + [r0, r1)
        a.ya = ya;
        e = qmv::launch_fx(a, s, &name);
        if (e != hipErrorNotSupported) return finish(e, name, (r1 - r0 + 3) / 4);
        // no split-K form for this K: the two halves as products of their
        // own, then the gate from the stored outputs (same bits)
        const int32_t F = W->rows / 2;
        a.ya = nullptr;
        e = qmv::launch_fx(a, s, &name);
        if (e == hipErrorNotSupported) e = qmv::launch_rows(a, s, &name);
        if (e != hipSuccess) return finish(e, name, 0);
        a.xq_out = nullptr;
        a.xd_out = nullptr;
        a.r0 = F + r0;
        a.r1 = F + r1;
        e = qmv::launch_fx(a, s, &name);
        if (e == hipErrorNotSupported) e = qmv::launch_rows(a, s, &name);
        if (e != hipSuccess) return finish(e, name, 0);
        const char *gname = "";
        e = qmv::launch_silu_mul(ya + r0, y + r0, y + F + r0, r1 - r0, s, &gname);
        return finish(e, name, (r1 - r0 + 15) / 16);
    }
    e = qmv::launch_fx(a, s, &name);
    if (e == hipErrorNotSupported) e = qmv::launch_rows(a, s, &name);
    return finish(e, name, (r1 - r0 + 15) / 16);
}

qmv_status matvec_pre(int qtype, float *y, const qmv_qtensor *W, const qmv_qact *x, int32_t r0,
                      int32_t r1, void *stream) {
    if (x == nullptr || x->q == nullptr || x->d == nullptr) return QMV_E_ARG;
    qmv_status st = check_weight(W, qtype);
    if (st != QMV_OK) return st;
    if (x->n != W->cols) return QMV_E_SHAPE;
    return rows_common(qtype, y, W, 1, nullptr, x->q, x->d, nullptr, r0, r1, stream);
}

qmv_status matvec_fx(int qtype, float *y, const qmv_qtensor *W, const float *x, qmv_qact *xq,
                     int32_t r0, int32_t r1, void *stream) {
    if (x == nullptr) return QMV_E_ARG;
    if (xq != nullptr && (xq->q == nullptr || xq->d == nullptr)) return QMV_E_ARG;
    return rows_common(qtype, y, W, 1, x, nullptr, nullptr, xq, r0, r1, stream);
}

qmv_status matvec_fx_rmsnorm(int qtype, float *y, const qmv_qtensor *W, const float *x, const float *w_norm,
                             float eps, qmv_qact *xq, int32_t r0, int32_t r1, void *stream) {
    if (x == nullptr || w_norm == nullptr) return QMV_E_ARG;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return QMV_E_ARG;
    if (xq != nullptr && (xq->q == nullptr || xq->d == nullptr)) return QMV_E_ARG;
    if (!aligned(w_norm, 16)) return QMV_E_ARG;
    return rows_common(qtype, y, W, 1, x, nullptr, nullptr, xq, r0, r1, stream, w_norm, eps);
}

qmv_status matvec_fx_silu_mul(int qtype, float *y, const qmv_qtensor *W, const float *g, const float *u,
                              qmv_qact *xq, int32_t r0, int32_t r1, void *stream) {
    if (g == nullptr || u == nullptr) return QMV_E_ARG;
    if (xq != nullptr && (xq->q == nullptr || xq->d == nullptr)) return QMV_E_ARG;
    if (!aligned(u, 16)) return QMV_E_ARG;
    return rows_common(qtype, y, W, 1, g, nullptr, nullptr, xq, r0, r1, stream, nullptr, 0.0f, u);
}

qmv_status matvec_fx_swiglu(int qtype, float *ya, float *y, const qmv_qtensor *W, const float *x,
                            const float *w_norm, float eps, qmv_qact *xq, int32_t p0, int32_t p1, void *stream) {
    if (x == nullptr) return QMV_E_ARG;
    if (w_norm != nullptr && (!(eps >= 0.0f) || !std::isfinite(eps) || !aligned(w_norm, 16))) return QMV_E_ARG;
    if (xq != nullptr && (xq->q == nullptr || xq->d == nullptr)) return QMV_E_ARG;
    qmv_status st = check_weight(W, qtype);
    if (st != QMV_OK) return st;
    if ((W->rows % 2) != 0) return QMV_E_SHAPE;
    if (p0 < 0 || p1 > W->rows / 2 || p0 > p1) return QMV_E_SHAPE;
    if (W->rows != 0 && (ya == nullptr || y == nullptr)) return QMV_E_ARG;
    if (!aligned(ya, 4)) return QMV_E_ARG;
    if (W->rows == 0) return rows_common(qtype, y, W, 1, x, nullptr, nullptr, xq, 0, 0, stream, w_norm, eps);
    return rows_common(qtype, y, W, 1, x, nullptr, nullptr, xq, p0, p1, stream, w_norm, eps, nullptr, ya);
}

qmv_status gemm_passes(int qtype, float *Y, const int8_t *wq, const float *wd, const void *pq, const float *pd,
                       int32_t rows, int32_t K, const qmv_qtensor *X, int32_t r0, int32_t r1, int dev, void *stream);

qmv_status gemm(int qtype, float *Y, const qmv_qtensor *W, const qmv_qtensor *X, int32_t r0, int32_t r1,
                void *stream) {
    if (X == nullptr || X->q == nullptr || X->d == nullptr) return QMV_E_ARG;
    qmv_status st = check_weight(W, qtype);
    if (st != QMV_OK) return st;
    if (Y == nullptr && W->rows != 0) return QMV_E_ARG;
    if (X->type != QMV_Q8_0) return QMV_E_FORMAT;
    if (X->rows < 1 || X->cols != W->cols) return QMV_E_SHAPE;
    if ((st = check_range(W, r0, r1)) != QMV_OK) return st;
    if (!aligned(X->q, 16) || !aligned(X->d, 4)) return QMV_E_ARG;
    if (X->rows <= 8)  // dot-product path: all rows in one pass over the weights
        return rows_common(qtype, Y, W, X->rows, nullptr, X->q, X->d, nullptr, r0, r1, stream);
    // matrix-core path: up to 64 activation rows per pass over the weights
    if (W->cols > 131072) return QMV_E_SHAPE;
    if ((st = check_weight_align(W)) != QMV_OK) return st;
    if (!aligned(Y, 4)) return QMV_E_ARG;
    int dev = -1;
    if ((st = device_check(&dev)) != QMV_OK) return st;
    if (r0 == r1) return QMV_OK;
    return gemm_passes(qtype, Y, W->q, W->d, nullptr, nullptr, W->rows, W->cols, X, r0, r1, dev, stream);
}

qmv_status gemm_packed(int qtype, float *Y, const qmv_packed *P, const qmv_qtensor *X, int32_t r0, int32_t r1,
                       void *stream) {
    if (P == nullptr || (P->rows != 0 && (P->q == nullptr || P->d == nullptr))) return QMV_E_ARG;
    if (X == nullptr || X->q == nullptr || X->d == nullptr || (Y == nullptr && P->rows != 0)) return QMV_E_ARG;
    if (P->type != qtype || X->type != QMV_Q8_0) return QMV_E_FORMAT;
    if (P->rows < 0 || P->cols <= 0 || (P->cols % QMV_QK) != 0 || P->cols > 131072) return QMV_E_SHAPE;
    if (X->rows < 1 || X->cols != P->cols) return QMV_E_SHAPE;
    if (r0 < 0 || r1 > P->rows || r0 > r1 || (r0 % 16) != 0) return QMV_E_SHAPE;
    if (!aligned(P->q, 16) || !aligned(P->d, 16) || !aligned(X->q, 16) || !aligned(X->d, 4) || !aligned(Y, 4))
        return QMV_E_ARG;
    int dev = -1;
    qmv_status st = device_check(&dev);
    if (st != QMV_OK) return st;
    if (r0 == r1) return QMV_OK;
    return gemm_passes(qtype, Y, nullptr, nullptr, P->q, P->d, P->rows, P->cols, X, r0, r1, dev, stream);
}

qmv_status matvec_zp_fx(float *y, const qmv_zptensor *W, const float *x, qmv_qact *xq_out, int32_t r0, int32_t r1,
                        void *stream) {
    if (W == nullptr || x == nullptr) return QMV_E_ARG;
    if (W->rows != 0 && (W->q == nullptr || W->d == nullptr || y == nullptr)) return QMV_E_ARG;
    if (W->bits != 4 && W->bits != 8) return QMV_E_FORMAT;
    if (W->rows < 0 || W->cols <= 0 || (W->cols % QMV_ZP_BLOCK) != 0 || W->cols > QMV_ZP_MAX_COLS)
        return QMV_E_SHAPE;
    const int64_t row_bytes = W->bits == 8 ? W->cols : W->cols / 2;
    if ((int64_t)W->rows * row_bytes > INT32_MAX) return QMV_E_SHAPE;
    if (r0 < 0 || r1 > W->rows || r0 > r1) return QMV_E_SHAPE;
    if (!aligned(W->q, 16) || !aligned(W->d, 4) || !aligned(x, 16) || !aligned(y, 4)) return QMV_E_ARG;
    if (xq_out != nullptr && (xq_out->q == nullptr || xq_out->d == nullptr || !aligned(xq_out->q, 16) ||
                              !aligned(xq_out->d, 4)))
        return QMV_E_ARG;
    int dev = -1;
    qmv_status st = device_check(&dev);
    if (st != QMV_OK) return st;
    if (xq_out != nullptr) xq_out->n = W->cols;
    if (r0 == r1 && xq_out == nullptr) return QMV_OK;
    qmv::ZpArgs a = {};
    a.bits = W->bits;
    a.y = y;
    a.wq = W->q;
    a.wd = W->d;
    a.wzp = W->zp;
    a.rows = W->rows;
    a.K = W->cols;
    a.x = x;
    a.xq_out = xq_out != nullptr ? xq_out->q : nullptr;
    a.xd_out = xq_out != nullptr ? xq_out->d : nullptr;
    a.r0 = r0;
    a.r1 = r1;
    const char *name = "";
    const int ncu = num_cu(dev);
    hipError_t e = qmv::launch_zp(a, ncu, static_cast<hipStream_t>(stream), &name);
    return finish(e, name, (long)(r1 - r0));
}

qmv_status matvec_q4k_fx(float *y, const qmv_q4ktensor *W, const float *x, qmv_qact *xq_out, int32_t r0, int32_t r1,
                         void *stream) {
    if (W == nullptr || x == nullptr) return QMV_E_ARG;
    if (W->rows != 0 && (W->q == nullptr || W->sc == nullptr || W->mn == nullptr || W->d == nullptr ||
                         W->dmin == nullptr || y == nullptr))
        return QMV_E_ARG;
    if (W->rows < 0 || W->cols <= 0 || (W->cols % QMV_Q4K_BLOCK) != 0 || W->cols > QMV_Q4K_MAX_COLS)
        return QMV_E_SHAPE;
    if ((int64_t)W->rows * (W->cols / 2) > INT32_MAX) return QMV_E_SHAPE;
    if (r0 < 0 || r1 > W->rows || r0 > r1) return QMV_E_SHAPE;
    if (!aligned(W->q, 16) || !aligned(W->d, 4) || !aligned(W->dmin, 4) || !aligned(x, 16) || !aligned(y, 4))
        return QMV_E_ARG;
    if (xq_out != nullptr && (xq_out->q == nullptr || xq_out->d == nullptr || !aligned(xq_out->q, 16) ||
                              !aligned(xq_out->d, 4)))
        return QMV_E_ARG;
    int dev = -1;
    qmv_status st = device_check(&dev);
    if (st != QMV_OK) return st;
    if (xq_out != nullptr) xq_out->n = W->cols;
    if (r0 == r1 && xq_out == nullptr) return QMV_OK;
    qmv::Q4kArgs a = {};
    a.y = y;
    a.wq = W->q;
    a.sc = W->sc;
    a.mn = W->mn;
    a.d = W->d;
    a.dmin = W->dmin;
    a.rows = W->rows;
    a.K = W->cols;
    a.x = x;
    a.xq_out = xq_out != nullptr ? xq_out->q : nullptr;
    a.xd_out = xq_out != nullptr ? xq_out->d : nullptr;
    a.r0 = r0;
    a.r1 = r1;
    const char *name = "";
    const int ncu = num_cu(dev);
    hipError_t e = qmv::launch_q4k(a, ncu, static_cast<hipStream_t>(stream), &name);
    return finish(e, name, (long)(r1 - r0));
}

// ceil(M / 64) matrix-core passes over the weights (row-major wq / wd, or
// packed pq / pd)
qmv_status gemm_passes(int qtype, float *Y, const int8_t *wq, const float *wd, const void *pq, const float *pd,
                       int32_t rows, int32_t K, const qmv_qtensor *X, int32_t r0, int32_t r1, int dev, void *stream) {
    const int32_t nb = K / QMV_QK;
    qmv_status st = QMV_OK;
    for (int32_t m0 = 0; m0 < X->rows; m0 += qmv::kGemmMaxRows) {
        qmv::GemmArgs a = {};
        a.qtype = qtype;
        a.Y = Y + (size_t)m0 * rows;
        a.wq = wq;
        a.wd = wd;
        a.pq = pq;
        a.pd = pd;
        a.rows = rows;
        a.K = K;
        a.xq = X->q + (size_t)m0 * K;
        a.xd = X->d + (size_t)m0 * nb;
        a.M = (X->rows - m0) < qmv::kGemmMaxRows ? (X->rows - m0) : qmv::kGemmMaxRows;
        a.r0 = r0;
        a.r1 = r1;
        const char *name = "";
        const int ncu = num_cu(dev);
        hipError_t e = qmv::launch_mm(a, ncu, static_cast<hipStream_t>(stream), &name);
        if ((st = finish(e, name, (r1 - r0 + 15) / 16)) != QMV_OK) return st;
    }
    return QMV_OK;
}

}  // namespace

namespace qmv {

hipError_t allow_lds(const void *kern, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    static std::mutex mu;
    static std::map<std::pair<const void *, int>, size_t> granted;  // (kernel, device) -> bytes
    std::lock_guard<std::mutex> lock(mu);
    size_t &g = granted[std::make_pair(kern, dev)];
    if (g >= bytes) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) g = bytes;
    return e;
}

}  // namespace qmv

extern "C" {

qmv_status qmv_device_check(void) { return device_check(nullptr); }

qmv_status qmv_quantize_q8(qmv_qact *out, const float *x, int64_t k, void *stream) {
    if (out == nullptr) return QMV_E_ARG;
    if (k < 0 || (k % QMV_QK) != 0 || k > INT32_MAX) return QMV_E_SHAPE;
    if (k == 0) {  // nothing to quantize: data pointers may be null
        out->n = 0;
        return QMV_OK;
    }
    if (out->q == nullptr || out->d == nullptr || x == nullptr) return QMV_E_ARG;
    if (!aligned(x, 16) || !aligned(out->q, 16) || !aligned(out->d, 4)) return QMV_E_ARG;
    qmv_status st = device_check(nullptr);
    if (st != QMV_OK) return st;
    out->n = (int32_t)k;
    const char *name = "";
    hipError_t e = qmv::launch_quant_q8(out->q, out->d, x, k / QMV_QK, static_cast<hipStream_t>(stream), &name);
    return finish(e, name, (long)(k / QMV_QK));
}

qmv_status qmv_quantize_weights(const qmv_qtensor *W, const float *w, void *stream) {
    qmv_status st = check_weight(W, 0);
    if (st != QMV_OK) return st;
    if (w == nullptr && W->rows != 0) return QMV_E_ARG;
    if (!aligned(w, 16)) return QMV_E_ARG;
    if ((st = check_weight_align(W)) != QMV_OK) return st;
    if ((st = device_check(nullptr)) != QMV_OK) return st;
    const int64_t nblk = (int64_t)W->rows * (W->cols / QMV_QK);
    if (nblk == 0) return QMV_OK;
    const char *name = "";
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = W->type == QMV_Q8_0 ? qmv::launch_quant_q8(W->q, W->d, w, nblk, s, &name)
                                       : qmv::launch_quant_q4(W->q, W->d, w, nblk, s, &name);
    return finish(e, name, (long)nblk);
}

qmv_status qmv_matvec_q8(float *y, const qmv_qtensor *W, const qmv_qact *x, int32_t r0, int32_t r1,
                         void *stream) {
    return matvec_pre(QMV_Q8_0, y, W, x, r0, r1, stream);
}

qmv_status qmv_matvec_q4(float *y, const qmv_qtensor *W, const qmv_qact *x, int32_t r0, int32_t r1,
                         void *stream) {
    return matvec_pre(QMV_Q4_0, y, W, x, r0, r1, stream);
}

qmv_status qmv_matvec_q8_fx(float *y, const qmv_qtensor *W, const float *x, qmv_qact *xq, int32_t r0,
                            int32_t r1, void *stream) {
    return matvec_fx(QMV_Q8_0, y, W, x, xq, r0, r1, stream);
}

qmv_status qmv_matvec_q4_fx(float *y, const qmv_qtensor *W, const float *x, qmv_qact *xq, int32_t r0,
                            int32_t r1, void *stream) {
    return matvec_fx(QMV_Q4_0, y, W, x, xq, r0, r1, stream);
}

qmv_status qmv_matvec_q8_fx_rmsnorm(float *y, const qmv_qtensor *W, const float *x, const float *w_norm,
                                    float eps, qmv_qact *xq, int32_t r0, int32_t r1, void *stream) {
    return matvec_fx_rmsnorm(QMV_Q8_0, y, W, x, w_norm, eps, xq, r0, r1, stream);
}

qmv_status qmv_matvec_q4_fx_rmsnorm(float *y, const qmv_qtensor *W, const float *x, const float *w_norm,
                                    float eps, qmv_qact *xq, int32_t r0, int32_t r1, void *stream) {
    return matvec_fx_rmsnorm(QMV_Q4_0, y, W, x, w_norm, eps, xq, r0, r1, stream);
}

qmv_status qmv_matvec_q8_fx_silu_mul(float *y, const qmv_qtensor *W, const float *g, const float *u,
                                     qmv_qact *xq, int32_t r0, int32_t r1, void *stream) {
    return matvec_fx_silu_mul(QMV_Q8_0, y, W, g, u, xq, r0, r1, stream);
}

qmv_status qmv_matvec_q4_fx_silu_mul(float *y, const qmv_qtensor *W, const float *g, const float *u,
                                     qmv_qact *xq, int32_t r0, int32_t r1, void *stream) {
    return matvec_fx_silu_mul(QMV_Q4_0, y, W, g, u, xq, r0, r1, stream);
}

qmv_status qmv_matvec_q8_fx_swiglu(float *a, float *y, const qmv_qtensor *W, const float *x, const float *w_norm,
                                   float eps, qmv_qact *xq, int32_t p0, int32_t p1, void *stream) {
    return matvec_fx_swiglu(QMV_Q8_0, a, y, W, x, w_norm, eps, xq, p0, p1, stream);
}

qmv_status qmv_matvec_q4_fx_swiglu(float *a, float *y, const qmv_qtensor *W, const float *x, const float *w_norm,
                                   float eps, qmv_qact *xq, int32_t p0, int32_t p1, void *stream) {
    return matvec_fx_swiglu(QMV_Q4_0, a, y, W, x, w_norm, eps, xq, p0, p1, stream);
}

qmv_status qmv_gemm_q8(float *Y, const qmv_qtensor *W, const qmv_qtensor *X, int32_t r0, int32_t r1,
                       void *stream) {
    return gemm(QMV_Q8_0, Y, W, X, r0, r1, stream);
}

qmv_status qmv_gemm_q4(float *Y, const qmv_qtensor *W, const qmv_qtensor *X, int32_t r0, int32_t r1,
                       void *stream) {
    return gemm(QMV_Q4_0, Y, W, X, r0, r1, stream);
}

qmv_status qmv_quantize_q8_b128(qmv_qact *out, const float *x, int64_t k, void *stream) {
    if (out == nullptr) return QMV_E_ARG;
    if (k < 0 || (k % QMV_ZP_BLOCK) != 0 || k > INT32_MAX) return QMV_E_SHAPE;
    if (k == 0) {
        out->n = 0;
        return QMV_OK;
    }
    if (out->q == nullptr || out->d == nullptr || x == nullptr) return QMV_E_ARG;
    if (!aligned(x, 16) || !aligned(out->q, 16) || !aligned(out->d, 4)) return QMV_E_ARG;
    qmv_status st = device_check(nullptr);
    if (st != QMV_OK) return st;
    out->n = (int32_t)k;
    const char *name = "";
    hipError_t e =
        qmv::launch_quant_b128(out->q, out->d, x, k / QMV_ZP_BLOCK, static_cast<hipStream_t>(stream), &name);
    return finish(e, name, (long)(k / QMV_ZP_BLOCK));
}

qmv_status qmv_matvec_zp_fx(float *y, const qmv_zptensor *W, const float *x, qmv_qact *xq, int32_t r0, int32_t r1,
                            void *stream) {
    return matvec_zp_fx(y, W, x, xq, r0, r1, stream);
}

qmv_status qmv_quantize_q8_b256(qmv_qact *out, const float *x, int64_t k, void *stream) {
    if (out == nullptr) return QMV_E_ARG;
    if (k < 0 || (k % QMV_Q4K_BLOCK) != 0 || k > INT32_MAX) return QMV_E_SHAPE;
    if (k == 0) {
        out->n = 0;
        return QMV_OK;
    }
    if (out->q == nullptr || out->d == nullptr || x == nullptr) return QMV_E_ARG;
    if (!aligned(x, 16) || !aligned(out->q, 16) || !aligned(out->d, 4)) return QMV_E_ARG;
    qmv_status st = device_check(nullptr);
    if (st != QMV_OK) return st;
    out->n = (int32_t)k;
    const char *name = "";
    hipError_t e =
        qmv::launch_quant_b256(out->q, out->d, x, k / QMV_Q4K_BLOCK, static_cast<hipStream_t>(stream), &name);
    return finish(e, name, (long)(k / QMV_Q4K_BLOCK));
}

qmv_status qmv_matvec_q4k_fx(float *y, const qmv_q4ktensor *W, const float *x, qmv_qact *xq, int32_t r0, int32_t r1,
                             void *stream) {
    return matvec_q4k_fx(y, W, x, xq, r0, r1, stream);
}

qmv_status qmv_pack_bytes(int32_t type, int32_t rows, int32_t cols, int64_t *q_bytes, int64_t *d_bytes) {
    if (q_bytes == nullptr || d_bytes == nullptr) return QMV_E_ARG;
    if (type != QMV_Q4_0 && type != QMV_Q8_0) return QMV_E_FORMAT;
    if (rows < 0 || cols <= 0 || (cols % QMV_QK) != 0 || cols > 131072) return QMV_E_SHAPE;
    *q_bytes = (int64_t)qmv::pack_q_bytes(type, rows, cols);
    *d_bytes = (int64_t)qmv::pack_d_bytes(rows, cols);
    return QMV_OK;
}

qmv_status qmv_pack_weights(qmv_packed *P, const qmv_qtensor *W, void *stream) {
    if (P == nullptr) return QMV_E_ARG;
    qmv_status st = check_weight(W, 0);
    if (st != QMV_OK) return st;
    if (W->rows != 0 && (P->q == nullptr || P->d == nullptr)) return QMV_E_ARG;
    if (W->cols > 131072) return QMV_E_SHAPE;
    if ((st = check_weight_align(W)) != QMV_OK) return st;
    if (!aligned(P->q, 16) || !aligned(P->d, 16)) return QMV_E_ARG;
    if ((st = device_check(nullptr)) != QMV_OK) return st;
    P->rows = W->rows;
    P->cols = W->cols;
    P->type = W->type;
    if (W->rows == 0) return QMV_OK;
    const char *name = "";
    hipError_t e = qmv::launch_pack(W->type, P->q, P->d, W->q, W->d, W->rows, W->cols,
                                    static_cast<hipStream_t>(stream), &name);
    return finish(e, name, (long)((W->rows + 15) / 16));
}

qmv_status qmv_gemm_q8_packed(float *Y, const qmv_packed *P, const qmv_qtensor *X, int32_t r0, int32_t r1,
                              void *stream) {
    return gemm_packed(QMV_Q8_0, Y, P, X, r0, r1, stream);
}

qmv_status qmv_gemm_q4_packed(float *Y, const qmv_packed *P, const qmv_qtensor *X, int32_t r0, int32_t r1,
                              void *stream) {
    return gemm_packed(QMV_Q4_0, Y, P, X, r0, r1, stream);
}

qmv_status qmv_rmsnorm(float *o, const float *x, const float *w, int64_t n, float eps, void *stream) {
    if (o == nullptr || x == nullptr || w == nullptr) return QMV_E_ARG;
    if (n <= 0 || (n % QMV_QK) != 0 || n > 131072) return QMV_E_SHAPE;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return QMV_E_ARG;
    if (!aligned(o, 16) || !aligned(x, 16) || !aligned(w, 16)) return QMV_E_ARG;
    qmv_status st = device_check(nullptr);
    if (st != QMV_OK) return st;
    const char *name = "";
    hipError_t e = qmv::launch_rmsnorm(o, x, w, (int32_t)n, eps, static_cast<hipStream_t>(stream), &name);
    return finish(e, name, 1);
}

qmv_status qmv_silu_mul(float *o, const float *g, const float *u, int64_t n, void *stream) {
    if (n < 0 || n > INT32_MAX) return QMV_E_SHAPE;
    if (n == 0) return QMV_OK;
    if (o == nullptr || g == nullptr || u == nullptr) return QMV_E_ARG;
    if (!aligned(o, 16) || !aligned(g, 16) || !aligned(u, 16)) return QMV_E_ARG;
    qmv_status st = device_check(nullptr);
    if (st != QMV_OK) return st;
    const char *name = "";
    hipError_t e = qmv::launch_silu_mul(o, g, u, n, static_cast<hipStream_t>(stream), &name);
    return finish(e, name, (long)(n / 1024));
}

qmv_status qmv_ceiling_stream_read(uint32_t *sink, const void *buf, int64_t bytes, int32_t workgroups,
                                   int32_t depth, void *stream) {
    if (sink == nullptr || buf == nullptr || !aligned(buf, 16) || !aligned(sink, 4)) return QMV_E_ARG;
    if (depth != 4 && depth != 8) return QMV_E_ARG;
    if (bytes < 16 || (bytes % 16) != 0 || workgroups < 1 || workgroups > 65536) return QMV_E_SHAPE;
    qmv_status st = device_check(nullptr);
    if (st != QMV_OK) return st;
    const char *name = "";
    hipError_t e = qmv::launch_ceiling_stream(sink, buf, bytes, workgroups, depth, static_cast<hipStream_t>(stream),
                                              &name);
    return finish(e, name, workgroups);
}

qmv_status qmv_ceiling_mfma_i8(uint32_t *sink, int32_t shape, int32_t iters, int32_t workgroups, int32_t a,
                               int32_t b, void *stream) {
    if (sink == nullptr || !aligned(sink, 4)) return QMV_E_ARG;
    if (shape < 0 || shape > 2) return QMV_E_ARG;
    if (iters < 0 || workgroups < 1 || workgroups > 65536) return QMV_E_SHAPE;
    qmv_status st = device_check(nullptr);
    if (st != QMV_OK) return st;
    const char *name = "";
    hipError_t e = qmv::launch_ceiling_mfma(sink, shape, iters, workgroups, a, b, static_cast<hipStream_t>(stream),
                                            &name);
    return finish(e, name, workgroups);
}

const char *qmv_status_str(qmv_status s) {
    switch (s) {
        case QMV_OK: return "QMV_OK";
        case QMV_E_SHAPE: return "QMV_E_SHAPE: bad shape, size mismatch or row range";
        case QMV_E_FORMAT: return "QMV_E_FORMAT: wrong quantization type tag";
        case QMV_E_ARG: return "QMV_E_ARG: null or misaligned pointer";
        case QMV_E_ARCH: return "QMV_E_ARCH: device is not gfx950";
        case QMV_E_DEVICE: return "QMV_E_DEVICE: no usable HIP device or launch failure";
    }
    return "unknown qmv_status";
}

const char *qmv_last_kernel(void) { return t_last_kernel; }

}  // extern "C"
