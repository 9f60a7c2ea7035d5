/*
 * qmv.h -- C ABI of libqmv: block-quantized weight x activation products
 * for LLM decode on one AMD Instinct MI355X (gfx950).
 *
 * Formats (Legacy-ISA ML Inference Runtime -- Design Spec, section 4,
 * "Quantization Formats"):
 *   - blocks of QK = 32 consecutive elements along K; every K is a multiple
 *     of 32;
 *   - Q8_0: one int8 per element, clamped to [-127, 127], plus one float32
 *     scale d per block (value = q * d);
 *   - Q4_0: 16 bytes per block, byte j holds element j in its low nibble and
 *     element j + 16 in its high nibble, value = (nibble - 8) * d, plus one
 *     float32 scale d per block;
 *   - structure-of-arrays: all quant bytes of a tensor in one array q, all
 *     scales in a second array d, both row-major over (row, block).
 *     Row r of a rows x cols tensor starts at q + r * cols (Q8_0) or
 *     q + r * cols / 2 (Q4_0) and at d + r * cols / 32.
 *
 * Arithmetic (section 4, "Integer dot per block"): per block the int8 dot
 * sumi = sum of w * qx is formed exactly in int32; the output is the fp32
 * sum over blocks of sumi * dw * dx.  The summation order over blocks is
 * the library's; results are within |y - y_ref| <= 1e-5 * sum_b |sumi * dw
 * * dx| + 1e-6 of the in-order sum, and quantized activations and every
 * block sum are bit-exact.
 *
 * Memory: every data pointer is a DEVICE pointer owned by the caller (for
 * example the storage of a torch tensor).  The library allocates nothing,
 * keeps no state besides a per-device architecture check, and never frees
 * caller memory.  The qmv_qtensor / qmv_qact structs themselves live in
 * host memory and are read during the call only.
 *
 * Streams: every call is asynchronous on `stream` (a hipStream_t; NULL =
 * the null stream).  A status of QMV_OK means the work was validated and
 * enqueued; a fault inside a kernel surfaces at the caller's next
 * synchronisation.
 *
 * Errors (section 6, "Error handling": library functions return a status,
 * never abort): arguments are checked before anything is enqueued and a
 * failed check enqueues nothing.  Order of checks: null pointers
 * (QMV_E_ARG), type tags (QMV_E_FORMAT), shapes (QMV_E_SHAPE), alignment
 * (QMV_E_ARG), then the device (QMV_E_DEVICE / QMV_E_ARCH).
 *
 * Preconditions not checked on the hot path: finite inputs; for
 * activation quantization a block maximum of 0 or at least FLT_MIN; Q8_0
 * weight quants in [-127, 127] (-128 is still computed exactly).
 */
#ifndef QMV_H
#define QMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (mirror the spec's section 6 status list, with the
 * instruction-set check replaced by a device-architecture check). */
typedef enum {
    QMV_OK = 0,
    QMV_E_SHAPE = 1,   /* K % 32 != 0, sizes disagree, bad row range, or a size beyond the documented limits */
    QMV_E_FORMAT = 2,  /* wrong type tag for the call */
    QMV_E_ARG = 3,     /* null or misaligned pointer */
    QMV_E_ARCH = 4,    /* the current device is not gfx950 */
    QMV_E_DEVICE = 5   /* no usable device, or the HIP runtime rejected a launch */
} qmv_status;

/* Type tags of qmv_qtensor.type (numeric values are this library's). */
enum { QMV_Q4_0 = 4, QMV_Q8_0 = 8 };

/* Block length. */
#define QMV_QK 32

/* On-chip LDS budget of the single-row and few-row products: the quantized
 * activation rows are staged in LDS, 40 bytes per 32-element block per
 * activation row (rounded up to 64 blocks), plus, for the fused calls, the
 * float32 activation itself (4 bytes per element, rounded up to 1 KiB),
 * and for the rmsnorm form 4 bytes per block (rounded up to a power of two)
 * of block sums.  That bounds K: at most 131072 for the pre-quantized
 * single-row product, 30720 for the fused one (30208 with rmsnorm), M * K
 * <= 131072 for M <= 8 activation rows.
 * The matrix-core product (M > 8) stages nothing but its 32 KiB of partial
 * sums. */
#define QMV_LDS_BYTES (160 * 1024)

/* A quantized weight matrix (spec section 4, ml_qtensor): rows x cols,
 * q = rows * cols bytes (Q8_0) or rows * cols / 2 bytes (Q4_0),
 * d = rows * cols / 32 floats.  q must be 16-byte aligned, d 4-byte
 * aligned.  Matrices with rows = 0 (here and in qmv_zptensor and
 * qmv_packed) may have null data pointers, and so may the (empty) outputs
 * y / Y of the calls on them: nothing is read or written. */
typedef struct {
    int8_t *q;
    float *d;
    int32_t rows;
    int32_t cols;
    uint8_t type;      /* QMV_Q4_0 or QMV_Q8_0 */
} qmv_qtensor;

/* A Q8_0 activation vector (spec section 4, ml_qact): q = n bytes, d = n/32
 * floats.  q must be 16-byte aligned, d 4-byte aligned. */
typedef struct {
    int8_t *q;
    float *d;
    int32_t n;
} qmv_qact;

/* ---------------------------------------------------------------------------
 * qmv_quantize_q8 -- Q8_0 quantization of k floats (spec section 5,
 * ml_k_quantize_q8; rule of section 4 "Q8 quantization" with the rounding
 * of section 5): per block d = amax / 127, q = trunc(x * (127 / amax) +
 * copysign(0.5, x)) with each float operation rounded separately,
 * amax = 0 giving d = 0 and q = 0.
 *   out->q : k bytes (16-byte aligned), out->d : k/32 floats.
 *   x      : k floats, 16-byte aligned.  k % 32 == 0, 0 <= k <= INT32_MAX.
 * Several activation rows of K elements each are quantized by one call
 * with k = M * K (blocks never straddle rows because K % 32 == 0).
 * Sets out->n = k.  k == 0 enqueues nothing and accepts null data
 * pointers (out itself must not be null).
 * ------------------------------------------------------------------------- */
qmv_status qmv_quantize_q8(qmv_qact *out, const float *x, int64_t k, void *stream);

/* ---------------------------------------------------------------------------
 * qmv_quantize_weights -- quantize a row-major float32 matrix w
 * (W->rows x W->cols, 16-byte aligned) into W's format.
 *   QMV_Q8_0 : the Q8_0 rule above (the same rule the spec applies to Q8_0
 *              weights and activations);
 *   QMV_Q4_0 : the spec fixes only the Q4_0 storage and that quantization is
 *              symmetric; this library's rule is the Q8_0 rule with 7 in
 *              place of 127 (d = amax / 7, value = clamp(trunc(x * (7 / amax)
 *              + copysign(0.5, x)), -8, 7), nibble = value + 8).
 * ------------------------------------------------------------------------- */
qmv_status qmv_quantize_weights(const qmv_qtensor *W, const float *w, void *stream);

/* ---------------------------------------------------------------------------
 * qmv_matvec_q8 / qmv_matvec_q4 -- y[r] = sum_b sumi(r, b) * dw(r, b) *
 * dx(b) for r in [r0, r1) (spec section 5, ml_k_matvec_q8 / _q4: rows
 * [r0, r1), the caller splits rows).
 *   y : W->rows floats indexed by the absolute row r; entries outside
 *       [r0, r1) are not written.
 *   W : type QMV_Q8_0 (resp. QMV_Q4_0).  x : Q8_0 activation, x->n == W->cols.
 *   0 <= r0 <= r1 <= W->rows; r0 == r1 enqueues nothing.
 *   Limit: K <= 131072 (QMV_LDS_BYTES).
 * ------------------------------------------------------------------------- */
qmv_status qmv_matvec_q8(float *y, const qmv_qtensor *W, const qmv_qact *x,
                         int32_t r0, int32_t r1, void *stream);
qmv_status qmv_matvec_q4(float *y, const qmv_qtensor *W, const qmv_qact *x,
                         int32_t r0, int32_t r1, void *stream);

/* ---------------------------------------------------------------------------
 * qmv_matvec_q8_fx / qmv_matvec_q4_fx -- the same product from a float32
 * activation x (W->cols floats, 16-byte aligned): the activation is
 * quantized to Q8_0 inside the kernel (the rule of qmv_quantize_q8, the
 * same bits) and never leaves the chip (limit: K <= 30720, the LDS budget
 * with the float32 activation staged).  If xq is not NULL, xq->q (W->cols
 * bytes) and xq->d (W->cols / 32 floats) also receive the quantized
 * activation and xq->n is set to W->cols.
 * ------------------------------------------------------------------------- */
qmv_status qmv_matvec_q8_fx(float *y, const qmv_qtensor *W, const float *x,
                            qmv_qact *xq, int32_t r0, int32_t r1, void *stream);
qmv_status qmv_matvec_q4_fx(float *y, const qmv_qtensor *W, const float *x,
                            qmv_qact *xq, int32_t r0, int32_t r1, void *stream);

/* ---------------------------------------------------------------------------
 * qmv_matvec_q8_fx_rmsnorm / qmv_matvec_q4_fx_rmsnorm -- the fused product
 * with the root-mean-square normalization that precedes every quantization
 * of a layer input in the spec's forward pass (section 6: h = rmsnorm(x);
 * qa = quantize_q8(h); ... = matvec(W, qa)), all in one launch:
 *   h_j = w_norm_j * (inv * x_j),  inv = 1 / sqrt(ss / K + eps),
 *   ss  = sum of x_j^2 (section 5 lists ml_k_rmsnorm(o, x, w, n, eps); the
 *         formula is the llama2.c one the spec follows elsewhere),
 * then h is quantized to Q8_0 (the qmv_quantize_q8 rule) and multiplied as
 * in qmv_matvec_q8_fx.  ss is summed pairwise: the 32 squares of each
 * 32-element block by recursive halving, then the block sums by recursive
 * halving over their count padded to a power of two with zeros.  Every
 * float operation is rounded on its own (no contraction; correctly rounded
 * division and square root), so the quantized h is bit-identical to that
 * definition evaluated on any IEEE binary32 machine.
 *   x, w_norm : W->cols floats each, 16-byte aligned, device memory.
 *   eps       : finite and >= 0 (QMV_E_ARG otherwise); with eps = 0 an
 *               all-zero x gives a non-finite inv (the caller's choice).
 *   xq        : NULL, or receives the quantized h (as in qmv_matvec_*_fx).
 *   K <= 30208 (the LDS budget; QMV_E_SHAPE beyond).
 *   Rows, y indexing and errors otherwise as qmv_matvec_q8_fx.
 * ------------------------------------------------------------------------- */
qmv_status qmv_matvec_q8_fx_rmsnorm(float *y, const qmv_qtensor *W, const float *x,
                                    const float *w_norm, float eps, qmv_qact *xq,
                                    int32_t r0, int32_t r1, void *stream);
qmv_status qmv_matvec_q4_fx_rmsnorm(float *y, const qmv_qtensor *W, const float *x,
                                    const float *w_norm, float eps, qmv_qact *xq,
                                    int32_t r0, int32_t r1, void *stream);

/* ---------------------------------------------------------------------------
 * qmv_matvec_q8_fx_silu_mul / qmv_matvec_q4_fx_silu_mul -- the fused product
 * whose activation is the FFN gate of the spec's forward pass (section 6:
 * silu_mul(g, u); x += matvec(W2, quantize_q8(g)); section 5 lists
 * ml_k_silu_mul(g, u, n): g = silu(g) * u), all in one launch:
 *   a_j = (g_j * (1 / (1 + exp(-g_j)))) * u_j,
 * each operation rounded on its own, then a is quantized to Q8_0 (the
 * qmv_quantize_q8 rule) and multiplied as in qmv_matvec_q8_fx.  exp is the
 * device math library's single-precision exp (a few ulp); the spec allows
 * its SIMD exp a relative error of 1e-6, so codes may differ by one from a
 * host evaluation where a * 127 / amax falls that close to a rounding
 * boundary.
 *   g, u : W->cols floats each, 16-byte aligned, device memory (they may be
 *          the two halves of one concatenated W1|W3 output).
 *   xq   : NULL, or receives the quantized a.
 *   K <= 30720, as qmv_matvec_q8_fx.
 *   Rows, y indexing and errors otherwise as qmv_matvec_q8_fx.
 * ------------------------------------------------------------------------- */
qmv_status qmv_matvec_q8_fx_silu_mul(float *y, const qmv_qtensor *W, const float *g,
                                     const float *u, qmv_qact *xq, int32_t r0, int32_t r1,
                                     void *stream);
qmv_status qmv_matvec_q4_fx_silu_mul(float *y, const qmv_qtensor *W, const float *g,
                                     const float *u, qmv_qact *xq, int32_t r0, int32_t r1,
                                     void *stream);

/* ---------------------------------------------------------------------------
 * qmv_matvec_q8_fx_swiglu / qmv_matvec_q4_fx_swiglu -- the FFN's first half
 * of a decode step in one launch (spec section 6: h = rmsnorm(x); qa =
 * quantize_q8(h); g = matvec(W1, qa); u = matvec(W3, qa); silu_mul(g, u)),
 * with W1 and W3 stacked as one matrix: W->rows = 2 F, rows 0 .. F - 1 the
 * gate W1 and rows F .. 2 F - 1 the up projection W3.  For pairs p0 <= j <
 * p1 (0 <= p0 <= p1 <= F):
 *   y[j] = (W h)[j],  y[F + j] = (W h)[F + j]   (as qmv_matvec_q8_fx, or
 *                                                 _fx_rmsnorm when w_norm)
 *   a[j] = (y[j] * (1 / (1 + exp(-y[j])))) * y[F + j]   (qmv_silu_mul's
 *          evaluation, so a is bit-identical to qmv_silu_mul on this y).
 * h = x when w_norm is NULL, else rmsnorm(x) * w_norm with eps as in
 * qmv_matvec_q8_fx_rmsnorm.  y has W->rows floats and a has F floats, both
 * indexed by absolute row (4-byte aligned); other entries are not written.
 * For 64 <= K / 32 <= 512 both halves and the gate come from one launch
 * (each workgroup takes a run of pairs, both of its rows' slices); for
 * other K the two halves run as the plain fused products and the gate as
 * a launch of its own (same bits).  W->rows odd or the pair range outside
 * [0, F] is QMV_E_SHAPE; other arguments and errors as qmv_matvec_q8_fx.
 * ------------------------------------------------------------------------- */
qmv_status qmv_matvec_q8_fx_swiglu(float *a, float *y, const qmv_qtensor *W, const float *x,
                                   const float *w_norm, float eps, qmv_qact *xq,
                                   int32_t p0, int32_t p1, void *stream);
qmv_status qmv_matvec_q4_fx_swiglu(float *a, float *y, const qmv_qtensor *W, const float *x,
                                   const float *w_norm, float eps, qmv_qact *xq,
                                   int32_t p0, int32_t p1, void *stream);

/* ---------------------------------------------------------------------------
 * The two neighbours as launches of their own (spec section 5 kernel list:
 * ml_k_rmsnorm(o, x, w, n, eps), ml_k_silu_mul(g, u, n)).  They evaluate
 * the same device functions, in the same order, as the fused activation
 * forms above, so e.g. qmv_rmsnorm then qmv_matvec_q4_fx gives the same bits
 * as qmv_matvec_q4_fx_rmsnorm (one launch more).
 *
 * qmv_rmsnorm: o_j = w_j * (inv * x_j), inv = 1 / sqrt(ss / n + eps), ss
 *   summed as qmv_matvec_q8_fx_rmsnorm states (pairwise within each
 *   32-element block, then pairwise over the zero-padded block sums).
 *   o, x, w: n floats each, device memory, 16-byte aligned; o may equal x.
 *   0 < n <= 131072, n % 32 == 0 (QMV_E_SHAPE otherwise); eps finite and
 *   >= 0 (QMV_E_ARG otherwise).  Runs as one workgroup.
 * qmv_silu_mul: o_j = (g_j * (1 / (1 + exp(-g_j)))) * u_j with the exp and
 *   reciprocal of qmv_matvec_q8_fx_silu_mul.  o, g, u: n floats each,
 *   device memory, 16-byte aligned; o may equal g or u.  0 <= n <=
 *   INT32_MAX; n == 0 enqueues nothing and accepts null pointers.
 * ------------------------------------------------------------------------- */
qmv_status qmv_rmsnorm(float *o, const float *x, const float *w, int64_t n, float eps, void *stream);
qmv_status qmv_silu_mul(float *o, const float *g, const float *u, int64_t n, void *stream);

/* ---------------------------------------------------------------------------
 * qmv_gemm_q8 / qmv_gemm_q4 -- the product for M activation rows at once:
 * X is a Q8_0 qmv_qtensor with X->rows = M, X->cols = W->cols, each row
 * quantized on its own; Y is M x W->rows row-major and
 *   Y[m * W->rows + r] = sum_b sumi(m, r, b) * dw(r, b) * dx(m, b)
 * for every m < M and r in [r0, r1); other entries are not written.
 * The spec defines the single-row product; this applies it to each row of
 * X while every weight byte is read from memory once per pass.
 *   1 <= M <= 8: the dot-product path, all M rows in one pass over the
 *   weights.
 *   M > 8: the int8 matrix-core path, one v_mfma instruction per 32-element
 *   block and tile, up to 64 activation rows per pass over the weights
 *   (ceil(M / 64) passes).
 *   Limits: M * K <= 131072 for M <= 8 (QMV_LDS_BYTES), K <= 131072 for
 *   M > 8.  Y must be 4-byte aligned, X->q 16-byte aligned.  The passes
 *   of one call are ordered on the stream; each output is written once.
 * ------------------------------------------------------------------------- */
qmv_status qmv_gemm_q8(float *Y, const qmv_qtensor *W, const qmv_qtensor *X,
                       int32_t r0, int32_t r1, void *stream);
qmv_status qmv_gemm_q4(float *Y, const qmv_qtensor *W, const qmv_qtensor *X,
                       int32_t r0, int32_t r1, void *stream);

/* ---------------------------------------------------------------------------
 * Exported-model format: 128-element blocks with a zero point ("ONNX
 * Runtime" page, section 3 "Match real exports -- BlkLen=128 CompInt8" and
 * section 4 "SQ8Bit").  A weight is (code - zp) * scale:
 *   q  : codes, rows x cols bytes (bits = 8) or rows x cols/2 bytes
 *        (bits = 4: element 2i in the low nibble of byte i, 2i + 1 in the
 *        high nibble), row-major, 16-byte aligned;
 *   d  : rows x cols/128 float32 scales, row-major, 4-byte aligned;
 *   zp : rows x cols/128 zero points, one byte each (for bits = 4 only the
 *        values 0..15 make sense, but any byte is taken as given), or NULL
 *        for the midpoint 2^(bits-1) (128 or 8).
 * ------------------------------------------------------------------------- */
#define QMV_ZP_BLOCK 128
#define QMV_ZP_MAX_COLS 65536

typedef struct {
    uint8_t *q;
    float *d;
    uint8_t *zp;
    int32_t rows;
    int32_t cols;
    uint8_t bits;      /* 4 or 8 */
} qmv_zptensor;

/* The Q8_0 rule of qmv_quantize_q8 applied to 128-element blocks (the
 * activation format of this product): out->q = k bytes, out->d = k/128
 * floats.  k % 128 == 0; otherwise as qmv_quantize_q8. */
qmv_status qmv_quantize_q8_b128(qmv_qact *out, const float *x, int64_t k, void *stream);

/* y[r] = sum over 128-element blocks b of sumi(r, b) * d(r, b) * dx(b) for r
 * in [r0, r1), sumi = sum over the block of (code - zp) * q exact in int32,
 * with (q, dx) the 128-block Q8_0 quantization of the float32 activation x
 * (W->cols floats, 16-byte aligned), done inside the kernel.  If xq is not
 * NULL it receives that quantized activation (q: cols bytes, 16-byte
 * aligned; d: cols/128 floats) and xq->n = cols.  Other entries of y are not
 * written.  Limits: cols % 128 == 0, cols <= QMV_ZP_MAX_COLS, rows * (bytes
 * per row) <= INT32_MAX.  Errors: QMV_E_ARG (null or misaligned pointers),
 * QMV_E_FORMAT (bits not 4 or 8), QMV_E_SHAPE (sizes, row range). */
qmv_status qmv_matvec_zp_fx(float *y, const qmv_zptensor *W, const float *x, qmv_qact *xq,
                            int32_t r0, int32_t r1, void *stream);

/* ---------------------------------------------------------------------------
 * K-quant super-blocks with the sub-block scales folded in the integer
 * domain ("SKaiNET-native-kernels" page, section "Proving an optimization
 * is safe before writing it": 4-bit weights, a 6-bit scale per 32 elements,
 * 8 sub-blocks per block, int8 activations; section "Accomplishments":
 * per-32 asymmetric minima).  The page gives neither the storage nor the
 * scale types; this library's reading: element i of sub-block b of
 * super-block k of a row has the value d[k] * sc[b] * w_i - dmin[k] * mn[b]:
 *   q    : rows x cols/2 bytes, 16 per 32-element sub-block in the Q4_0
 *          order (element j in the low nibble of byte j, element j + 16 in
 *          the high nibble), w_i the nibble as stored; 16-byte aligned;
 *   sc,mn: rows x cols/32 bytes, the sub-block scale and minimum (0..63);
 *   d,dmin: rows x cols/256 float32 (4-byte aligned).
 * All row-major.  Matrices with rows = 0 may have null pointers.
 * ------------------------------------------------------------------------- */
#define QMV_Q4K_BLOCK 256
#define QMV_Q4K_MAX_COLS 65536

typedef struct {
    uint8_t *q;
    uint8_t *sc;
    uint8_t *mn;
    float *d;
    float *dmin;
    int32_t rows;
    int32_t cols;
} qmv_q4ktensor;

/* The Q8_0 rule of qmv_quantize_q8 applied to 256-element blocks (the
 * activation format of the K-quant product): out->q = k bytes, out->d =
 * k/256 floats.  k % 256 == 0; otherwise as qmv_quantize_q8. */
qmv_status qmv_quantize_q8_b256(qmv_qact *out, const float *x, int64_t k, void *stream);

/* y[r] for r in [r0, r1): per super-block, S1 = sum_b sc_b * (sum_i w_i q_i)
 * and S2 = sum_b mn_b * (sum_i q_i), exact in int32 (|S1| <= 8*63*32*127*15,
 * the page's bound), and y[r] = sum over super-blocks of (S1 * d - S2 * dmin)
 * * dx in float32, with (q, dx) the 256-block Q8_0 quantization of the
 * float32 activation x (W->cols floats, 16-byte aligned) done inside the
 * kernel.  If xq is not NULL it receives that quantized activation
 * (q: cols bytes, 16-byte aligned; d: cols/256 floats) and xq->n = cols.
 * Other entries of y are not written.  Limits: cols % 256 == 0,
 * cols <= QMV_Q4K_MAX_COLS, rows * cols / 2 <= INT32_MAX.  Errors:
 * QMV_E_ARG (null or misaligned pointers), QMV_E_SHAPE (sizes, row range). */
qmv_status qmv_matvec_q4k_fx(float *y, const qmv_q4ktensor *W, const float *x, qmv_qact *xq,
                             int32_t r0, int32_t r1, void *stream);

/* ---------------------------------------------------------------------------
 * Pack-once weight layout for the matrix-core product.  The spec stores
 * weights row-major (section 4 table); its companion write-ups on
 * block-quantized products re-lay the weights once, ahead of time, into the
 * order the multiply instruction consumes them.  Here the unit is a tile of
 * 16 weight rows by 4 blocks (128 elements), units of one tile consecutive
 * (nq = ceil(cols / 128) of them), tiles in row order:
 *   q of unit u = T * nq + Q (tile T, block quad Q): 1024 bytes (Q4_0) or
 *     2048 bytes (Q8_0) at u * 1024 or u * 2048.  Lane l = 16 g + i (row
 *     16 T + i, elements 8 g .. 8 g + 7 of each block) owns, for block
 *     4 Q + b, Q4_0: the 4 bytes at 16 l + 4 b, byte j holding element
 *     8 g + j in its low nibble and 8 g + 4 + j in its high nibble (nibble =
 *     value + 8, as stored); Q8_0: the 8 bytes at 1024 (b / 2) + 16 l +
 *     8 (b % 2), elements 8 g .. 8 g + 7.
 *   d of unit u: 64 floats at 64 u, row 16 T + r and block 4 Q + b at 4 r + b.
 * Rows past the matrix and blocks past cols hold value 0 and scale 0.
 * Packing is a permutation of the stored bytes and scales; the packed
 * product computes the same sums in the same order as qmv_gemm_* on the
 * row-major weights for M > 8, so the two give the same bits.
 * ------------------------------------------------------------------------- */
typedef struct {
    void *q;           /* packed quants, 16-byte aligned */
    float *d;          /* packed scales, 16-byte aligned */
    int32_t rows;      /* set by qmv_pack_weights */
    int32_t cols;
    uint8_t type;      /* QMV_Q4_0 or QMV_Q8_0 */
} qmv_packed;

/* Bytes the packed form of a type x rows x cols matrix needs: q_bytes =
 * ceil(rows / 16) * ceil(cols / 128) * (1024 or 2048), d_bytes =
 * ceil(rows / 16) * ceil(cols / 128) * 256.  Host only (no device call).
 * Errors: QMV_E_ARG (null outputs), QMV_E_FORMAT (type), QMV_E_SHAPE
 * (rows < 0, cols <= 0, cols % 32 != 0 or cols > 131072). */
qmv_status qmv_pack_bytes(int32_t type, int32_t rows, int32_t cols, int64_t *q_bytes, int64_t *d_bytes);

/* Writes W (row-major, as qmv_quantize_weights leaves it) into P->q / P->d
 * (caller-allocated, sizes from qmv_pack_bytes) in the layout above, and
 * sets P->rows, P->cols and P->type from W.  Enqueued on stream; W is
 * unchanged.  Errors as qmv_quantize_weights, plus QMV_E_ARG for a null or
 * misaligned P->q / P->d and QMV_E_SHAPE for cols > 131072. */
qmv_status qmv_pack_weights(qmv_packed *P, const qmv_qtensor *W, void *stream);

/* The product of qmv_gemm_q8 / qmv_gemm_q4 on packed weights, on the
 * matrix-core path for every M >= 1 (for M <= 8 the row-major call's
 * dot-product path reads the weights at a higher rate).  r0 must be a
 * multiple of 16 (r1 is free).  Y, X, limits and errors as qmv_gemm_*, with
 * QMV_E_FORMAT when P->type is not the call's type. */
qmv_status qmv_gemm_q8_packed(float *Y, const qmv_packed *P, const qmv_qtensor *X,
                              int32_t r0, int32_t r1, void *stream);
qmv_status qmv_gemm_q4_packed(float *Y, const qmv_packed *P, const qmv_qtensor *X,
                              int32_t r0, int32_t r1, void *stream);

/* ---------------------------------------------------------------------------
 * Measurement helpers (not on the product path).  The bench divides each
 * kernel's rate by what these reach on the same chip: the rate at which a
 * plain kernel streams device memory (the "ONNX Runtime" page, "How we got
 * there" item 1, sets its kernel against a STREAM floor; the
 * "SKaiNET-native-kernels" page measures effective weight bandwidth as
 * bytes over time) and the rate of the int8 matrix-core instructions with
 * their operands in registers.
 *
 * qmv_ceiling_stream_read: reads `bytes` (a multiple of 16, at least 16) of
 *   buf (device memory, 16-byte aligned) with `workgroups` (1 .. 65536)
 *   workgroups of 1024 threads in rounds: in each round every thread issues
 *   `depth` (4 or 8) 16-byte non-temporal loads (consecutive threads read
 *   consecutive 16-byte pieces; the round covers depth x threads pieces)
 *   before using any.  sink[w] (workgroups uint32 of device memory) receives the XOR
 *   of the 32-bit words workgroup w read, so the XOR over all of sink is the
 *   XOR of every 32-bit word of buf.
 * qmv_ceiling_mfma_i8: `workgroups` (1 .. 65536) workgroups of 4
 *   wavefronts; each wavefront runs 4 independent chains of `iters` (>= 0)
 *   instructions of one shape (0: v_mfma_i32_16x16x32_i8, 1:
 *   v_mfma_i32_16x16x64_i8, 2: v_mfma_i32_32x32x32_i8) on operands whose
 *   bytes are all a (the A operand) and all b (B), as signed bytes.  Every
 *   result element ends at iters * kdepth * a * b (kdepth = 32, 64, 32), and
 *   sink[4 w + v] (4 * workgroups uint32 of device memory) receives the sum
 *   modulo 2^32 of the 4 chains' elements of wavefront v of workgroup w:
 *   4 * E * iters * kdepth * a * b with E = 256 (16 x 16 shapes) or 1024
 *   (32 x 32).  Each launch performs workgroups * 16 * iters * 2 * E *
 *   kdepth integer operations.
 * Errors: QMV_E_ARG (null or misaligned pointers, depth or shape out of
 * range), QMV_E_SHAPE (sizes out of range), then the device checks.
 * ------------------------------------------------------------------------- */
qmv_status qmv_ceiling_stream_read(uint32_t *sink, const void *buf, int64_t bytes, int32_t workgroups,
                                   int32_t depth, void *stream);
qmv_status qmv_ceiling_mfma_i8(uint32_t *sink, int32_t shape, int32_t iters, int32_t workgroups, int32_t a,
                               int32_t b, void *stream);

/* Text of a status code (static storage). */
const char *qmv_status_str(qmv_status s);

/* Name of the kernel variant the calling thread's last successful call
 * enqueued ("" before any); with the environment variable QMV_DIAG=1 every
 * launch is also printed to stderr.  The string is thread-local and valid
 * until the thread's next call. */
const char *qmv_last_kernel(void);

/* Checks that the current HIP device is usable and is a gfx950, caching the
 * answer per device (every call does this on its own; this entry point
 * lets a caller check up front).  Returns QMV_OK, QMV_E_DEVICE or
 * QMV_E_ARCH. */
qmv_status qmv_device_check(void);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
