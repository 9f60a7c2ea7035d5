/*
 * qmv_oracle.c -- plain, slow, obviously-correct CPU oracle for the
 * block-quantized weight x activation product of LLM decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no source, header, table or helper with
 * the HIP library; the only thing the two have in common is the byte layout
 * of the formats, which both take from the design spec below.
 *
 * Source of every rule here: "Legacy-ISA ML Inference Runtime -- Design
 * Spec" (jonpark0.github.io/krafla), sections 4 (Quantization Formats),
 * 5 (Kernel Interface) and 7 (Testing, Verification, Benchmarks).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math (no FMA is ever
 * formed; every float operation rounds to nearest-even in binary32).
 *
 * Parity status per function (what pins it is listed in the test suite):
 *   orc_quantize_q8     pinned (closed forms, detector vectors, invariants,
 *                       textbook rounding at unit scale, round-trip bound)
 *   orc_quantize_q4     pinned (nibble layout, closed forms, round-trip)
 *   orc_block_sums_*    pinned (closed forms, int64 brute force)
 *   orc_matvec_*        pinned (fp64 brute force within the error bound,
 *                       exact sums at unit scale, sign/power-of-two/row
 *                       permutation invariants); its individual fp32
 *                       roundings are defined only by this order of
 *                       operations: "parity unpinned" beyond the bound.
 *   orc_gemm_*          pinned (M=1 slice and per-row equality with matvec)
 *   orc_tol_abs         pinned (closed forms)
 *   orc_sumsq           pinned (a hand-derived pairwise sum that a left-to-
 *                       right sum would not give, exact integer sums)
 *   orc_rmsnorm         pinned (closed forms at constant input, sign and
 *                       power-of-two invariants, fp64 brute force)
 *   orc_silu_mul        pinned (closed forms at 0 and at saturation, the
 *                       identity silu(g) - silu(-g) = g, fp64 brute force)
 *   orc_quantize_q8_b128  pinned (equal to orc_quantize_q8 where each
 *                       128-block's four 32-blocks share one maximum;
 *                       closed forms; one scale per 128 elements)
 *   orc_block_sums_zp   pinned (closed forms at the code extremes, the
 *                       nibble order by one-hot activations, reduction to
 *                       the Q8_0 / Q4_0 sums at the default zero point,
 *                       int64 brute force)
 *   orc_matvec_zp       pinned (fp64 brute force within the error bound,
 *                       exact sums at unit scales, reduction to the
 *                       symmetric formats)
 *   orc_tol_abs_zp      pinned (closed forms)
 *
 *   orc_quantize_q8_b256  pinned (equal to orc_quantize_q8 where each
 *                       256-block's 32-blocks share one maximum; one scale
 *                       per 256 elements)
 *   orc_superblock_sums_q4k  pinned (the page's own bound 8*63*32*127*15 at
 *                       the extremes, the nibble layout by one-hot
 *                       activations, reduction to the Q4_0 sums, int64
 *                       brute force)
 *   orc_matvec_q4k      pinned (fp64 brute force within the error bound,
 *                       exact at unit scales)
 *   orc_tol_abs_q4k     pinned (fp64 brute force)
 *
 * The K-quant super-block functions (orc_*_q4k, orc_quantize_q8_b256)
 * follow "SKaiNET-native-kernels" (devpost.com), sections "Proving an
 * optimization is safe before writing it" and "Accomplishments that we're
 * proud of".
 *
 * The zero-point format (the orc_*_zp functions) follows a second page:
 * "ONNX Runtime" (opensolvers.com/apps/onnx.html), sections 3 (BlkLen=128
 * CompInt8) and 4 (SQ8Bit: B' = B - 128, block sums scaled by
 * -scale * (zp - 128), zp = 128 when the export gives none).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QK 32 /* block length, spec section 4 */

/* ------------------------------------------------------------------------
 * Q8_0 quantization (spec section 4 "Q8 quantization" bullet, and the
 * section 5 rounding rule).  Per block of 32 consecutive values:
 *   amax = max |x_i|,   d = amax / 127,   id = 127 / amax  (0 when amax=0),
 *   q_i  = trunc(x_i * id + copysign(0.5, x_i))   (half away from zero),
 *   q_i clamped to [-127, 127];  amax = 0 gives d = 0 and every q_i = 0.
 * Each of the two float operations on x_i rounds separately (contraction
 * is off for this translation unit).  n must be a multiple of 32.
 * ---------------------------------------------------------------------- */
void orc_quantize_q8(const float *x, int64_t n, int8_t *q, float *d)
{
    for (int64_t b = 0; b < n / QK; ++b) {
        const float *xb = x + b * QK;
        float amax = 0.0f;
        for (int i = 0; i < QK; ++i) {
            float a = fabsf(xb[i]);
            if (a > amax)
                amax = a;
        }
        float db = amax / 127.0f;
        float id = (amax != 0.0f) ? 127.0f / amax : 0.0f;
        for (int i = 0; i < QK; ++i) {
            float v = xb[i] * id;
            float t = v + copysignf(0.5f, xb[i]);
            int qi = (int)truncf(t);
            if (qi > 127)
                qi = 127;
            if (qi < -127)
                qi = -127;
            q[b * QK + i] = (int8_t)qi;
        }
        d[b] = db;
    }
}

/* ------------------------------------------------------------------------
 * Q4_0 quantization of weights.  The spec fixes only the storage (section
 * 4 table: 16 bytes per block, byte j holds element j in its low nibble and
 * element j+16 in its high nibble, value = nibble - 8 in [-8, 7]) and that
 * quantization is symmetric.  The plain symmetric reading used here mirrors
 * the Q8_0 rule with 7 in place of 127:
 *   d = amax / 7,  id = 7 / amax (0 when amax = 0),
 *   v_i = clamp(trunc(x_i * id + copysign(0.5, x_i)), -8, 7),
 *   nibble_i = v_i + 8.
 * q receives n/2 bytes, d receives n/32 scales.
 * ---------------------------------------------------------------------- */
void orc_quantize_q4(const float *x, int64_t n, uint8_t *q, float *d)
{
    for (int64_t b = 0; b < n / QK; ++b) {
        const float *xb = x + b * QK;
        float amax = 0.0f;
        for (int i = 0; i < QK; ++i) {
            float a = fabsf(xb[i]);
            if (a > amax)
                amax = a;
        }
        float db = amax / 7.0f;
        float id = (amax != 0.0f) ? 7.0f / amax : 0.0f;
        int nib[QK];
        for (int i = 0; i < QK; ++i) {
            float v = xb[i] * id;
            float t = v + copysignf(0.5f, xb[i]);
            int qi = (int)truncf(t);
            if (qi > 7)
                qi = 7;
            if (qi < -8)
                qi = -8;
            nib[i] = qi + 8;
        }
        for (int j = 0; j < QK / 2; ++j)
            q[b * (QK / 2) + j] = (uint8_t)(nib[j] | (nib[j + QK / 2] << 4));
        d[b] = db;
    }
}

/* Weight element i (0..31) of a Q4_0 block, as a signed value (section 4
 * table and the section 5 note on Q4 kernels: mask 0x0F / shift 4, then
 * subtract 8). */
static int q4_elem(const uint8_t *blk, int i)
{
    int nib = (i < QK / 2) ? (blk[i] & 0x0F) : (blk[i - QK / 2] >> 4);
    return nib - 8;
}

/* ------------------------------------------------------------------------
 * Integer block dot products (section 4 "Integer dot per block"):
 *   sumi(r, b) = sum over i < 32 of w(r, 32b+i) * qx(32b+i), in int32.
 * out has (r1 - r0) * nb entries, row-major, nb = cols / 32.
 * ---------------------------------------------------------------------- */
void orc_block_sums_q8(const int8_t *wq, int32_t cols, const int8_t *xq,
                       int32_t r0, int32_t r1, int32_t *out)
{
    int32_t nb = cols / QK;
    for (int32_t r = r0; r < r1; ++r)
        for (int32_t b = 0; b < nb; ++b) {
            const int8_t *w = wq + (int64_t)r * cols + (int64_t)b * QK;
            const int8_t *xv = xq + (int64_t)b * QK;
            int32_t s = 0;
            for (int i = 0; i < QK; ++i)
                s += (int32_t)w[i] * (int32_t)xv[i];
            out[(int64_t)(r - r0) * nb + b] = s;
        }
}

void orc_block_sums_q4(const uint8_t *wq, int32_t cols, const int8_t *xq,
                       int32_t r0, int32_t r1, int32_t *out)
{
    int32_t nb = cols / QK;
    for (int32_t r = r0; r < r1; ++r)
        for (int32_t b = 0; b < nb; ++b) {
            const uint8_t *blk = wq + (int64_t)r * (cols / 2) + (int64_t)b * (QK / 2);
            const int8_t *xv = xq + (int64_t)b * QK;
            int32_t s = 0;
            for (int i = 0; i < QK; ++i)
                s += (int32_t)q4_elem(blk, i) * (int32_t)xv[i];
            out[(int64_t)(r - r0) * nb + b] = s;
        }
}

/* ------------------------------------------------------------------------
 * Matrix-vector product (section 5 kernel interface: rows [r0, r1) of W
 * times the Q8_0 activation; section 4 accumulation rule):
 *   s = 0;  for each block b in ascending order:
 *       s = s + ((float)sumi * dw[r, b]) * dx[b]
 *   y[r] = s            (y is indexed by the absolute row r)
 * Rows outside [r0, r1) are not written.
 * ---------------------------------------------------------------------- */
static float row_q8(const int8_t *wq, const float *wd, int32_t cols,
                    const int8_t *xq, const float *xd, int32_t r)
{
    int32_t nb = cols / QK;
    float s = 0.0f;
    for (int32_t b = 0; b < nb; ++b) {
        const int8_t *w = wq + (int64_t)r * cols + (int64_t)b * QK;
        const int8_t *xv = xq + (int64_t)b * QK;
        int32_t sumi = 0;
        for (int i = 0; i < QK; ++i)
            sumi += (int32_t)w[i] * (int32_t)xv[i];
        float t = (float)sumi * wd[(int64_t)r * nb + b];
        t = t * xd[b];
        s = s + t;
    }
    return s;
}

static float row_q4(const uint8_t *wq, const float *wd, int32_t cols,
                    const int8_t *xq, const float *xd, int32_t r)
{
    int32_t nb = cols / QK;
    float s = 0.0f;
    for (int32_t b = 0; b < nb; ++b) {
        const uint8_t *blk = wq + (int64_t)r * (cols / 2) + (int64_t)b * (QK / 2);
        const int8_t *xv = xq + (int64_t)b * QK;
        int32_t sumi = 0;
        for (int i = 0; i < QK; ++i)
            sumi += (int32_t)q4_elem(blk, i) * (int32_t)xv[i];
        float t = (float)sumi * wd[(int64_t)r * nb + b];
        t = t * xd[b];
        s = s + t;
    }
    return s;
}

void orc_matvec_q8(float *y, const int8_t *wq, const float *wd, int32_t cols,
                   const int8_t *xq, const float *xd, int32_t r0, int32_t r1)
{
    for (int32_t r = r0; r < r1; ++r)
        y[r] = row_q8(wq, wd, cols, xq, xd, r);
}

void orc_matvec_q4(float *y, const uint8_t *wq, const float *wd, int32_t cols,
                   const int8_t *xq, const float *xd, int32_t r0, int32_t r1)
{
    for (int32_t r = r0; r < r1; ++r)
        y[r] = row_q4(wq, wd, cols, xq, xd, r);
}

/* ------------------------------------------------------------------------
 * Several activation rows at once: X is M rows of Q8_0 (each row quantized
 * on its own, cols/32 scales per row); Y[m * rows + r] is the matvec of row
 * m of X, for r in [r0, r1).  The spec defines the single-row product only;
 * this is that product applied to each row of X.
 * ---------------------------------------------------------------------- */
void orc_gemm_q8(float *Y, const int8_t *wq, const float *wd, int32_t rows,
                 int32_t cols, const int8_t *xq, const float *xd, int32_t m,
                 int32_t r0, int32_t r1)
{
    int32_t nb = cols / QK;
    for (int32_t i = 0; i < m; ++i)
        orc_matvec_q8(Y + (int64_t)i * rows, wq, wd, cols,
                      xq + (int64_t)i * cols, xd + (int64_t)i * nb, r0, r1);
}

void orc_gemm_q4(float *Y, const uint8_t *wq, const float *wd, int32_t rows,
                 int32_t cols, const int8_t *xq, const float *xd, int32_t m,
                 int32_t r0, int32_t r1)
{
    int32_t nb = cols / QK;
    for (int32_t i = 0; i < m; ++i)
        orc_matvec_q4(Y + (int64_t)i * rows, wq, wd, cols,
                      xq + (int64_t)i * cols, xd + (int64_t)i * nb, r0, r1);
}

/* ------------------------------------------------------------------------
 * Tolerance aid: A(r) = sum over blocks of |sumi * dw * dx| in binary64,
 * the scale against which an fp32 result of any summation order is judged
 * (|y - y_ref| <= 1e-5 * A + 1e-6).  type is 8 (Q8_0) or 4 (Q4_0).
 * out[r - r0] receives A(r).
 * ---------------------------------------------------------------------- */
void orc_tol_abs(int type, const void *wq, const float *wd, int32_t cols,
                 const int8_t *xq, const float *xd, int32_t r0, int32_t r1,
                 double *out)
{
    int32_t nb = cols / QK;
    for (int32_t r = r0; r < r1; ++r) {
        double a = 0.0;
        for (int32_t b = 0; b < nb; ++b) {
            const int8_t *xv = xq + (int64_t)b * QK;
            int64_t sumi = 0;
            if (type == 8) {
                const int8_t *w = (const int8_t *)wq + (int64_t)r * cols + (int64_t)b * QK;
                for (int i = 0; i < QK; ++i)
                    sumi += (int64_t)w[i] * xv[i];
            } else {
                const uint8_t *blk = (const uint8_t *)wq + (int64_t)r * (cols / 2) + (int64_t)b * (QK / 2);
                for (int i = 0; i < QK; ++i)
                    sumi += (int64_t)q4_elem(blk, i) * xv[i];
            }
            a += fabs((double)sumi * (double)wd[(int64_t)r * nb + b] * (double)xd[b]);
        }
        out[r - r0] = a;
    }
}

/* ------------------------------------------------------------------------
 * Root-mean-square normalization ahead of a quantization (spec section 5
 * kernel list, ml_k_rmsnorm(o, x, w, n, eps); section 6 forward pass, where
 * every quantize_q8 of a layer input follows one).  The spec lists the
 * signature only; the formula read here is the llama2.c one the spec
 * follows elsewhere (section 5, RoPE bullet):
 *   ss = sum over j of x_j^2,  inv = 1 / sqrt(ss / n + eps),
 *   o_j = w_j * (inv * x_j).
 * The spec leaves the order of the sum open.  Read here: pairwise
 * summation (recursive halving) of the 32 squares of each 32-element block
 * of the Q8_0 format, then pairwise summation of the block sums with their
 * count padded to a power of two by zeros (adding a zero is exact, so the
 * padding changes no rounding).  Every float operation rounds to
 * nearest-even in binary32; sqrtf and the divisions are correctly rounded.
 * n must be a positive multiple of 32 (at most 2^24).
 * ---------------------------------------------------------------------- */
static float pairwise_sum(const float *v, int64_t n)  /* n a power of two */
{
    if (n == 1)
        return v[0];
    return pairwise_sum(v, n / 2) + pairwise_sum(v + n / 2, n / 2);
}

float orc_sumsq(const float *x, int64_t n)
{
    int64_t nb = n / QK, p = 1;
    while (p < nb)
        p *= 2;
    float *bs = calloc((size_t)p, sizeof(float));  /* zeros past nb */
    if (bs == NULL)
        return NAN;
    float sq[QK];
    for (int64_t b = 0; b < nb; ++b) {
        for (int i = 0; i < QK; ++i)
            sq[i] = x[b * QK + i] * x[b * QK + i];
        bs[b] = pairwise_sum(sq, QK);
    }
    float ss = pairwise_sum(bs, p);
    free(bs);
    return ss;
}

void orc_rmsnorm(float *o, const float *x, const float *w, int64_t n, float eps)
{
    float ss = orc_sumsq(x, n);
    float mean = ss / (float)n;
    float inv = 1.0f / sqrtf(mean + eps);
    for (int64_t j = 0; j < n; ++j)
        o[j] = w[j] * (inv * x[j]);
}

/* ------------------------------------------------------------------------
 * The FFN gate (spec section 5 kernel list, ml_k_silu_mul(g, u, n):
 * g = silu(g) * u; section 6 forward pass: silu_mul(g, u), then
 * quantize_q8(g) ahead of W2).  silu(v) = v * sigmoid(v), evaluated as the
 * llama2.c reference the spec follows: v * (1 / (1 + expf(-v))), then * u,
 * each float operation rounded on its own.  expf is the C library's (the
 * spec's scalar path; its SIMD paths use an exp with relative error at
 * most 1e-6, so results of this step are defined to that accuracy).
 * ---------------------------------------------------------------------- */
void orc_silu_mul(float *o, const float *g, const float *u, int64_t n)
{
    for (int64_t j = 0; j < n; ++j) {
        float v = g[j];
        float s = 1.0f / (1.0f + expf(-v));
        v = v * s;
        o[j] = v * u[j];
    }
}

/* ------------------------------------------------------------------------
 * Block length 128 with a zero point ("ONNX Runtime" page, sections 3 and
 * 4: the real exports use 128-element blocks; 8-bit weights are unsigned
 * codes B with a per-block zero point zp, the weight value being B - zp,
 * and the activation is quantized to int8 per block of the same length
 * (CompInt8)).
 *
 * Readings where the page is silent:
 *   - a weight value is (code - zp) * scale, fp32 scale per block; zp is one
 *     byte per block, and a missing zp array means the midpoint 2^(bits-1)
 *     (the page: zp = 128 when the export omits it; the same midpoint rule
 *     for 4 bits gives 8);
 *   - 4-bit codes: two per byte, element 2i in the low nibble of byte i and
 *     element 2i + 1 in the high nibble;
 *   - the activation rule is the spec's Q8_0 rule applied to 128-element
 *     blocks (one scale per 128 elements);
 *   - the accumulation is the spec's, per 128-element block:
 *       y[r] = sum over blocks, ascending, of ((float)sumi * dw) * dx,
 *       sumi = sum over the block of (code - zp) * q, exact in int32.
 * ---------------------------------------------------------------------- */
#define BL 128

void orc_quantize_q8_b128(const float *x, int64_t n, int8_t *q, float *d)
{
    for (int64_t b = 0; b < n / BL; ++b) {
        const float *xb = x + b * BL;
        float amax = 0.0f;
        for (int i = 0; i < BL; ++i) {
            float a = fabsf(xb[i]);
            if (a > amax)
                amax = a;
        }
        float db = amax / 127.0f;
        float id = (amax != 0.0f) ? 127.0f / amax : 0.0f;
        for (int i = 0; i < BL; ++i) {
            float v = xb[i] * id;
            float t = v + copysignf(0.5f, xb[i]);
            int qi = (int)truncf(t);
            if (qi > 127)
                qi = 127;
            if (qi < -127)
                qi = -127;
            q[b * BL + i] = (int8_t)qi;
        }
        d[b] = db;
    }
}

/* Code of element i of a row (bits 8: byte i; bits 4: see above). */
static int zp_code(const uint8_t *row, int bits, int64_t i)
{
    if (bits == 8)
        return row[i];
    uint8_t byte = row[i / 2];
    return (i % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
}

static int zp_of(const uint8_t *wzp, int bits, int32_t nb, int32_t r, int32_t b)
{
    if (wzp == 0)
        return 1 << (bits - 1);
    return wzp[(int64_t)r * nb + b];
}

static int32_t zp_block_sum(int bits, const uint8_t *wq, const uint8_t *wzp,
                            int32_t cols, const int8_t *xq, int32_t r, int32_t b)
{
    int32_t nb = cols / BL;
    const uint8_t *row = wq + (int64_t)r * (bits == 8 ? cols : cols / 2);
    int zp = zp_of(wzp, bits, nb, r, b);
    int32_t s = 0;
    for (int i = 0; i < BL; ++i) {
        int64_t e = (int64_t)b * BL + i;
        s += (int32_t)(zp_code(row, bits, e) - zp) * (int32_t)xq[e];
    }
    return s;
}

/* out has (r1 - r0) * (cols / 128) entries, row-major. */
void orc_block_sums_zp(int bits, const uint8_t *wq, const uint8_t *wzp, int32_t cols,
                       const int8_t *xq, int32_t r0, int32_t r1, int32_t *out)
{
    int32_t nb = cols / BL;
    for (int32_t r = r0; r < r1; ++r)
        for (int32_t b = 0; b < nb; ++b)
            out[(int64_t)(r - r0) * nb + b] = zp_block_sum(bits, wq, wzp, cols, xq, r, b);
}

void orc_matvec_zp(float *y, int bits, const uint8_t *wq, const float *wd,
                   const uint8_t *wzp, int32_t cols, const int8_t *xq,
                   const float *xd, int32_t r0, int32_t r1)
{
    int32_t nb = cols / BL;
    for (int32_t r = r0; r < r1; ++r) {
        float s = 0.0f;
        for (int32_t b = 0; b < nb; ++b) {
            int32_t sumi = zp_block_sum(bits, wq, wzp, cols, xq, r, b);
            float t = (float)sumi * wd[(int64_t)r * nb + b];
            t = t * xd[b];
            s = s + t;
        }
        y[r] = s;
    }
}

/* A(r) = sum over blocks of |sumi * dw * dx| in binary64 (the scale of the
 * tolerance |y - y_ref| <= 1e-5 * A + 1e-6). */
void orc_tol_abs_zp(int bits, const uint8_t *wq, const float *wd, const uint8_t *wzp,
                    int32_t cols, const int8_t *xq, const float *xd, int32_t r0,
                    int32_t r1, double *out)
{
    int32_t nb = cols / BL;
    for (int32_t r = r0; r < r1; ++r) {
        double a = 0.0;
        for (int32_t b = 0; b < nb; ++b) {
            int32_t sumi = zp_block_sum(bits, wq, wzp, cols, xq, r, b);
            a += fabs((double)sumi * (double)wd[(int64_t)r * nb + b] * (double)xd[b]);
        }
        out[r - r0] = a;
    }
}

/* ------------------------------------------------------------------------
 * K-quant super-blocks ("SKaiNET-native-kernels", section "Proving an
 * optimization is safe before writing it": 4-bit weights w in [0, 15],
 * 32 elements per sub-block, a 6-bit sub-block scale s <= 63, 8 sub-blocks
 * per block, int8 activations, and the sub-block scale folded in the
 * integer domain, sum over b of s_b * (sum over i of a_i * w_i), before one
 * conversion to float; section "Accomplishments that we're proud of": the
 * format keeps per-32 asymmetric minima).
 *
 * Readings where the page is silent (it gives neither the storage nor the
 * scale types):
 *   - weight element i of sub-block b of super-block k of row r has the
 *     value d[r,k] * sc[r,8k+b] * w_i - dmin[r,k] * mn[r,8k+b]: a 6-bit
 *     scale and a 6-bit minimum per 32 elements (one byte each, 0..63), two
 *     fp32 super-block scales per 256 elements;
 *   - the nibbles of a sub-block take the spec's Q4_0 layout (16 bytes,
 *     element j in the low nibble of byte j, element j + 16 in the high
 *     nibble), stored as they are (no offset);
 *   - the activation is quantized with the spec's Q8_0 rule on 256-element
 *     blocks, so that one activation scale covers a super-block and the fold
 *     is one exact integer:
 *       S1 = sum_b sc_b * (sum_i w_i * q_i),   S2 = sum_b mn_b * (sum_i q_i),
 *       y[r] = sum over super-blocks, ascending, of
 *              (((float)S1 * d) - ((float)S2 * dmin)) * dx.
 *     |S1| <= 8*63*32*127*15 = 30,723,840 and |S2| <= 8*63*32*127 =
 *     2,048,256, both exact in int32.  S1 can exceed 2^24, so (float)S1
 *     may round: that conversion is one of the rounded float operations of
 *     the rule.
 * ---------------------------------------------------------------------- */
#define SBK 256
#define SUBK 32

void orc_quantize_q8_b256(const float *x, int64_t n, int8_t *q, float *d)
{
    for (int64_t b = 0; b < n / SBK; ++b) {
        const float *xb = x + b * SBK;
        float amax = 0.0f;
        for (int i = 0; i < SBK; ++i) {
            float a = fabsf(xb[i]);
            if (a > amax)
                amax = a;
        }
        float db = amax / 127.0f;
        float id = (amax != 0.0f) ? 127.0f / amax : 0.0f;
        for (int i = 0; i < SBK; ++i) {
            float v = xb[i] * id;
            float t = v + copysignf(0.5f, xb[i]);
            int qi = (int)truncf(t);
            if (qi > 127)
                qi = 127;
            if (qi < -127)
                qi = -127;
            q[b * SBK + i] = (int8_t)qi;
        }
        d[b] = db;
    }
}

/* nibble of element i (0..31) of a 16-byte sub-block, as stored */
static int q4k_nib(const uint8_t *sub, int i)
{
    return (i < 16) ? (sub[i] & 0x0F) : (sub[i - 16] >> 4);
}

static void q4k_sums(const uint8_t *wq, const uint8_t *sc, const uint8_t *mn, int32_t cols,
                     const int8_t *xq, int32_t r, int32_t k, int32_t *s1, int32_t *s2)
{
    int32_t nsub = cols / SUBK;
    int64_t a = 0, m = 0;
    for (int b = 0; b < SBK / SUBK; ++b) {
        int32_t sb = k * (SBK / SUBK) + b;
        const uint8_t *sub = wq + (int64_t)r * (cols / 2) + (int64_t)sb * 16;
        const int8_t *xv = xq + (int64_t)sb * SUBK;
        int64_t dot = 0, qs = 0;
        for (int i = 0; i < SUBK; ++i) {
            dot += (int64_t)q4k_nib(sub, i) * xv[i];
            qs += xv[i];
        }
        a += (int64_t)sc[(int64_t)r * nsub + sb] * dot;
        m += (int64_t)mn[(int64_t)r * nsub + sb] * qs;
    }
    *s1 = (int32_t)a;
    *s2 = (int32_t)m;
}

/* s1, s2 each have (r1 - r0) * (cols / 256) entries, row-major. */
void orc_superblock_sums_q4k(const uint8_t *wq, const uint8_t *sc, const uint8_t *mn, int32_t cols,
                             const int8_t *xq, int32_t r0, int32_t r1, int32_t *s1, int32_t *s2)
{
    int32_t nk = cols / SBK;
    for (int32_t r = r0; r < r1; ++r)
        for (int32_t k = 0; k < nk; ++k)
            q4k_sums(wq, sc, mn, cols, xq, r, k, s1 + (int64_t)(r - r0) * nk + k,
                     s2 + (int64_t)(r - r0) * nk + k);
}

void orc_matvec_q4k(float *y, const uint8_t *wq, const uint8_t *sc, const uint8_t *mn,
                    const float *d, const float *dmin, int32_t cols, const int8_t *xq,
                    const float *xd, int32_t r0, int32_t r1)
{
    int32_t nk = cols / SBK;
    for (int32_t r = r0; r < r1; ++r) {
        float s = 0.0f;
        for (int32_t k = 0; k < nk; ++k) {
            int32_t s1, s2;
            q4k_sums(wq, sc, mn, cols, xq, r, k, &s1, &s2);
            float t = (float)s1 * d[(int64_t)r * nk + k];
            float u = (float)s2 * dmin[(int64_t)r * nk + k];
            float v = t - u;
            v = v * xd[k];
            s = s + v;
        }
        y[r] = s;
    }
}

/* A(r) = sum over super-blocks of |dx| * (|S1 * d| + |S2 * dmin|) in binary64:
 * the scale of the tolerance |y - y_ref| <= 1e-5 * A + 1e-6. */
void orc_tol_abs_q4k(const uint8_t *wq, const uint8_t *sc, const uint8_t *mn, const float *d,
                     const float *dmin, int32_t cols, const int8_t *xq, const float *xd,
                     int32_t r0, int32_t r1, double *out)
{
    int32_t nk = cols / SBK;
    for (int32_t r = r0; r < r1; ++r) {
        double a = 0.0;
        for (int32_t k = 0; k < nk; ++k) {
            int32_t s1, s2;
            q4k_sums(wq, sc, mn, cols, xq, r, k, &s1, &s2);
            a += fabs((double)xd[k]) * (fabs((double)s1 * d[(int64_t)r * nk + k]) +
                                        fabs((double)s2 * dmin[(int64_t)r * nk + k]));
        }
        out[r - r0] = a;
    }
}
