"""Pins of the CPU oracle against facts fixed by the design spec and by
mathematics -- never against the oracle itself.

Each check raises AssertionError when the oracle in use (oracle.oracle.lib(),
which a test may swap for a build with a planted mistake) disagrees with:
  * closed forms the spec states (zero block, the +-127 clamp, the nibble
    layout, the largest block sum),
  * textbook rounding (Python's decimal ROUND_HALF_UP, i.e. half away from
    zero) where the spec's rule reduces to it exactly,
  * detector vectors whose expected values are derived by hand,
  * exact invariants (sign symmetry, powers of two, row permutations,
    row sub-ranges),
  * brute force: int64 block sums and float64 dequantized dot products
    (numpy), with the spec's tolerance.

Rules: "Legacy-ISA ML Inference Runtime -- Design Spec", section 4
(Quantization Formats), section 5 (Kernel Interface, rounding bullet) and
section 7 (Testing: test_kernels / test_quant).
"""
from __future__ import annotations

import decimal
import json
import os

import numpy as np

from oracle import oracle as orc

QK = 32
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32_from_bits(h) -> np.float32:
    return np.array([int(h, 16) if isinstance(h, str) else h], np.uint32).view(np.float32)[0]


def half_away(x: float) -> int:
    """Textbook round-half-away-from-zero of the exact binary value x."""
    return int(decimal.Decimal(float(x)).quantize(decimal.Decimal(1), rounding=decimal.ROUND_HALF_UP))


# ---------------------------------------------------------------------------
# Independent numpy readers of the storage layout (section 4 table).
# ---------------------------------------------------------------------------

def q4_values(q: np.ndarray) -> np.ndarray:
    """[rows, K/2] uint8 -> [rows, K] int64 values nibble - 8, element j of a
    block from the low nibble of byte j (j < 16), element j from the high
    nibble of byte j - 16 (j >= 16)."""
    rows = q.shape[0]
    b = q.reshape(rows, -1, 16).astype(np.int64)
    lo = b & 0x0F
    hi = b >> 4
    return (np.concatenate([lo, hi], axis=2) - 8).reshape(rows, -1)


def w_values(qtype, q):
    return q.astype(np.int64) if qtype == 8 else q4_values(q)


def brute_matvec64(qtype, wq, wd, xq, xd):
    """float64 sum over k of (w_k * dw) * (qx_k * dx): the dequantized dot."""
    w = w_values(qtype, wq).astype(np.float64)
    rows, k = w.shape
    wdeq = (w.reshape(rows, k // QK, QK) * wd.astype(np.float64)[:, :, None]).reshape(rows, k)
    xdeq = (xq.astype(np.float64).reshape(-1, QK) * xd.astype(np.float64).reshape(-1)[:, None]).reshape(-1)
    return wdeq @ xdeq


def brute_abs_terms64(qtype, wq, wd, xq, xd):
    """float64 A(r) = sum_b |sumi * dw * dx| from int64 brute-force sums."""
    w = w_values(qtype, wq)
    rows, k = w.shape
    s = (w.reshape(rows, k // QK, QK) * xq.astype(np.int64).reshape(1, k // QK, QK)).sum(axis=2)
    return np.abs(s.astype(np.float64) * wd.astype(np.float64) * xd.astype(np.float64).reshape(1, -1)).sum(axis=1)


# ---------------------------------------------------------------------------
# Q8_0 quantization pins
# ---------------------------------------------------------------------------

def check_q8_zero_block():
    x = np.zeros(64, np.float32)
    x[32:] = -0.0
    q, d = orc.quantize_q8(x)
    assert np.all(q == 0) and np.all(d == 0.0), "zero block must give d = 0 and q = 0"


def check_q8_equal_block():
    for c in (0.37, 1.0, 3.0e-3, 1234.5):
        c32 = np.float32(c)
        x = np.full(32, c32, np.float32)
        q, d = orc.quantize_q8(x)
        assert np.all(q == 127), "a block of equal positive values quantizes to 127"
        assert d[0] == c32 / np.float32(127.0), "d = amax / 127 (IEEE binary32 division)"
        q, d = orc.quantize_q8(-x)
        assert np.all(q == -127) and d[0] == c32 / np.float32(127.0)


def check_q8_clamp_and_range():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(32 * 512).astype(np.float32) * np.float32(3.0)
    x[::97] *= np.float32(50.0)
    q, d = orc.quantize_q8(x)
    assert q.min() >= -127 and q.max() <= 127, "quants clamped to [-127, 127]"
    # the element of largest magnitude in each block maps to +-127
    xb = x.reshape(-1, QK)
    qb = q.reshape(-1, QK)
    i = np.argmax(np.abs(xb), axis=1)
    top = qb[np.arange(len(i)), i]
    assert np.all(np.abs(top) == 127), "amax element maps to +-127"
    assert np.all(np.sign(top) == np.sign(xb[np.arange(len(i)), i]))


def check_q8_unit_scale_textbook():
    # amax = 127 makes id = 127/127 = 1 and d = 1 exactly, so q = trunc(x + copysign(0.5, x));
    # for x on a 1/8 grid the addition is exact and this is textbook half-away rounding.
    k = np.arange(-1016, 1017, dtype=np.int64)
    vals = (k / 8.0).astype(np.float32)
    vals = vals[np.abs(vals) <= 127]
    pad = (-len(vals)) % 31
    vals = np.concatenate([vals, np.zeros(pad, np.float32)])
    blocks = vals.reshape(-1, 31)
    x = np.concatenate([np.full((len(blocks), 1), 127.0, np.float32), blocks], axis=1)
    q, d = orc.quantize_q8(x.reshape(-1))
    assert np.all(d == 1.0)
    expect = np.array([[half_away(v) for v in row] for row in x], np.int64)
    assert np.array_equal(q.reshape(x.shape).astype(np.int64), expect), "unit-scale rounding is half away from zero"
    # random values not within 2^-20 of a half-integer also round textbook-style
    rng = np.random.default_rng(12)
    r = rng.uniform(-126.9, 126.9, size=(64, 31)).astype(np.float32)
    frac = np.abs(np.abs(r.astype(np.float64)) - np.floor(np.abs(r.astype(np.float64))) - 0.5)
    r[frac < 2.0 ** -20] = 0.25
    x = np.concatenate([np.full((64, 1), 127.0, np.float32), r], axis=1)
    q, _ = orc.quantize_q8(x.reshape(-1))
    expect = np.array([[half_away(v) for v in row] for row in x], np.int64)
    assert np.array_equal(q.reshape(x.shape).astype(np.int64), expect)


def check_q8_ties():
    x = np.zeros(32, np.float32)
    x[0] = 127.0
    x[1:7] = [2.5, -2.5, 0.5, -0.5, 1.5, 126.5]
    q, _ = orc.quantize_q8(x)
    assert list(q[1:7]) == [3, -3, 1, -1, 2, 127], "ties go away from zero"


def check_q8_detectors():
    for case in golden("q8_rounding_detectors.json")["cases"]:
        amax = f32_from_bits(case["amax_bits"])
        xv = f32_from_bits(case["x_bits"])
        x = np.zeros(32, np.float32)
        x[0] = amax
        x[5] = xv
        x[9] = -xv
        q, _ = orc.quantize_q8(x)
        assert q[5] == case["q"] and q[9] == -case["q"], case["why"]


def check_q8_invariants():
    rng = np.random.default_rng(13)
    x = rng.standard_normal(32 * 256).astype(np.float32)
    q, d = orc.quantize_q8(x)
    qn, dn = orc.quantize_q8(-x)
    assert np.array_equal(qn, -q) and np.array_equal(dn, d), "q(-x) = -q(x), d(-x) = d(x)"
    for k in (-7, -1, 1, 5):
        s = np.float32(2.0 ** k)
        qs, ds = orc.quantize_q8(x * s)
        assert np.array_equal(qs, q) and np.array_equal(ds, d * s), "power-of-two scaling"


def check_q8_roundtrip():
    # section 7, test_quant: quantize -> dequantize error <= d/2 per element
    rng = np.random.default_rng(14)
    x = rng.standard_normal(32 * 1024).astype(np.float32)
    x[::50] *= np.float32(20.0)
    q, d = orc.quantize_q8(x)
    xb = x.reshape(-1, QK).astype(np.float64)
    deq = q.reshape(-1, QK).astype(np.float64) * d.astype(np.float64)[:, None]
    err = np.abs(deq - xb)
    amax = np.abs(xb).max(axis=1)
    # d/2 plus a few binary32 roundings of the amax-sized intermediate values
    bound = d.astype(np.float64)[:, None] / 2 + 4 * amax[:, None] * 2.0 ** -24
    assert np.all(err <= bound), "round trip within d/2"


# ---------------------------------------------------------------------------
# Q4_0 quantization pins
# ---------------------------------------------------------------------------

def check_q4_layout():
    spec = golden("spec_constants.json")["q4_0"]
    v = np.array([(i % 15) - 7 for i in range(32)], np.int64)  # -7..7, each element distinct within a half
    v[3] = 7
    c = np.float32(0.125)
    x = (v * 0.125).astype(np.float32)        # amax = 7c exactly, id = 7/amax = 8, x*id = v exactly
    q, d = orc.quantize_q4(x)
    assert q.shape == (spec["bytes_per_block"],)
    assert d[0] == np.float32(7 * c) / np.float32(7.0)
    lo, hi = spec["low_nibble_elems"], spec["high_nibble_elems"]
    for j in range(16):
        assert (q[j] & 0x0F) == v[lo[0] + j] + spec["offset"], "low nibble of byte j holds element j"
        assert (q[j] >> 4) == v[hi[0] + j] + spec["offset"], "high nibble of byte j holds element j+16"


def check_q4_closed_forms():
    x = np.zeros(64, np.float32)
    x[32:] = 0.3
    q, d = orc.quantize_q4(x)
    assert np.all(q[:16] == 0x88) and d[0] == 0.0, "zero block: nibble 8 (value 0), d = 0"
    assert np.all(q[16:] == 0xFF) and d[1] == np.float32(0.3) / np.float32(7.0), "equal block: value 7"
    q, d = orc.quantize_q4(-x)
    assert np.all(q[16:] == 0x11), "equal negative block: value -7 (nibble 1)"


def check_q4_roundtrip():
    rng = np.random.default_rng(15)
    x = rng.standard_normal(32 * 512).astype(np.float32)
    q, d = orc.quantize_q4(x)
    vals = q4_values(q.reshape(1, -1)).reshape(-1, QK)
    assert vals.min() >= -8 and vals.max() <= 7
    deq = vals.astype(np.float64) * d.astype(np.float64)[:, None]
    xb = x.reshape(-1, QK).astype(np.float64)
    amax = np.abs(xb).max(axis=1)
    bound = d.astype(np.float64)[:, None] / 2 + 4 * amax[:, None] * 2.0 ** -24
    assert np.all(np.abs(deq - xb) <= bound)


# ---------------------------------------------------------------------------
# Block sums
# ---------------------------------------------------------------------------

def check_block_sum_closed_forms():
    spec = golden("spec_constants.json")
    wq = np.full((1, 32), 127, np.int8)
    xq = np.full(32, 127, np.int8)
    s = orc.block_sums(8, wq, xq)
    assert s[0, 0] == spec["max_abs_block_sum_q8"] == 32 * 127 * 127
    s = orc.block_sums(8, wq, -xq)
    assert s[0, 0] == -spec["max_abs_block_sum_q8"]
    w4 = np.zeros((1, 16), np.uint8)           # every nibble 0 -> value -8
    s = orc.block_sums(4, w4, np.full(32, -127, np.int8))
    assert s[0, 0] == 32 * 8 * 127
    w4 = np.full((1, 16), 0x0F, np.uint8)      # low nibbles 15 (+7), high nibbles 0 (-8)
    xq = np.concatenate([np.ones(16, np.int8), np.full(16, 2, np.int8)])
    s = orc.block_sums(4, w4, xq)
    assert s[0, 0] == 16 * 7 * 1 + 16 * (-8) * 2


def check_block_sums_brute():
    rng = np.random.default_rng(16)
    for qtype in (8, 4):
        rows, k = 7, 32 * 9
        if qtype == 8:
            wq = rng.integers(-128, 128, size=(rows, k), dtype=np.int16).astype(np.int8)
        else:
            wq = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
        xq = rng.integers(-128, 128, size=k, dtype=np.int16).astype(np.int8)
        got = orc.block_sums(qtype, wq, xq)
        w = w_values(qtype, wq).reshape(rows, k // QK, QK)
        want = (w * xq.astype(np.int64).reshape(1, k // QK, QK)).sum(axis=2)
        assert np.array_equal(got.astype(np.int64), want)
        got = orc.block_sums(qtype, wq, xq, 2, 5)
        assert np.array_equal(got.astype(np.int64), want[2:5])


# ---------------------------------------------------------------------------
# Matvec / gemm
# ---------------------------------------------------------------------------

def _tiny_problem(rng, qtype, rows, k):
    if qtype == 8:
        wq = rng.integers(-127, 128, size=(rows, k), dtype=np.int16).astype(np.int8)
    else:
        wq = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    wd = (np.exp2(rng.uniform(-8, 0, size=(rows, k // QK))) * rng.uniform(0.5, 2, size=(rows, k // QK))).astype(np.float32)
    x = rng.standard_normal(k).astype(np.float32)
    xq, xd = orc.quantize_q8(x)
    return wq, wd, xq, xd


def check_matvec_brute64():
    rng = np.random.default_rng(17)
    for qtype in (8, 4):
        for rows, k in ((1, 32), (5, 64), (13, 32 * 11), (4, 32 * 40)):
            wq, wd, xq, xd = _tiny_problem(rng, qtype, rows, k)
            y = orc.matvec(qtype, wq, wd, xq, xd)
            y64 = brute_matvec64(qtype, wq, wd, xq, xd)
            a64 = brute_abs_terms64(qtype, wq, wd, xq, xd)
            assert np.all(np.abs(y.astype(np.float64) - y64) <= 1e-5 * a64 + 1e-6), "fp64 brute force"
            assert np.allclose(orc.tol_abs(qtype, wq, wd, xq, xd), a64, rtol=1e-12, atol=0), "A(r)"


def check_matvec_unit_scales():
    # dw = dx = 1: y[r] = sum_b sumi exactly while |sum| < 2^24
    rng = np.random.default_rng(18)
    for qtype in (8, 4):
        rows, k = 9, 32 * 16
        wq, _, xq, _ = _tiny_problem(rng, qtype, rows, k)
        ones_w = np.ones((rows, k // QK), np.float32)
        ones_x = np.ones(k // QK, np.float32)
        y = orc.matvec(qtype, wq, ones_w, xq, ones_x)
        want = (w_values(qtype, wq) * xq.astype(np.int64)[None, :]).sum(axis=1)
        assert np.all(np.abs(want) < 2 ** 24)
        # integers below 2^24 in magnitude before the exact comparison (a wrong
        # oracle may produce values no int64 holds)
        assert np.all(np.abs(y) < 2.0 ** 24) and np.array_equal(y.astype(np.int64), want)
        # one-hot dx isolates one block's sum at any K
        for b in (0, k // QK - 1, 5):
            oh = np.zeros(k // QK, np.float32)
            oh[b] = 1.0
            y = orc.matvec(qtype, wq, ones_w, xq, oh)
            wb = w_values(qtype, wq)[:, b * QK:(b + 1) * QK]
            assert np.all(np.isfinite(y))
            assert np.array_equal(y.astype(np.int64), (wb * xq[b * QK:(b + 1) * QK].astype(np.int64)).sum(axis=1))


def check_matvec_invariants():
    rng = np.random.default_rng(19)
    for qtype in (8, 4):
        rows, k = 11, 32 * 7
        wq, wd, xq, xd = _tiny_problem(rng, qtype, rows, k)
        y = orc.matvec(qtype, wq, wd, xq, xd)
        yn = orc.matvec(qtype, wq, wd, (-xq.astype(np.int16)).astype(np.int8), xd)
        assert np.array_equal(yn, -y), "y(-x) = -y(x)"
        ys = orc.matvec(qtype, wq, wd, xq, xd * np.float32(0.25))
        assert np.array_equal(ys, y * np.float32(0.25)), "y(x * 2^-2) = y(x) * 2^-2"
        perm = rng.permutation(rows)
        yp = orc.matvec(qtype, wq[perm], wd[perm], xq, xd)
        assert np.array_equal(yp, y[perm]), "row permutation"
        sentinel = np.full(rows, np.float32(-7.5))
        ysub = orc.matvec(qtype, wq, wd, xq, xd, 3, 8, y=sentinel.copy())
        assert np.array_equal(ysub[3:8], y[3:8]), "rows [r0, r1) match the full run"
        assert np.all(ysub[:3] == -7.5) and np.all(ysub[8:] == -7.5), "rows outside [r0, r1) untouched"
        ye = orc.matvec(qtype, wq, wd, xq, xd, 4, 4, y=sentinel.copy())
        assert np.all(ye == -7.5), "empty range writes nothing"


def check_gemm_rows():
    rng = np.random.default_rng(20)
    for qtype in (8, 4):
        rows, k, m = 6, 32 * 5, 3
        wq, wd, _, _ = _tiny_problem(rng, qtype, rows, k)
        X = rng.standard_normal((m, k)).astype(np.float32)
        xq, xd = orc.quantize_q8(X)
        # per-row quantization of X equals quantizing the flattened M*K array
        xq1, xd1 = orc.quantize_q8(X.reshape(-1))
        assert np.array_equal(xq1.reshape(m, k), xq) and np.array_equal(xd1.reshape(m, -1), xd)
        Y = orc.gemm(qtype, wq, wd, xq, xd)
        for i in range(m):
            assert np.array_equal(Y[i], orc.matvec(qtype, wq, wd, xq[i], xd[i]))
            y64 = brute_matvec64(qtype, wq, wd, xq[i], xd[i])
            a64 = brute_abs_terms64(qtype, wq, wd, xq[i], xd[i])
            assert np.all(np.abs(Y[i].astype(np.float64) - y64) <= 1e-5 * a64 + 1e-6)


def check_sumsq_pairwise_order():
    """The rmsnorm sum of squares in its stated order, on inputs where the
    order decides the rounding (values derived by hand):
      * one block: x_0 = 1, x_1..x_31 = 2^-12 (squares 1 and 2^-24).  Pairwise:
        1 + 2^-24 ties to 1; the fifteen other pairs give 2^-23 each; then
        1 + 2^-23, + 2^-22, + 2^-21, + 2^-20 are exact: 1 + 15 * 2^-23.  A
        left-to-right sum stays at 1 (every + 2^-24 ties back to 1).
      * four blocks with sums 1, 2^-24, 2^-24, 2^-24: pairwise over the
        blocks, (1 + 2^-24) + (2^-24 + 2^-24) = 1 + 2^-23; left to right, 1.
      * three blocks (padded to four): sums 1, 2^-24, 2^-24 -> (1 + 2^-24) +
        (2^-24 + 0) = 1 + 2^-24 -> 1."""
    x = np.zeros(64, np.float32)
    x[0] = 1.0
    x[1:32] = np.float32(2.0 ** -12)
    assert orc.sumsq(x) == np.float32(1.0 + 15 * 2.0 ** -23)
    x = np.zeros(128, np.float32)
    x[0] = 1.0
    x[32] = x[64] = x[96] = np.float32(2.0 ** -12)
    assert orc.sumsq(x) == np.float32(1.0 + 2.0 ** -23)
    assert orc.sumsq(x[:96]) == np.float32(1.0)
    # integer squares: every order is exact
    rng = np.random.default_rng(21)
    xi = rng.integers(-40, 41, size=32 * 28).astype(np.float32)
    assert orc.sumsq(xi) == np.float32(int((xi.astype(np.int64) ** 2).sum()))


def check_rmsnorm_closed_forms():
    """Constant input: ss / n is the constant's square exactly, so with
    eps = 0, inv * x rounds to exactly 1 and o = w bit for bit (x = 1, and
    x = 3 where inv = RN(1/3) and RN(RN(1/3) * 3) = 1).  A zero input gives
    zeros (eps > 0 keeps inv finite)."""
    for n in (4096, 896, 64):
        w = (np.arange(n, dtype=np.float32) - np.float32(n / 3)) * np.float32(0.01)
        for c in (1.0, 3.0, -1.0):
            o = orc.rmsnorm(np.full(n, c, np.float32), w, 0.0)
            assert np.array_equal(o, w * np.float32(np.sign(c))), (n, c)
        o = orc.rmsnorm(np.zeros(n, np.float32), w, 1e-5)
        assert np.all(o == 0.0)


def check_rmsnorm_invariants_and_brute():
    rng = np.random.default_rng(22)
    for n, sigma, eps in ((4096, 1.0, 1e-5), (2048, 0.01, 1e-4), (896, 3.0, 1e-6), (32 * 13, 0.5, 0.5)):
        x = (rng.standard_normal(n) * sigma).astype(np.float32)
        w = (1.0 + 0.1 * rng.standard_normal(n)).astype(np.float32)
        o = orc.rmsnorm(x, w, eps)
        # float64 brute force: binary32 rounding of a few operations only
        x64, w64 = x.astype(np.float64), w.astype(np.float64)
        o64 = w64 * x64 / np.sqrt((x64 * x64).sum() / n + eps)
        assert np.all(np.abs(o - o64) <= 4 * np.finfo(np.float32).eps * np.abs(o64) + 1e-30), n
        assert np.array_equal(orc.rmsnorm(-x, w, eps), -o)
        # powers of two scale every step exactly (eps = 0)
        o0 = orc.rmsnorm(x, w, 0.0)
        for k in (-3, 5):
            assert np.array_equal(orc.rmsnorm(x * np.float32(2.0 ** k), w, 0.0), o0), (n, k)


def check_silu_mul():
    """silu(0) = 0; far from 0 the sigmoid saturates exactly in binary32
    (1 + expf(-v) rounds to 1 for v >= 17, so o = v * u; expf(-v) overflows
    to +inf for v <= -89, so o = +-0); silu(g) - silu(-g) = g; and fp64
    brute force within a few binary32 roundings (the C library's expf is
    within 1 ulp)."""
    u = np.array([1.0, -2.5, 3.0, 0.125], np.float32)
    assert np.all(orc.silu_mul(np.zeros(4, np.float32), u) == 0.0)
    for v in (17.0, 40.0, 100.0):
        g = np.full(4, v, np.float32)
        assert np.array_equal(orc.silu_mul(g, u), g * u), v
    for v in (-89.0, -100.0, -1e30):
        assert np.all(orc.silu_mul(np.full(4, v, np.float32), u) == 0.0), v
    rng = np.random.default_rng(23)
    g = (rng.standard_normal(4096) * 4.0).astype(np.float32)
    u = rng.standard_normal(4096).astype(np.float32)
    ones = np.ones_like(g)
    d = orc.silu_mul(g, ones).astype(np.float64) - orc.silu_mul(-g, ones).astype(np.float64)
    assert np.all(np.abs(d - g) <= 4 * np.finfo(np.float32).eps * np.abs(g))
    g64, u64 = g.astype(np.float64), u.astype(np.float64)
    o64 = g64 / (1.0 + np.exp(-g64)) * u64
    o = orc.silu_mul(g, u).astype(np.float64)
    assert np.all(np.abs(o - o64) <= 6 * np.finfo(np.float32).eps * np.abs(o64) + 1e-37)


# ---------------------------------------------------------------------------
# Block length 128 with a zero point ("ONNX Runtime" page, sections 3 and 4;
# the readings are listed in the oracle's C file)
# ---------------------------------------------------------------------------

BL = 128


def zp_codes(bits, wq):
    """[rows, K or K/2] uint8 -> [rows, K] int64 codes; 4 bits: element 2i
    from the low nibble of byte i, element 2i + 1 from the high nibble."""
    if bits == 8:
        return wq.astype(np.int64)
    lo = (wq & 0x0F).astype(np.int64)
    hi = (wq >> 4).astype(np.int64)
    return np.stack([lo, hi], axis=2).reshape(wq.shape[0], -1)


def zp_values(bits, wq, wzp):
    c = zp_codes(bits, wq)
    rows, k = c.shape
    z = np.full((rows, k // BL), 1 << (bits - 1), np.int64) if wzp is None else wzp.astype(np.int64)
    return c - np.repeat(z, BL, axis=1)


def _zp_problem(rng, bits, rows, k, with_zp=True):
    nb = k // BL
    wq = rng.integers(0, 256, size=(rows, k if bits == 8 else k // 2), dtype=np.uint8)
    wzp = rng.integers(0, 1 << bits, size=(rows, nb), dtype=np.uint8) if with_zp else None
    wd = (np.exp2(rng.uniform(-8, 0, size=(rows, nb))) * rng.uniform(0.5, 2, size=(rows, nb))).astype(np.float32)
    xq, xd = orc.quantize_q8_b128(rng.standard_normal(k).astype(np.float32))
    return wq, wd, wzp, xq, xd


def check_b128_quantize():
    rng = np.random.default_rng(30)
    # every 32-sub-block carries the same largest magnitude: the rule on
    # 128-element blocks gives the (pinned) Q8_0 codes and four equal scales
    x = rng.uniform(-1, 1, size=512).astype(np.float32)
    x[::32] = np.where(rng.random(16) < 0.5, -1.5, 1.5).astype(np.float32)
    q, d = orc.quantize_q8_b128(x)
    q8, d8 = orc.quantize_q8(x)
    assert q.shape == (512,) and d.shape == (4,)
    assert np.array_equal(q, q8) and np.array_equal(np.repeat(d, 4), d8)
    # one scale per 128 elements: integers with a single 127 per block give
    # id = 1 and q = x in every sub-block, where Q8_0 would rescale the others
    x = rng.integers(-60, 61, size=256).astype(np.float32)
    x[5] = 127.0
    x[128 + 100] = -127.0
    q, d = orc.quantize_q8_b128(x)
    assert np.array_equal(q, x.astype(np.int8)) and np.array_equal(d, np.float32([1.0, 1.0]))
    q8, _ = orc.quantize_q8(x)
    assert not np.array_equal(q8, q)
    # zero block
    x[128:] = 0.0
    q, d = orc.quantize_q8_b128(x)
    assert d[1] == 0 and not np.any(q[128:])


def check_zp_block_sum_closed_forms():
    k = 256
    x127 = np.full(k, 127, np.int8)
    w = np.full((1, k), 255, np.uint8)
    s = orc.block_sums_zp(8, w, np.zeros((1, 2), np.uint8), x127)
    assert np.array_equal(s, [[128 * 255 * 127] * 2])                    # largest |sumi|, 8 bits
    s = orc.block_sums_zp(8, np.zeros((1, k), np.uint8), None, x127)
    assert np.array_equal(s, [[-128 * 128 * 127] * 2])                   # default zp = 128
    s = orc.block_sums_zp(8, np.full((1, k), 128, np.uint8), None, x127)
    assert not np.any(s)
    zp = np.uint8([[17, 250]])
    w = np.repeat(zp, BL, axis=1)
    assert not np.any(orc.block_sums_zp(8, w, zp, x127))                 # codes equal to zp
    w4 = np.full((1, k // 2), 0xFF, np.uint8)
    s = orc.block_sums_zp(4, w4, np.zeros((1, 2), np.uint8), -x127)
    assert np.array_equal(s, [[-128 * 15 * 127] * 2])
    s = orc.block_sums_zp(4, np.zeros((1, k // 2), np.uint8), None, x127)
    assert np.array_equal(s, [[-128 * 8 * 127] * 2])                     # default zp = 8
    w4 = np.full((1, k // 2), 0x88, np.uint8)
    assert not np.any(orc.block_sums_zp(4, w4, None, x127))


def check_zp_nibble_order():
    """One-hot activations read single elements: element 2i is the low
    nibble of byte i, element 2i + 1 the high nibble."""
    k = 128
    b = np.arange(64, dtype=np.uint8)
    w4 = ((b % 16) | ((15 - (b % 16)) << 4)).astype(np.uint8).reshape(1, 64)
    zp = np.uint8([[3]])
    for e in (0, 1, 2, 7, 64, 127):
        x = np.zeros(k, np.int8)
        x[e] = 1
        s = orc.block_sums_zp(4, w4, zp, x)
        byte = int(w4[0, e // 2])
        want = ((byte & 0x0F) if e % 2 == 0 else (byte >> 4)) - 3
        assert s[0, 0] == want, e


def check_zp_reduces_to_symmetric():
    """At the default zero point the values are those of the symmetric
    formats: 8 bits, B - 128 = the int8 with the top bit flipped (Q8_0);
    4 bits, nibble - 8 (Q4_0 after moving each element to its Q4_0 byte).
    The sums over the four 32-sub-blocks equal the (pinned) Q8_0 / Q4_0
    block sums."""
    rng = np.random.default_rng(31)
    rows, k = 3, 384
    xq = rng.integers(-127, 128, size=k, dtype=np.int16).astype(np.int8)
    B = rng.integers(0, 256, size=(rows, k), dtype=np.uint8)
    s = orc.block_sums_zp(8, B, None, xq)
    s8 = orc.block_sums(8, (B ^ 0x80).view(np.int8), xq)
    assert np.array_equal(s, s8.reshape(rows, -1, 4).sum(axis=2))
    w4 = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    nib = zp_codes(4, w4).reshape(rows, k // QK, QK)           # stored nibble per element
    q40 = (nib[:, :, :16] | (nib[:, :, 16:] << 4)).astype(np.uint8).reshape(rows, k // 2)
    s = orc.block_sums_zp(4, w4, None, xq)
    s4 = orc.block_sums(4, q40, xq)
    assert np.array_equal(s, s4.reshape(rows, -1, 4).sum(axis=2))


def check_zp_block_sums_brute():
    rng = np.random.default_rng(32)
    for bits in (8, 4):
        for with_zp in (True, False):
            rows, k = 6, 128 * 5
            wq, _, wzp, _, _ = _zp_problem(rng, bits, rows, k, with_zp)
            xq = rng.integers(-128, 128, size=k, dtype=np.int16).astype(np.int8)
            got = orc.block_sums_zp(bits, wq, wzp, xq)
            v = zp_values(bits, wq, wzp).reshape(rows, k // BL, BL)
            want = (v * xq.astype(np.int64).reshape(1, k // BL, BL)).sum(axis=2)
            assert np.array_equal(got.astype(np.int64), want)
            assert np.array_equal(orc.block_sums_zp(bits, wq, wzp, xq, 1, 4).astype(np.int64), want[1:4])


def check_zp_matvec_brute64():
    rng = np.random.default_rng(33)
    for bits in (8, 4):
        for rows, k in ((1, 128), (7, 384), (3, 128 * 38)):
            wq, wd, wzp, xq, xd = _zp_problem(rng, bits, rows, k, with_zp=(rows != 3))
            y = orc.matvec_zp(bits, wq, wd, wzp, xq, xd)
            v = zp_values(bits, wq, wzp)
            nb = k // BL
            wdeq = (v.reshape(rows, nb, BL) * wd.astype(np.float64)[:, :, None]).reshape(rows, k)
            xdeq = (xq.astype(np.float64).reshape(nb, BL) * xd.astype(np.float64)[:, None]).reshape(k)
            y64 = wdeq @ xdeq
            sums = (v.reshape(rows, nb, BL) * xq.astype(np.int64).reshape(1, nb, BL)).sum(axis=2)
            a64 = np.abs(sums * wd.astype(np.float64) * xd.astype(np.float64)[None, :]).sum(axis=1)
            assert np.all(np.abs(y.astype(np.float64) - y64) <= 1e-5 * a64 + 1e-6), "fp64 brute force"
            assert np.allclose(orc.tolerance_zp(bits, wq, wd, wzp, xq, xd), 1e-5 * a64 + 1e-6, rtol=1e-12, atol=0)


def check_zp_matvec_unit_scales():
    """dw = dx = 1: y is the exact sum of the block sums; rows outside
    [r0, r1) keep their value."""
    rng = np.random.default_rng(34)
    for bits in (8, 4):
        rows, k = 5, 128 * 6
        wq, _, wzp, _, _ = _zp_problem(rng, bits, rows, k)
        xq = rng.integers(-20, 21, size=k, dtype=np.int16).astype(np.int8)
        ones_w = np.ones((rows, k // BL), np.float32)
        ones_x = np.ones(k // BL, np.float32)
        want = (zp_values(bits, wq, wzp) * xq.astype(np.int64)).sum(axis=1)
        assert np.abs(want).max() < 2 ** 24
        y = orc.matvec_zp(bits, wq, ones_w, wzp, xq, ones_x)
        assert np.all(np.abs(y) < 2 ** 24), "sums at unit scales are exact integers below 2^24"
        assert np.array_equal(y.astype(np.int64), want)
        y = orc.matvec_zp(bits, wq, ones_w, wzp, xq, ones_x, 1, 3, y=np.full(rows, -7.5, np.float32))
        assert np.all(y[[0, 3, 4]] == -7.5) and np.all(np.abs(y[1:3]) < 2 ** 24)
        assert np.array_equal(y[1:3].astype(np.int64), want[1:3])


# ---------------------------------------------------------------------------
# K-quant super-blocks ("SKaiNET-native-kernels" page; readings in the
# oracle's C file): value = d * sc_b * w - dmin * mn_b, 256-element
# activation blocks, S1 = sum_b sc_b sum_i w_i q_i, S2 = sum_b mn_b sum_i q_i
# ---------------------------------------------------------------------------

SBK = 256


def q4k_nibbles(wq):
    """[rows, K/2] uint8 -> [rows, K] int64 stored nibbles, per 32-element
    sub-block: element j < 16 from the low nibble of byte j, element j >= 16
    from the high nibble of byte j - 16."""
    rows = wq.shape[0]
    b = wq.reshape(rows, -1, 16).astype(np.int64)
    return np.concatenate([b & 0x0F, b >> 4], axis=2).reshape(rows, -1)


def _q4k_problem(rng, rows, k):
    nsub, nk = k // QK, k // SBK
    wq = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    sc = rng.integers(0, 64, size=(rows, nsub), dtype=np.uint8)
    mn = rng.integers(0, 64, size=(rows, nsub), dtype=np.uint8)
    d = (np.exp2(rng.uniform(-10, -4, size=(rows, nk)))).astype(np.float32)
    dmin = (np.exp2(rng.uniform(-10, -4, size=(rows, nk)))).astype(np.float32)
    xq, xd = orc.quantize_q8_b256(rng.standard_normal(k).astype(np.float32))
    return wq, sc, mn, d, dmin, xq, xd


def _q4k_brute_sums(wq, sc, mn, xq):
    rows = wq.shape[0]
    w = q4k_nibbles(wq).reshape(rows, -1, QK)
    a = xq.astype(np.int64).reshape(1, -1, QK)
    dots = (w * a).sum(axis=2)                        # [rows, nsub]
    qs = a.sum(axis=2)                                # [1, nsub]
    s1 = (sc.astype(np.int64) * dots).reshape(rows, -1, 8).sum(axis=2)
    s2 = (mn.astype(np.int64) * qs).reshape(rows, -1, 8).sum(axis=2)
    return s1, s2


def check_b256_quantize():
    rng = np.random.default_rng(40)
    x = rng.uniform(-1, 1, size=512).astype(np.float32)
    x[::32] = np.where(rng.random(16) < 0.5, -1.5, 1.5).astype(np.float32)
    q, d = orc.quantize_q8_b256(x)
    q8, d8 = orc.quantize_q8(x)
    assert d.shape == (2,) and np.array_equal(q, q8) and np.array_equal(np.repeat(d, 8), d8)
    x = rng.integers(-60, 61, size=512).astype(np.float32)
    x[200] = 127.0
    x[256 + 3] = -127.0
    q, d = orc.quantize_q8_b256(x)
    assert np.array_equal(q, x.astype(np.int8)) and np.array_equal(d, np.float32([1.0, 1.0]))


def check_q4k_fold_bound():
    """The page's bound, reached exactly: all nibbles 15, scales 63,
    activations 127 give S1 = 8*63*32*127*15; minima 63 give S2 =
    8*63*32*127; negated activations negate both."""
    g = golden("q4k_fold_bound.json")
    assert g["fold_bound"] == 8 * 63 * 32 * 127 * 15 and abs(g["fold_bound"] - g["fold_bound_as_printed"]) < 5e4
    rows, k = 1, 512
    wq = np.full((rows, k // 2), 0xFF, np.uint8)
    sc = np.full((rows, k // QK), 63, np.uint8)
    mn = np.full((rows, k // QK), 63, np.uint8)
    x = np.full(k, 127, np.int8)
    s1, s2 = orc.superblock_sums_q4k(wq, sc, mn, x)
    assert np.all(s1 == g["fold_bound"]) and np.all(s2 == g["min_term_bound"])
    s1, s2 = orc.superblock_sums_q4k(wq, sc, mn, -x)
    assert np.all(s1 == -g["fold_bound"]) and np.all(s2 == -g["min_term_bound"])


def check_q4k_layout_by_one_hot():
    """A one-hot activation at element e reads sc_b * nibble(e) and mn_b."""
    k = 256
    b = np.arange(128, dtype=np.uint8)
    wq = ((b % 16) | ((15 - (b % 16)) << 4)).astype(np.uint8).reshape(1, 128)
    sc = (np.arange(8, dtype=np.uint8) + 1).reshape(1, 8)
    mn = (np.arange(8, dtype=np.uint8) * 3 + 2).reshape(1, 8)
    for e in (0, 5, 15, 16, 31, 32, 100, 255):
        x = np.zeros(k, np.int8)
        x[e] = 1
        s1, s2 = orc.superblock_sums_q4k(wq, sc, mn, x)
        sub, j = divmod(e, 32)
        byte = int(wq[0, sub * 16 + (j % 16)])
        nib = (byte & 0x0F) if j < 16 else (byte >> 4)
        assert s1[0, 0] == int(sc[0, sub]) * nib and s2[0, 0] == int(mn[0, sub]), e


def check_q4k_reduces_to_q4_0():
    """Scales 1 and minima 8 give the values nibble - 8 of Q4_0 (same nibble
    layout): S1 - S2 is the sum of the (pinned) Q4_0 block sums over the
    super-block."""
    rng = np.random.default_rng(41)
    rows, k = 3, 768
    wq = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    xq = rng.integers(-127, 128, size=k, dtype=np.int16).astype(np.int8)
    ones = np.ones((rows, k // QK), np.uint8)
    s1, s2 = orc.superblock_sums_q4k(wq, ones, 8 * ones, xq)
    s40 = orc.block_sums(4, wq, xq).reshape(rows, -1, 8).sum(axis=2)
    assert np.array_equal(s1.astype(np.int64) - s2, s40)


def check_q4k_sums_brute():
    rng = np.random.default_rng(42)
    rows, k = 5, 1024
    wq, sc, mn, _, _, _, _ = _q4k_problem(rng, rows, k)
    xq = rng.integers(-128, 128, size=k, dtype=np.int16).astype(np.int8)
    s1, s2 = orc.superblock_sums_q4k(wq, sc, mn, xq)
    b1, b2 = _q4k_brute_sums(wq, sc, mn, xq)
    assert np.array_equal(s1.astype(np.int64), b1) and np.array_equal(s2.astype(np.int64), b2)
    s1, s2 = orc.superblock_sums_q4k(wq, sc, mn, xq, 1, 4)
    assert np.array_equal(s1.astype(np.int64), b1[1:4]) and np.array_equal(s2.astype(np.int64), b2[1:4])


def check_q4k_matvec_brute64():
    rng = np.random.default_rng(43)
    for rows, k in ((1, 256), (7, 768), (3, 256 * 22)):
        wq, sc, mn, d, dmin, xq, xd = _q4k_problem(rng, rows, k)
        y = orc.matvec_q4k(wq, sc, mn, d, dmin, xq, xd)
        w = q4k_nibbles(wq).astype(np.float64).reshape(rows, -1, QK)
        scale = (np.repeat(d.astype(np.float64), 8, axis=1) * sc)[:, :, None]
        minv = (np.repeat(dmin.astype(np.float64), 8, axis=1) * mn)[:, :, None]
        wdeq = (scale * w - minv).reshape(rows, k)
        xdeq = (xq.astype(np.float64).reshape(-1, SBK) * xd.astype(np.float64)[:, None]).reshape(k)
        y64 = wdeq @ xdeq
        b1, b2 = _q4k_brute_sums(wq, sc, mn, xq)
        a64 = (np.abs(xd.astype(np.float64))[None, :] *
               (np.abs(b1 * d.astype(np.float64)) + np.abs(b2 * dmin.astype(np.float64)))).sum(axis=1)
        assert np.all(np.abs(y.astype(np.float64) - y64) <= 1e-5 * a64 + 1e-6), "fp64 brute force"
        assert np.allclose(orc.tolerance_q4k(wq, sc, mn, d, dmin, xq, xd), 1e-5 * a64 + 1e-6, rtol=1e-12, atol=0)


def check_q4k_unit_scales():
    """d = dmin = dx = 1: y = sum over super-blocks of S1 - S2, exact."""
    rng = np.random.default_rng(44)
    rows, k = 4, 512
    wq, sc, mn, _, _, _, _ = _q4k_problem(rng, rows, k)
    sc = (sc % 4).astype(np.uint8)
    xq = rng.integers(-20, 21, size=k, dtype=np.int16).astype(np.int8)
    one = np.ones((rows, k // SBK), np.float32)
    y = orc.matvec_q4k(wq, sc, mn, one, one, xq, np.ones(k // SBK, np.float32))
    b1, b2 = _q4k_brute_sums(wq, sc, mn, xq)
    want = (b1 - b2).sum(axis=1)
    assert np.abs(b1).max() < 2 ** 24 and np.all(np.abs(y) < 2 ** 24)
    assert np.array_equal(y.astype(np.int64), want)


ALL_CHECKS = [
    check_q8_zero_block, check_q8_equal_block, check_q8_clamp_and_range,
    check_q8_unit_scale_textbook, check_q8_ties, check_q8_detectors,
    check_q8_invariants, check_q8_roundtrip,
    check_q4_layout, check_q4_closed_forms, check_q4_roundtrip,
    check_block_sum_closed_forms, check_block_sums_brute,
    check_matvec_brute64, check_matvec_unit_scales, check_matvec_invariants,
    check_gemm_rows,
    check_sumsq_pairwise_order, check_rmsnorm_closed_forms, check_rmsnorm_invariants_and_brute,
    check_silu_mul,
    check_b128_quantize, check_zp_block_sum_closed_forms, check_zp_nibble_order,
    check_zp_reduces_to_symmetric, check_zp_block_sums_brute, check_zp_matvec_brute64,
    check_zp_matvec_unit_scales,
    check_b256_quantize, check_q4k_fold_bound, check_q4k_layout_by_one_hot, check_q4k_reduces_to_q4_0,
    check_q4k_sums_brute, check_q4k_matvec_brute64, check_q4k_unit_scales,
]


def failing_checks():
    """Names of the checks that fail against the oracle build in use."""
    bad = []
    for c in ALL_CHECKS:
        try:
            c()
        except AssertionError:
            bad.append(c.__name__)
    return bad
