"""ctypes wrapper around the C oracle (``qmv_oracle.c``).

TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the
bench's CPU-baseline leg may import this module.  It knows nothing of the
HIP library and never imports it.

Every function takes and returns host numpy arrays.  The arithmetic lives in
the C file; this module only marshals buffers.  Rules and citations are in
the C file's comments (Legacy-ISA ML Inference Runtime -- Design Spec,
sections 4, 5 and 7).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

QK = 32
_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmv_oracle.c")
_LIB = os.path.join(_HERE, "libqmv_oracle.so")

# -ffp-contract=off: no multiply-add is ever fused, each float op rounds once.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fno-tree-vectorize"]


def build(force: bool = True) -> str:
    """Compile the oracle into a shared object next to its source."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Lib:
    """Typed handle on one build of the oracle shared object."""

    def __init__(self, path: str):
        self.path = path
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        sigs = {
            "orc_quantize_q8": [P, i64, P, P],
            "orc_quantize_q4": [P, i64, P, P],
            "orc_block_sums_q8": [P, i32, P, i32, i32, P],
            "orc_block_sums_q4": [P, i32, P, i32, i32, P],
            "orc_matvec_q8": [P, P, P, i32, P, P, i32, i32],
            "orc_matvec_q4": [P, P, P, i32, P, P, i32, i32],
            "orc_gemm_q8": [P, P, P, i32, i32, P, P, i32, i32, i32],
            "orc_gemm_q4": [P, P, P, i32, i32, P, P, i32, i32, i32],
            "orc_tol_abs": [ctypes.c_int, P, P, i32, P, P, i32, i32, P],
            "orc_rmsnorm": [P, P, P, i64, ctypes.c_float],
            "orc_silu_mul": [P, P, P, i64],
            "orc_quantize_q8_b128": [P, i64, P, P],
            "orc_block_sums_zp": [ctypes.c_int, P, P, i32, P, i32, i32, P],
            "orc_matvec_zp": [P, ctypes.c_int, P, P, P, i32, P, P, i32, i32],
            "orc_tol_abs_zp": [ctypes.c_int, P, P, P, i32, P, P, i32, i32, P],
            "orc_quantize_q8_b256": [P, i64, P, P],
            "orc_superblock_sums_q4k": [P, P, P, i32, P, i32, i32, P, P],
            "orc_matvec_q4k": [P, P, P, P, P, P, i32, P, P, i32, i32],
            "orc_tol_abs_q4k": [P, P, P, P, P, i32, P, P, i32, i32, P],
        }
        for name, args in sigs.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = None
            setattr(self, name, f)
        self.orc_sumsq = L.orc_sumsq
        self.orc_sumsq.argtypes = [P, i64]
        self.orc_sumsq.restype = ctypes.c_float


_lib = None
_override = None


def lib() -> _Lib:
    """The oracle build in use (the committed source, unless a test has
    swapped in another build with use_build())."""
    global _lib
    if _override is not None:
        return _override
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _Lib(_LIB)
    return _lib


def build_variant(src_text: str, out_path: str) -> str:
    """Compile an edited copy of the oracle source (used by the tests that
    plant a mistake in the oracle to show the pins catch it)."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", *CFLAGS, src, "-o", out_path, "-lm"])
    return out_path


class use_build:
    """Context manager: route every oracle call through another build."""

    def __init__(self, path: str):
        self.handle = _Lib(path)

    def __enter__(self):
        global _override
        self.prev = _override
        _override = self.handle
        return self.handle

    def __exit__(self, *exc):
        global _override
        _override = self.prev
        return False


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32)


def quantize_q8(x):
    """Q8_0 quantization of a float32 array whose size is a multiple of 32.
    Returns (q int8 of x.shape, d float32 of shape x.shape[:-1] + (n/32,))."""
    x = _f32(x)
    assert x.size % QK == 0 and x.shape[-1] % QK == 0
    q = np.empty(x.shape, np.int8)
    d = np.empty(x.shape[:-1] + (x.shape[-1] // QK,), np.float32)
    lib().orc_quantize_q8(_p(x), x.size, _p(q), _p(d))
    return q, d


def quantize_q4(x):
    """Q4_0 quantization of a float32 array (last dim multiple of 32).
    Returns (q uint8 of shape [..., n/2], d float32 [..., n/32])."""
    x = _f32(x)
    assert x.shape[-1] % QK == 0
    q = np.empty(x.shape[:-1] + (x.shape[-1] // 2,), np.uint8)
    d = np.empty(x.shape[:-1] + (x.shape[-1] // QK,), np.float32)
    lib().orc_quantize_q4(_p(x), x.size, _p(q), _p(d))
    return q, d


def _check_w(qtype, wq, wd):
    rows = wd.shape[0]
    nb = wd.shape[1]
    cols = nb * QK
    if qtype == 8:
        assert wq.dtype == np.int8 and wq.shape == (rows, cols)
    elif qtype == 4:
        assert wq.dtype == np.uint8 and wq.shape == (rows, cols // 2)
    else:
        raise ValueError("qtype must be 4 or 8")
    assert wd.dtype == np.float32
    return rows, cols


def block_sums(qtype, wq, xq, r0=None, r1=None):
    """int32 block sums sumi[r - r0, b] for rows [r0, r1)."""
    wq = np.ascontiguousarray(wq)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    rows = wq.shape[0]
    cols = xq.shape[-1]
    r0 = 0 if r0 is None else r0
    r1 = rows if r1 is None else r1
    out = np.zeros((r1 - r0, cols // QK), np.int32)
    f = lib().orc_block_sums_q8 if qtype == 8 else lib().orc_block_sums_q4
    f(_p(wq), cols, _p(xq), r0, r1, _p(out))
    return out


def matvec(qtype, wq, wd, xq, xd, r0=None, r1=None, y=None):
    """y[r] for r in [r0, r1); other entries of y are left as given
    (zeros by default)."""
    wq = np.ascontiguousarray(wq)
    wd = _f32(wd)
    rows, cols = _check_w(qtype, wq, wd)
    xq = np.ascontiguousarray(xq, dtype=np.int8).reshape(-1)
    xd = _f32(xd).reshape(-1)
    assert xq.size == cols and xd.size == cols // QK
    r0 = 0 if r0 is None else r0
    r1 = rows if r1 is None else r1
    if y is None:
        y = np.zeros(rows, np.float32)
    f = lib().orc_matvec_q8 if qtype == 8 else lib().orc_matvec_q4
    f(_p(y), _p(wq), _p(wd), cols, _p(xq), _p(xd), r0, r1)
    return y


def gemm(qtype, wq, wd, xq, xd, r0=None, r1=None, Y=None):
    """Y[m, r] for every row m of X and r in [r0, r1)."""
    wq = np.ascontiguousarray(wq)
    wd = _f32(wd)
    rows, cols = _check_w(qtype, wq, wd)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    xd = _f32(xd)
    m = xq.shape[0]
    assert xq.shape == (m, cols) and xd.shape == (m, cols // QK)
    r0 = 0 if r0 is None else r0
    r1 = rows if r1 is None else r1
    if Y is None:
        Y = np.zeros((m, rows), np.float32)
    f = lib().orc_gemm_q8 if qtype == 8 else lib().orc_gemm_q4
    f(_p(Y), _p(wq), _p(wd), rows, cols, _p(xq), _p(xd), m, r0, r1)
    return Y


def tol_abs(qtype, wq, wd, xq, xd, r0=None, r1=None):
    """A(r) = sum_b |sumi * dw * dx| in float64, for r in [r0, r1)."""
    wq = np.ascontiguousarray(wq)
    wd = _f32(wd)
    rows, cols = _check_w(qtype, wq, wd)
    xq = np.ascontiguousarray(xq, dtype=np.int8).reshape(-1)
    xd = _f32(xd).reshape(-1)
    r0 = 0 if r0 is None else r0
    r1 = rows if r1 is None else r1
    out = np.zeros(r1 - r0, np.float64)
    lib().orc_tol_abs(qtype, _p(wq), _p(wd), cols, _p(xq), _p(xd), r0, r1, _p(out))
    return out


def tolerance(qtype, wq, wd, xq, xd, r0=None, r1=None):
    """Allowed |y - y_ref| per row: 1e-5 * A(r) + 1e-6."""
    return 1e-5 * tol_abs(qtype, wq, wd, xq, xd, r0, r1) + 1e-6


def sumsq(x):
    """The rmsnorm sum of squares in its stated order (pairwise within each
    32-element block, then pairwise over the zero-padded block sums)."""
    x = _f32(x).reshape(-1)
    assert x.size % QK == 0 and x.size > 0
    return np.float32(lib().orc_sumsq(_p(x), x.size))


def rmsnorm(x, w, eps):
    """o_j = w_j * (inv * x_j), inv = 1 / sqrt(sumsq(x) / n + eps), binary32."""
    x = _f32(x).reshape(-1)
    w = _f32(w).reshape(-1)
    assert x.size == w.size and x.size % QK == 0 and x.size > 0
    o = np.empty_like(x)
    lib().orc_rmsnorm(_p(o), _p(x), _p(w), x.size, float(eps))
    return o


def silu_mul(g, u):
    """o_j = (g_j * (1 / (1 + expf(-g_j)))) * u_j in binary32."""
    g = _f32(g).reshape(-1)
    u = _f32(u).reshape(-1)
    assert g.size == u.size
    o = np.empty_like(g)
    lib().orc_silu_mul(_p(o), _p(g), _p(u), g.size)
    return o


# ---------------------------------------------------------------------------
# Block length 128 with a zero point (rules in the C file: "ONNX Runtime"
# page, sections 3 and 4).  Weights: codes uint8 [rows, K] (bits 8) or
# [rows, K/2] (bits 4), scales float32 [rows, K/128], zero points uint8
# [rows, K/128] or None (the midpoint 2^(bits-1)).
BL = 128


def quantize_q8_b128(x):
    """The Q8_0 rule on 128-element blocks: (q int8 of x.shape, d float32
    [..., n/128])."""
    x = _f32(x)
    assert x.shape[-1] % BL == 0
    q = np.empty(x.shape, np.int8)
    d = np.empty(x.shape[:-1] + (x.shape[-1] // BL,), np.float32)
    lib().orc_quantize_q8_b128(_p(x), x.size, _p(q), _p(d))
    return q, d


def _check_zp(bits, wq, wd, wzp):
    rows, nb = wd.shape
    cols = nb * BL
    assert bits in (4, 8)
    assert wq.dtype == np.uint8 and wq.shape == (rows, cols if bits == 8 else cols // 2)
    assert wd.dtype == np.float32
    if wzp is not None:
        assert wzp.dtype == np.uint8 and wzp.shape == (rows, nb)
    return rows, cols


def _zp_ptr(wzp):
    return None if wzp is None else _p(wzp)


def block_sums_zp(bits, wq, wzp, xq, r0=None, r1=None):
    """int32 sumi[r - r0, b] = sum over the block of (code - zp) * q."""
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.int8).reshape(-1)
    cols = xq.size
    rows = wq.shape[0]
    if wzp is not None:
        wzp = np.ascontiguousarray(wzp, dtype=np.uint8)
    r0 = 0 if r0 is None else r0
    r1 = rows if r1 is None else r1
    out = np.zeros((r1 - r0, cols // BL), np.int32)
    lib().orc_block_sums_zp(bits, _p(wq), _zp_ptr(wzp), cols, _p(xq), r0, r1, _p(out))
    return out


def matvec_zp(bits, wq, wd, wzp, xq, xd, r0=None, r1=None, y=None):
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    wd = _f32(wd)
    if wzp is not None:
        wzp = np.ascontiguousarray(wzp, dtype=np.uint8)
    rows, cols = _check_zp(bits, wq, wd, wzp)
    xq = np.ascontiguousarray(xq, dtype=np.int8).reshape(-1)
    xd = _f32(xd).reshape(-1)
    assert xq.size == cols and xd.size == cols // BL
    r0 = 0 if r0 is None else r0
    r1 = rows if r1 is None else r1
    if y is None:
        y = np.zeros(rows, np.float32)
    lib().orc_matvec_zp(_p(y), bits, _p(wq), _p(wd), _zp_ptr(wzp), cols, _p(xq), _p(xd), r0, r1)
    return y


def tolerance_zp(bits, wq, wd, wzp, xq, xd, r0=None, r1=None):
    """Per-row bound 1e-5 * sum_b |sumi * dw * dx| + 1e-6 for rows [r0, r1)."""
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    wd = _f32(wd)
    if wzp is not None:
        wzp = np.ascontiguousarray(wzp, dtype=np.uint8)
    rows, cols = _check_zp(bits, wq, wd, wzp)
    xq = np.ascontiguousarray(xq, dtype=np.int8).reshape(-1)
    xd = _f32(xd).reshape(-1)
    r0 = 0 if r0 is None else r0
    r1 = rows if r1 is None else r1
    out = np.zeros(r1 - r0, np.float64)
    lib().orc_tol_abs_zp(bits, _p(wq), _p(wd), _zp_ptr(wzp), cols, _p(xq), _p(xd), r0, r1, _p(out))
    return 1e-5 * out + 1e-6


# ---------------------------------------------------------------------------
# K-quant super-blocks (rules in the C file: "SKaiNET-native-kernels" page).
# Weights: nibbles uint8 [rows, K/2], sub-block scales and minima uint8
# [rows, K/32] (0..63), super-block scales d and dmin float32 [rows, K/256].
SBK = 256


def quantize_q8_b256(x):
    """The Q8_0 rule on 256-element blocks: (q int8 of x.shape, d float32 [..., n/256])."""
    x = _f32(x)
    assert x.shape[-1] % SBK == 0
    q = np.empty(x.shape, np.int8)
    d = np.empty(x.shape[:-1] + (x.shape[-1] // SBK,), np.float32)
    lib().orc_quantize_q8_b256(_p(x), x.size, _p(q), _p(d))
    return q, d


def _q4k_args(wq, sc, mn, d=None, dmin=None):
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    sc = np.ascontiguousarray(sc, dtype=np.uint8)
    mn = np.ascontiguousarray(mn, dtype=np.uint8)
    rows, nsub = sc.shape
    cols = nsub * QK
    assert cols % SBK == 0 and wq.shape == (rows, cols // 2) and mn.shape == (rows, nsub)
    if d is not None:
        d = _f32(d)
        dmin = _f32(dmin)
        assert d.shape == dmin.shape == (rows, cols // SBK)
    return wq, sc, mn, d, dmin, rows, cols


def superblock_sums_q4k(wq, sc, mn, xq, r0=None, r1=None):
    """(S1, S2) int32 [r1 - r0, K/256]: S1 = sum_b sc_b * sum_i w_i q_i,
    S2 = sum_b mn_b * sum_i q_i."""
    wq, sc, mn, _, _, rows, cols = _q4k_args(wq, sc, mn)
    xq = np.ascontiguousarray(xq, dtype=np.int8).reshape(-1)
    assert xq.size == cols
    r0 = 0 if r0 is None else r0
    r1 = rows if r1 is None else r1
    s1 = np.zeros((r1 - r0, cols // SBK), np.int32)
    s2 = np.zeros((r1 - r0, cols // SBK), np.int32)
    lib().orc_superblock_sums_q4k(_p(wq), _p(sc), _p(mn), cols, _p(xq), r0, r1, _p(s1), _p(s2))
    return s1, s2


def matvec_q4k(wq, sc, mn, d, dmin, xq, xd, r0=None, r1=None, y=None):
    wq, sc, mn, d, dmin, rows, cols = _q4k_args(wq, sc, mn, d, dmin)
    xq = np.ascontiguousarray(xq, dtype=np.int8).reshape(-1)
    xd = _f32(xd).reshape(-1)
    assert xq.size == cols and xd.size == cols // SBK
    r0 = 0 if r0 is None else r0
    r1 = rows if r1 is None else r1
    if y is None:
        y = np.zeros(rows, np.float32)
    lib().orc_matvec_q4k(_p(y), _p(wq), _p(sc), _p(mn), _p(d), _p(dmin), cols, _p(xq), _p(xd), r0, r1)
    return y


def tolerance_q4k(wq, sc, mn, d, dmin, xq, xd, r0=None, r1=None):
    """Per-row bound 1e-5 * sum_k |dx| (|S1 d| + |S2 dmin|) + 1e-6."""
    wq, sc, mn, d, dmin, rows, cols = _q4k_args(wq, sc, mn, d, dmin)
    xq = np.ascontiguousarray(xq, dtype=np.int8).reshape(-1)
    xd = _f32(xd).reshape(-1)
    r0 = 0 if r0 is None else r0
    r1 = rows if r1 is None else r1
    out = np.zeros(r1 - r0, np.float64)
    lib().orc_tol_abs_q4k(_p(wq), _p(sc), _p(mn), _p(d), _p(dmin), cols, _p(xq), _p(xd), r0, r1, _p(out))
    return 1e-5 * out + 1e-6
