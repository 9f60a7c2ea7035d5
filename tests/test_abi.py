"""The C-ABI library on the CPU: it loads, exports every entry point the
public header declares, and rejects bad arguments with the documented
status codes before touching any device.  No compute call runs here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmv.h")
# QMV_ABI_LIB: another build of the same library (the sanitizer tier runs
# these tests against a host-sanitized build)
LIB = os.environ.get("QMV_ABI_LIB") or os.path.join(ROOT, "block_quantized_decode_amd", "libqmv.so")

OK, E_SHAPE, E_FORMAT, E_ARG, E_ARCH, E_DEVICE = range(6)
Q4, Q8 = 4, 8


class QT(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("d", ctypes.c_void_p), ("rows", ctypes.c_int32),
                ("cols", ctypes.c_int32), ("type", ctypes.c_uint8)]


class QA(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("d", ctypes.c_void_p), ("n", ctypes.c_int32)]


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmv_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from block_quantized_decode_amd import build
        build.build()
    L = ctypes.CDLL(LIB)
    for f in declared_functions():
        getattr(L, f).restype = ctypes.c_int
    L.qmv_status_str.restype = ctypes.c_char_p
    L.qmv_last_kernel.restype = ctypes.c_char_p
    return L


def test_header_declares_the_product_calls():
    names = declared_functions()
    for n in ("qmv_quantize_q8", "qmv_quantize_weights", "qmv_matvec_q8", "qmv_matvec_q4",
              "qmv_matvec_q8_fx", "qmv_matvec_q4_fx", "qmv_gemm_q8", "qmv_gemm_q4",
              "qmv_matvec_q8_fx_rmsnorm", "qmv_matvec_q4_fx_rmsnorm",
              "qmv_matvec_q8_fx_silu_mul", "qmv_matvec_q4_fx_silu_mul",
              "qmv_matvec_q8_fx_swiglu", "qmv_matvec_q4_fx_swiglu", "qmv_rmsnorm", "qmv_silu_mul",
              "qmv_pack_bytes", "qmv_pack_weights", "qmv_gemm_q8_packed", "qmv_gemm_q4_packed",
              "qmv_quantize_q8_b128", "qmv_matvec_zp_fx", "qmv_quantize_q8_b256", "qmv_matvec_q4k_fx",
              "qmv_status_str", "qmv_last_kernel", "qmv_device_check"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in qmv.h but not exported"


def test_status_strings(lib):
    for code in range(6):
        assert lib.qmv_status_str(code).decode().startswith("QMV_")
    assert lib.qmv_last_kernel().decode() == ""


# Fake, never-dereferenced addresses: every call below fails validation on
# the host, before any device is queried or any kernel launched.
A = 0x10000          # 64 KiB-aligned
B = 0x20000
Y = 0x30000


def _w(rows=8, cols=64, t=Q8, q=A, d=B):
    return QT(q, d, rows, cols, t)


def _x(n=64, q=A + 0x1000, d=B + 0x1000):
    return QA(q, d, n)


@pytest.mark.parametrize("fn,t", [("qmv_matvec_q8", Q8), ("qmv_matvec_q4", Q4)])
def test_matvec_validation(lib, fn, t):
    f = getattr(lib, fn)
    other = Q4 if t == Q8 else Q8
    W, X = _w(t=t), _x()
    assert f(None, ctypes.byref(W), ctypes.byref(X), 0, 8, None) == E_ARG            # null y
    assert f(Y, None, ctypes.byref(X), 0, 8, None) == E_ARG                          # null W
    assert f(Y, ctypes.byref(W), None, 0, 8, None) == E_ARG                          # null x
    assert f(Y, ctypes.byref(_w(t=other)), ctypes.byref(X), 0, 8, None) == E_FORMAT  # wrong type
    assert f(Y, ctypes.byref(_w(t=7)), ctypes.byref(X), 0, 8, None) == E_FORMAT      # unknown type
    assert f(Y, ctypes.byref(_w(t=t, cols=48)), ctypes.byref(_x(48)), 0, 8, None) == E_SHAPE  # K % 32
    assert f(Y, ctypes.byref(W), ctypes.byref(_x(96)), 0, 8, None) == E_SHAPE       # x->n != K
    assert f(Y, ctypes.byref(W), ctypes.byref(X), -1, 8, None) == E_SHAPE           # r0 < 0
    assert f(Y, ctypes.byref(W), ctypes.byref(X), 0, 9, None) == E_SHAPE            # r1 > rows
    assert f(Y, ctypes.byref(W), ctypes.byref(X), 5, 4, None) == E_SHAPE            # r0 > r1
    big = _w(t=t, cols=32 * 5000)
    assert f(Y, ctypes.byref(big), ctypes.byref(_x(32 * 5000)), 0, 8, None) == E_SHAPE  # beyond LDS limit
    assert f(Y, ctypes.byref(_w(t=t, q=A + 8)), ctypes.byref(X), 0, 8, None) == E_ARG   # q not 16-aligned
    assert f(Y, ctypes.byref(_w(t=t, d=B + 2)), ctypes.byref(X), 0, 8, None) == E_ARG   # d not 4-aligned
    assert f(Y, ctypes.byref(W), ctypes.byref(_x(q=A + 0x1004)), 0, 8, None) == E_ARG  # x q misaligned
    assert f(Y + 2, ctypes.byref(W), ctypes.byref(X), 0, 8, None) == E_ARG            # y misaligned


@pytest.mark.parametrize("fn,t", [("qmv_matvec_q8_fx", Q8), ("qmv_matvec_q4_fx", Q4)])
def test_matvec_fx_validation(lib, fn, t):
    f = getattr(lib, fn)
    W = _w(t=t)
    assert f(Y, ctypes.byref(W), None, None, 0, 8, None) == E_ARG
    assert f(Y, ctypes.byref(W), A + 0x1008, None, 0, 8, None) == E_ARG                # x not 16-aligned
    bad = QA(0, B, 0)
    assert f(Y, ctypes.byref(W), A + 0x1000, ctypes.byref(bad), 0, 8, None) == E_ARG  # xq with null q
    assert f(Y, ctypes.byref(_w(t=Q4 if t == Q8 else Q8)), A + 0x1000, None, 0, 8, None) == E_FORMAT
    assert f(Y, ctypes.byref(W), A + 0x1000, None, 3, 2, None) == E_SHAPE


@pytest.mark.parametrize("fn,t", [("qmv_matvec_q8_fx_rmsnorm", Q8), ("qmv_matvec_q4_fx_rmsnorm", Q4)])
def test_matvec_fx_rmsnorm_validation(lib, fn, t):
    f = getattr(lib, fn)
    P = ctypes.c_void_p
    f.argtypes = [P, P, P, P, ctypes.c_float, P, ctypes.c_int32, ctypes.c_int32, P]
    W = _w(t=t)
    X, N = A + 0x1000, A + 0x2000
    assert f(Y, ctypes.byref(W), None, N, 1e-5, None, 0, 8, None) == E_ARG                 # null x
    assert f(Y, ctypes.byref(W), X, None, 1e-5, None, 0, 8, None) == E_ARG                 # null w_norm
    for eps in (-1.0, float("nan"), float("inf")):
        assert f(Y, ctypes.byref(W), X, N, eps, None, 0, 8, None) == E_ARG, eps
    assert f(Y, ctypes.byref(W), X, N + 4, 1e-5, None, 0, 8, None) == E_ARG               # w_norm misaligned
    assert f(Y, ctypes.byref(W), X + 8, N, 1e-5, None, 0, 8, None) == E_ARG               # x misaligned
    assert f(Y, ctypes.byref(W), X, N, 1e-5, ctypes.byref(QA(0, B, 0)), 0, 8, None) == E_ARG
    assert f(Y, ctypes.byref(_w(t=Q4 if t == Q8 else Q8)), X, N, 1e-5, None, 0, 8, None) == E_FORMAT
    assert f(Y, ctypes.byref(_w(t=t, cols=32 * 945)), X, N, 1e-5, None, 0, 8, None) == E_SHAPE  # beyond LDS
    st = lib.qmv_device_check()
    for cols in (32 * 33, 32 * 63, 32 * 513, 32 * 944):   # every K up to the LDS budget passes the checks
        assert f(Y, ctypes.byref(_w(t=t, cols=cols)), X, N, 1e-5, None, 3, 3, None) in (st, OK), cols
    assert f(Y, ctypes.byref(W), X, N, 1e-5, None, 3, 2, None) == E_SHAPE


@pytest.mark.parametrize("fn,t", [("qmv_matvec_q8_fx_silu_mul", Q8), ("qmv_matvec_q4_fx_silu_mul", Q4)])
def test_matvec_fx_silu_mul_validation(lib, fn, t):
    f = getattr(lib, fn)
    P = ctypes.c_void_p
    f.argtypes = [P, P, P, P, P, ctypes.c_int32, ctypes.c_int32, P]
    W = _w(t=t)
    G, U = A + 0x1000, A + 0x2000
    assert f(Y, ctypes.byref(W), None, U, None, 0, 8, None) == E_ARG                      # null g
    assert f(Y, ctypes.byref(W), G, None, None, 0, 8, None) == E_ARG                      # null u
    assert f(Y, ctypes.byref(W), G + 4, U, None, 0, 8, None) == E_ARG                     # g misaligned
    assert f(Y, ctypes.byref(W), G, U + 8, None, 0, 8, None) == E_ARG                     # u misaligned
    assert f(Y, ctypes.byref(W), G, U, ctypes.byref(QA(A, 0, 0)), 0, 8, None) == E_ARG    # xq with null d
    assert f(Y, ctypes.byref(_w(t=Q4 if t == Q8 else Q8)), G, U, None, 0, 8, None) == E_FORMAT
    assert f(Y, ctypes.byref(_w(t=t, cols=32 * 961)), G, U, None, 0, 8, None) == E_SHAPE   # beyond LDS
    st = lib.qmv_device_check()
    for cols in (32 * 33, 32 * 63, 32 * 513, 32 * 960):
        assert f(Y, ctypes.byref(_w(t=t, cols=cols)), G, U, None, 3, 3, None) in (st, OK), cols
    assert f(Y, ctypes.byref(W), G, U, None, 0, 9, None) == E_SHAPE


@pytest.mark.parametrize("fn,t", [("qmv_matvec_q8_fx_swiglu", Q8), ("qmv_matvec_q4_fx_swiglu", Q4)])
def test_matvec_fx_swiglu_validation(lib, fn, t):
    f = getattr(lib, fn)
    P = ctypes.c_void_p
    f.argtypes = [P, P, P, P, P, ctypes.c_float, P, ctypes.c_int32, ctypes.c_int32, P]
    W = _w(t=t)                       # 8 rows: F = 4 pairs
    X, N, Ya = A + 0x1000, A + 0x2000, Y + 0x1000
    assert f(Ya, Y, ctypes.byref(W), None, N, 1e-5, None, 0, 4, None) == E_ARG            # null x
    assert f(None, Y, ctypes.byref(W), X, N, 1e-5, None, 0, 4, None) == E_ARG              # null a
    assert f(Ya, None, ctypes.byref(W), X, N, 1e-5, None, 0, 4, None) == E_ARG             # null y
    assert f(Ya + 2, Y, ctypes.byref(W), X, N, 1e-5, None, 0, 4, None) == E_ARG            # a misaligned
    for eps in (-1.0, float("nan"), float("inf")):
        assert f(Ya, Y, ctypes.byref(W), X, N, eps, None, 0, 4, None) == E_ARG, eps
    assert f(Ya, Y, ctypes.byref(W), X, N + 4, 1e-5, None, 0, 4, None) == E_ARG           # w_norm misaligned
    assert f(Ya, Y, ctypes.byref(W), X + 8, None, 0.0, None, 0, 4, None) == E_ARG          # x misaligned
    assert f(Ya, Y, ctypes.byref(W), X, N, 1e-5, ctypes.byref(QA(0, B, 0)), 0, 4, None) == E_ARG
    assert f(Ya, Y, ctypes.byref(_w(t=Q4 if t == Q8 else Q8)), X, N, 1e-5, None, 0, 4, None) == E_FORMAT
    assert f(Ya, Y, ctypes.byref(_w(rows=7, t=t)), X, N, 1e-5, None, 0, 3, None) == E_SHAPE   # odd rows
    assert f(Ya, Y, ctypes.byref(W), X, N, 1e-5, None, 0, 5, None) == E_SHAPE              # p1 > F
    assert f(Ya, Y, ctypes.byref(W), X, N, 1e-5, None, -1, 2, None) == E_SHAPE
    assert f(Ya, Y, ctypes.byref(W), X, N, 1e-5, None, 3, 2, None) == E_SHAPE
    assert f(Ya, Y, ctypes.byref(_w(t=t, cols=32 * 945)), X, N, 1e-5, None, 0, 4, None) == E_SHAPE
    st = lib.qmv_device_check()
    assert f(Ya, Y, ctypes.byref(_w(t=t, cols=32 * 960)), X, None, 0.0, None, 0, 0, None) in (st, OK)
    assert f(None, None, ctypes.byref(QT(0, 0, 0, 64, t)), X, None, 0.0, None, 0, 0, None) in (st, OK)


def test_neighbour_validation(lib):
    P = ctypes.c_void_p
    f = lib.qmv_rmsnorm
    f.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_float, P]
    O, X, N = Y, A + 0x1000, A + 0x2000
    assert f(None, X, N, 64, 1e-5, None) == E_ARG
    assert f(O, None, N, 64, 1e-5, None) == E_ARG
    assert f(O, X, None, 64, 1e-5, None) == E_ARG
    for n in (0, -32, 48, 131072 + 32):
        assert f(O, X, N, n, 1e-5, None) == E_SHAPE, n
    for eps in (-1.0, float("nan"), float("inf")):
        assert f(O, X, N, 64, eps, None) == E_ARG, eps
    assert f(O + 4, X, N, 64, 1e-5, None) == E_ARG
    assert f(O, X + 8, N, 64, 1e-5, None) == E_ARG
    assert f(O, X, N + 4, 64, 1e-5, None) == E_ARG
    g = lib.qmv_silu_mul
    g.argtypes = [P, P, P, ctypes.c_int64, P]
    assert g(None, None, None, 0, None) == OK                      # n = 0: nothing to do
    assert g(O, X, N, -1, None) == E_SHAPE
    assert g(O, X, N, 2 ** 31, None) == E_SHAPE
    assert g(None, X, N, 5, None) == E_ARG
    assert g(O, None, N, 5, None) == E_ARG
    assert g(O, X, None, 5, None) == E_ARG
    assert g(O + 4, X, N, 5, None) == E_ARG
    st = lib.qmv_device_check()
    if st != OK:
        assert f(O, X, N, 96, 0.0, None) == st
        assert g(O, X, N, 5, None) == st


@pytest.mark.parametrize("fn,t", [("qmv_gemm_q8", Q8), ("qmv_gemm_q4", Q4)])
def test_gemm_validation(lib, fn, t):
    f = getattr(lib, fn)
    W = _w(t=t)
    X = QT(A + 0x1000, B + 0x1000, 4, 64, Q8)
    assert f(None, ctypes.byref(W), ctypes.byref(X), 0, 8, None) == E_ARG
    assert f(Y, ctypes.byref(W), None, 0, 8, None) == E_ARG
    assert f(Y, ctypes.byref(W), ctypes.byref(QT(A, B, 4, 64, Q4)), 0, 8, None) == E_FORMAT  # X must be Q8_0
    assert f(Y, ctypes.byref(W), ctypes.byref(QT(A, B, 4, 96, Q8)), 0, 8, None) == E_SHAPE  # K mismatch
    assert f(Y, ctypes.byref(W), ctypes.byref(QT(A, B, 0, 64, Q8)), 0, 8, None) == E_SHAPE  # M = 0
    assert f(Y, ctypes.byref(W), ctypes.byref(X), 0, 9, None) == E_SHAPE
    assert f(Y, ctypes.byref(W), ctypes.byref(QT(A + 4, B, 4, 64, Q8)), 0, 8, None) == E_ARG


def test_pack_bytes(lib):
    """Sizes of the packed layout: ceil(rows / 16) tiles x ceil(cols / 128)
    units of 1024 (Q4_0) or 2048 (Q8_0) bytes of quants and 256 of scales."""
    qb, db = ctypes.c_int64(-1), ctypes.c_int64(-1)
    f = lib.qmv_pack_bytes
    for t, rows, cols, want_q, want_d in ((Q4, 16, 128, 1024, 256), (Q8, 16, 128, 2048, 256),
                                          (Q4, 17, 160, 4 * 1024, 4 * 256), (Q8, 1, 32, 2048, 256),
                                          (Q4, 11008, 4096, 688 * 32 * 1024, 688 * 32 * 256),
                                          (Q8, 0, 64, 0, 0)):
        assert f(t, rows, cols, ctypes.byref(qb), ctypes.byref(db)) == OK
        assert (qb.value, db.value) == (want_q, want_d), (t, rows, cols)
    assert f(Q4, 16, 128, None, ctypes.byref(db)) == E_ARG
    assert f(5, 16, 128, ctypes.byref(qb), ctypes.byref(db)) == E_FORMAT
    for rows, cols in ((-1, 128), (16, 0), (16, 100), (16, 131072 + 32)):
        assert f(Q4, rows, cols, ctypes.byref(qb), ctypes.byref(db)) == E_SHAPE, (rows, cols)


@pytest.mark.parametrize("fn,t", [("qmv_gemm_q8_packed", Q8), ("qmv_gemm_q4_packed", Q4)])
def test_gemm_packed_validation(lib, fn, t):
    f = getattr(lib, fn)
    P = QT(A + 0x4000, B + 0x4000, 40, 64, t)  # qmv_packed has the layout of qmv_qtensor
    X = QT(A + 0x1000, B + 0x1000, 20, 64, Q8)
    assert f(None, ctypes.byref(P), ctypes.byref(X), 0, 40, None) == E_ARG
    assert f(Y, None, ctypes.byref(X), 0, 40, None) == E_ARG
    assert f(Y, ctypes.byref(QT(0, B, 40, 64, t)), ctypes.byref(X), 0, 40, None) == E_ARG
    assert f(Y, ctypes.byref(QT(A, B, 40, 64, 12 - t)), ctypes.byref(X), 0, 40, None) == E_FORMAT
    assert f(Y, ctypes.byref(P), ctypes.byref(QT(A, B, 20, 64, Q4)), 0, 40, None) == E_FORMAT
    assert f(Y, ctypes.byref(P), ctypes.byref(QT(A, B, 20, 96, Q8)), 0, 40, None) == E_SHAPE  # K mismatch
    assert f(Y, ctypes.byref(P), ctypes.byref(X), 8, 40, None) == E_SHAPE   # r0 not a multiple of 16
    assert f(Y, ctypes.byref(P), ctypes.byref(X), 0, 41, None) == E_SHAPE
    assert f(Y, ctypes.byref(QT(A, B + 4, 40, 64, t)), ctypes.byref(X), 0, 40, None) == E_ARG  # scales 16-aligned
    W = _w(t=t)
    assert lib.qmv_pack_weights(None, ctypes.byref(W), None) == E_ARG
    assert lib.qmv_pack_weights(ctypes.byref(QT(A + 8, B, 0, 0, 0)), ctypes.byref(W), None) == E_ARG
    assert lib.qmv_pack_weights(ctypes.byref(P), ctypes.byref(_w(t=5)), None) == E_FORMAT
    assert lib.qmv_pack_weights(ctypes.byref(P), ctypes.byref(_w(t=t, cols=33)), None) == E_SHAPE


class ZT(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("d", ctypes.c_void_p), ("zp", ctypes.c_void_p), ("rows", ctypes.c_int32),
                ("cols", ctypes.c_int32), ("bits", ctypes.c_uint8)]


@pytest.mark.parametrize("bits", [4, 8])
def test_matvec_zp_validation(lib, bits):
    f = lib.qmv_matvec_zp_fx
    P = ctypes.c_void_p
    f.argtypes = [P, P, P, P, ctypes.c_int32, ctypes.c_int32, P]
    Wz = ZT(A, B, A + 0x8000, 8, 256, bits)
    X = A + 0x1000
    assert f(None, ctypes.byref(Wz), X, None, 0, 8, None) == E_ARG
    assert f(Y, None, X, None, 0, 8, None) == E_ARG
    assert f(Y, ctypes.byref(Wz), None, None, 0, 8, None) == E_ARG
    assert f(Y, ctypes.byref(ZT(0, B, 0, 8, 256, bits)), X, None, 0, 8, None) == E_ARG
    assert f(Y, ctypes.byref(ZT(A, B, 0, 8, 256, 5)), X, None, 0, 8, None) == E_FORMAT
    for cols in (0, 64, 200, 65536 + 128):
        assert f(Y, ctypes.byref(ZT(A, B, 0, 8, cols, bits)), X, None, 0, 8, None) == E_SHAPE, cols
    big = (1 << 31) // (65536 if bits == 8 else 32768) + 1   # rows * row bytes past INT32_MAX
    assert f(Y, ctypes.byref(ZT(A, B, 0, big, 65536, bits)), X, None, 0, 8, None) == E_SHAPE
    assert f(Y, ctypes.byref(Wz), X, None, 0, 9, None) == E_SHAPE
    assert f(Y, ctypes.byref(Wz), X, None, 5, 4, None) == E_SHAPE
    assert f(Y, ctypes.byref(ZT(A + 8, B, 0, 8, 256, bits)), X, None, 0, 8, None) == E_ARG   # q 16-aligned
    assert f(Y, ctypes.byref(Wz), X + 8, None, 0, 8, None) == E_ARG                         # x 16-aligned
    act = QA(A + 8, B, 0)
    assert f(Y, ctypes.byref(Wz), X, ctypes.byref(act), 0, 8, None) == E_ARG
    g = lib.qmv_quantize_q8_b128
    g.argtypes = [P, P, ctypes.c_int64, P]
    act = QA(A, B, 0)
    assert g(ctypes.byref(act), Y, 96, None) == E_SHAPE
    assert g(None, Y, 128, None) == E_ARG
    empty = QA(0, 0, 7)
    assert g(ctypes.byref(empty), None, 0, None) == OK and empty.n == 0


class KT(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("sc", ctypes.c_void_p), ("mn", ctypes.c_void_p), ("d", ctypes.c_void_p),
                ("dmin", ctypes.c_void_p), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


def _kt(rows=8, cols=512, q=A, sc=A + 0x4000, mn=A + 0x5000, d=B, dmin=B + 0x100):
    return KT(q, sc, mn, d, dmin, rows, cols)


def test_matvec_q4k_validation(lib):
    f = lib.qmv_matvec_q4k_fx
    P = ctypes.c_void_p
    f.argtypes = [P, P, P, P, ctypes.c_int32, ctypes.c_int32, P]
    X = A + 0x1000
    assert f(None, ctypes.byref(_kt()), X, None, 0, 8, None) == E_ARG
    assert f(Y, None, X, None, 0, 8, None) == E_ARG
    assert f(Y, ctypes.byref(_kt()), None, None, 0, 8, None) == E_ARG
    for field in ("q", "sc", "mn", "d", "dmin"):
        assert f(Y, ctypes.byref(_kt(**{field: 0})), X, None, 0, 8, None) == E_ARG, field
    for cols in (0, 128, 300, 65536 + 256):
        assert f(Y, ctypes.byref(_kt(cols=cols)), X, None, 0, 8, None) == E_SHAPE, cols
    assert f(Y, ctypes.byref(_kt()), X, None, 0, 9, None) == E_SHAPE
    assert f(Y, ctypes.byref(_kt()), X, None, 3, 2, None) == E_SHAPE
    assert f(Y, ctypes.byref(_kt(q=A + 8)), X, None, 0, 8, None) == E_ARG
    assert f(Y, ctypes.byref(_kt()), X + 4, None, 0, 8, None) == E_ARG
    assert f(Y, ctypes.byref(_kt(d=B + 2)), X, None, 0, 8, None) == E_ARG
    g = lib.qmv_quantize_q8_b256
    g.argtypes = [P, P, ctypes.c_int64, P]
    assert g(ctypes.byref(QA(A, B, 0)), Y, 128, None) == E_SHAPE
    assert g(None, Y, 256, None) == E_ARG
    empty = QA(0, 0, 7)
    assert g(ctypes.byref(empty), None, 0, None) == OK and empty.n == 0


def test_zero_rows_accept_null_pointers(lib):
    """A matrix without rows may have null data pointers (and a null output):
    the calls get past argument checking, to the device check (QMV_E_DEVICE
    or QMV_E_ARCH here), or return QMV_OK where a gfx950 is present."""
    P = ctypes.c_void_p
    fine = (OK, E_DEVICE, E_ARCH)
    W0 = QT(0, 0, 0, 64, Q8)
    X = QT(A + 0x1000, B + 0x1000, 20, 64, Q8)
    assert lib.qmv_matvec_q8(None, ctypes.byref(W0), ctypes.byref(_x()), 0, 0, None) in fine
    assert lib.qmv_gemm_q8(None, ctypes.byref(W0), ctypes.byref(X), 0, 0, None) in fine
    assert lib.qmv_quantize_weights(ctypes.byref(W0), None, None) in fine
    assert lib.qmv_pack_weights(ctypes.byref(QT(0, 0, 0, 0, 0)), ctypes.byref(W0), None) in fine
    assert lib.qmv_gemm_q8_packed(None, ctypes.byref(QT(0, 0, 0, 64, Q8)), ctypes.byref(X), 0, 0, None) in fine
    f = lib.qmv_matvec_zp_fx
    f.argtypes = [P, P, P, P, ctypes.c_int32, ctypes.c_int32, P]
    assert f(None, ctypes.byref(ZT(0, 0, 0, 0, 256, 8)), A + 0x1000, None, 0, 0, None) in fine
    f = lib.qmv_matvec_q4k_fx
    f.argtypes = [P, P, P, P, ctypes.c_int32, ctypes.c_int32, P]
    assert f(None, ctypes.byref(KT(0, 0, 0, 0, 0, 0, 512)), A + 0x1000, None, 0, 0, None) in fine
    # with rows, null pointers are still refused
    assert lib.qmv_matvec_q8(Y, ctypes.byref(QT(0, 0, 8, 64, Q8)), ctypes.byref(_x()), 0, 0, None) == E_ARG
    assert lib.qmv_matvec_q8(None, ctypes.byref(_w()), ctypes.byref(_x()), 0, 0, None) == E_ARG


def test_quantize_validation(lib):
    act = QA(A, B, 0)
    assert lib.qmv_quantize_q8(None, ctypes.c_void_p(Y), ctypes.c_int64(64), None) == E_ARG
    assert lib.qmv_quantize_q8(ctypes.byref(act), None, ctypes.c_int64(64), None) == E_ARG
    empty = QA(0, 0, 5)
    assert lib.qmv_quantize_q8(ctypes.byref(empty), None, ctypes.c_int64(0), None) == OK  # k = 0: nothing to do
    assert empty.n == 0
    assert lib.qmv_quantize_q8(ctypes.byref(act), ctypes.c_void_p(Y), ctypes.c_int64(40), None) == E_SHAPE
    assert lib.qmv_quantize_q8(ctypes.byref(act), ctypes.c_void_p(Y), ctypes.c_int64(-32), None) == E_SHAPE
    assert lib.qmv_quantize_q8(ctypes.byref(act), ctypes.c_void_p(Y + 4), ctypes.c_int64(64), None) == E_ARG
    W = _w(t=Q4)
    assert lib.qmv_quantize_weights(ctypes.byref(W), None, None) == E_ARG
    assert lib.qmv_quantize_weights(ctypes.byref(_w(t=5)), ctypes.c_void_p(Y), None) == E_FORMAT
    assert lib.qmv_quantize_weights(ctypes.byref(_w(t=Q8, cols=33)), ctypes.c_void_p(Y), None) == E_SHAPE


def test_no_device_is_an_error_not_a_crash(lib):
    """Valid arguments on a machine without a usable GPU: the device check
    reports QMV_E_DEVICE (or QMV_E_ARCH on a non-gfx950 GPU) and nothing is
    launched.  Skipped where a gfx950 is present, since the fake pointers
    would then be used."""
    st = lib.qmv_device_check()
    if st == OK:
        pytest.skip("a gfx950 device is present")
    assert st in (E_DEVICE, E_ARCH)
    W, X = _w(t=Q8), _x()
    assert lib.qmv_matvec_q8(Y, ctypes.byref(W), ctypes.byref(X), 0, 8, None) == st
    assert lib.qmv_matvec_q4_fx(Y, ctypes.byref(_w(t=Q4)), A + 0x1000, None, 0, 8, None) == st
    f = lib.qmv_matvec_q8_fx_rmsnorm
    P = ctypes.c_void_p
    f.argtypes = [P, P, P, P, ctypes.c_float, P, ctypes.c_int32, ctypes.c_int32, P]
    assert f(Y, ctypes.byref(W), A + 0x1000, A + 0x2000, 1e-5, None, 0, 8, None) == st
    f = lib.qmv_matvec_q8_fx_silu_mul
    f.argtypes = [P, P, P, P, P, ctypes.c_int32, ctypes.c_int32, P]
    assert f(Y, ctypes.byref(W), A + 0x1000, A + 0x2000, None, 0, 8, None) == st
    act = QA(A, B, 0)
    assert lib.qmv_quantize_q8(ctypes.byref(act), ctypes.c_void_p(Y), ctypes.c_int64(64), None) == st
    PK = QT(A + 0x4000, B + 0x4000, 0, 0, 0)
    assert lib.qmv_pack_weights(ctypes.byref(PK), ctypes.byref(W), None) == st
    PK = QT(A + 0x4000, B + 0x4000, 8, 64, Q8)
    assert lib.qmv_gemm_q8_packed(Y, ctypes.byref(PK), ctypes.byref(QT(A + 0x1000, B + 0x1000, 20, 64, Q8)),
                                  0, 8, None) == st
    f = lib.qmv_matvec_zp_fx
    f.argtypes = [P, P, P, P, ctypes.c_int32, ctypes.c_int32, P]
    assert f(Y, ctypes.byref(ZT(A, B, 0, 8, 256, 8)), A + 0x1000, None, 0, 8, None) == st
    g = lib.qmv_quantize_q8_b128
    g.argtypes = [P, P, ctypes.c_int64, P]
    assert g(ctypes.byref(QA(A, B, 0)), Y, 128, None) == st
    f = lib.qmv_matvec_q4k_fx
    f.argtypes = [P, P, P, P, ctypes.c_int32, ctypes.c_int32, P]
    assert f(Y, ctypes.byref(_kt()), A + 0x1000, None, 0, 8, None) == st
    assert lib.qmv_last_kernel().decode() == ""


def test_ceiling_validation(lib):
    """The measurement entry points check their arguments like the rest."""
    P = ctypes.c_void_p
    f = lib.qmv_ceiling_stream_read
    f.argtypes = [P, P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P]
    assert f(None, A, 1024, 4, 4, None) == E_ARG
    assert f(Y, None, 1024, 4, 4, None) == E_ARG
    assert f(Y, A + 8, 1024, 4, 4, None) == E_ARG        # buffer not 16-byte aligned
    assert f(Y, A, 1024, 4, 3, None) == E_ARG            # depth 4 or 8
    assert f(Y, A, 1000, 4, 4, None) == E_SHAPE          # not a multiple of 16
    assert f(Y, A, 0, 4, 4, None) == E_SHAPE
    assert f(Y, A, 1024, 0, 4, None) == E_SHAPE
    assert f(Y, A, 1024, 65537, 4, None) == E_SHAPE
    g = lib.qmv_ceiling_mfma_i8
    g.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P]
    assert g(None, 0, 10, 4, 1, 1, None) == E_ARG
    assert g(Y + 2, 0, 10, 4, 1, 1, None) == E_ARG
    assert g(Y, 3, 10, 4, 1, 1, None) == E_ARG           # shape 0..2
    assert g(Y, 0, -1, 4, 1, 1, None) == E_SHAPE
    assert g(Y, 0, 10, 0, 1, 1, None) == E_SHAPE
    st = lib.qmv_device_check()
    if st != OK:
        assert f(Y, A, 1024, 4, 4, None) == st
        assert g(Y, 1, 10, 4, 1, 1, None) == st
