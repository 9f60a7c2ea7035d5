"""Thin ctypes binding of libqmv (include/qmv.h).

Argument marshalling only: torch tensors are passed as device pointers with
the current HIP stream; every step of the computation runs in the library's
gfx950 kernels.  There is no CPU or PyTorch fallback: if libqmv.so has not
been built, or a call fails, an exception is raised.

Function names follow the C ABI (qmv_quantize_q8, qmv_matvec_q4_fx, ...).
Tensors hold the SoA formats of the header: a Q4_0 matrix is
(q: uint8 or int8 [rows, K/2], d: float32 [rows, K/32]); a Q8_0 matrix or
activation is (q: int8 [..., K], d: float32 [..., K/32]).
"""
from __future__ import annotations

import ctypes
import os

import torch

QK = 32
QMV_Q4_0 = 4
QMV_Q8_0 = 8

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmv.so")

STATUS = {0: "QMV_OK", 1: "QMV_E_SHAPE", 2: "QMV_E_FORMAT", 3: "QMV_E_ARG", 4: "QMV_E_ARCH",
          5: "QMV_E_DEVICE"}


class QmvError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)}")


class QTensor(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("d", ctypes.c_void_p), ("rows", ctypes.c_int32),
                ("cols", ctypes.c_int32), ("type", ctypes.c_uint8)]


class QAct(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("d", ctypes.c_void_p), ("n", ctypes.c_int32)]


class ZpTensor(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("d", ctypes.c_void_p), ("zp", ctypes.c_void_p), ("rows", ctypes.c_int32),
                ("cols", ctypes.c_int32), ("bits", ctypes.c_uint8)]


class Q4kTensor(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("sc", ctypes.c_void_p), ("mn", ctypes.c_void_p), ("d", ctypes.c_void_p),
                ("dmin", ctypes.c_void_p), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


class Packed(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("d", ctypes.c_void_p), ("rows", ctypes.c_int32),
                ("cols", ctypes.c_int32), ("type", ctypes.c_uint8)]


_lib = None

# name -> argtypes (restype c_int = qmv_status)
_P = ctypes.c_void_p
_SIGS = {
    "qmv_quantize_q8": [ctypes.POINTER(QAct), _P, ctypes.c_int64, _P],
    "qmv_quantize_weights": [ctypes.POINTER(QTensor), _P, _P],
    "qmv_matvec_q8": [_P, ctypes.POINTER(QTensor), ctypes.POINTER(QAct), ctypes.c_int32, ctypes.c_int32, _P],
    "qmv_matvec_q4": [_P, ctypes.POINTER(QTensor), ctypes.POINTER(QAct), ctypes.c_int32, ctypes.c_int32, _P],
    "qmv_matvec_q8_fx": [_P, ctypes.POINTER(QTensor), _P, ctypes.POINTER(QAct), ctypes.c_int32, ctypes.c_int32, _P],
    "qmv_matvec_q4_fx": [_P, ctypes.POINTER(QTensor), _P, ctypes.POINTER(QAct), ctypes.c_int32, ctypes.c_int32, _P],
    "qmv_matvec_q8_fx_rmsnorm": [_P, ctypes.POINTER(QTensor), _P, _P, ctypes.c_float, ctypes.POINTER(QAct),
                                 ctypes.c_int32, ctypes.c_int32, _P],
    "qmv_matvec_q4_fx_rmsnorm": [_P, ctypes.POINTER(QTensor), _P, _P, ctypes.c_float, ctypes.POINTER(QAct),
                                 ctypes.c_int32, ctypes.c_int32, _P],
    "qmv_matvec_q8_fx_silu_mul": [_P, ctypes.POINTER(QTensor), _P, _P, ctypes.POINTER(QAct), ctypes.c_int32,
                                  ctypes.c_int32, _P],
    "qmv_matvec_q4_fx_silu_mul": [_P, ctypes.POINTER(QTensor), _P, _P, ctypes.POINTER(QAct), ctypes.c_int32,
                                  ctypes.c_int32, _P],
    "qmv_matvec_q8_fx_swiglu": [_P, _P, ctypes.POINTER(QTensor), _P, _P, ctypes.c_float, ctypes.POINTER(QAct),
                                ctypes.c_int32, ctypes.c_int32, _P],
    "qmv_matvec_q4_fx_swiglu": [_P, _P, ctypes.POINTER(QTensor), _P, _P, ctypes.c_float, ctypes.POINTER(QAct),
                                ctypes.c_int32, ctypes.c_int32, _P],
    "qmv_gemm_q8": [_P, ctypes.POINTER(QTensor), ctypes.POINTER(QTensor), ctypes.c_int32, ctypes.c_int32, _P],
    "qmv_gemm_q4": [_P, ctypes.POINTER(QTensor), ctypes.POINTER(QTensor), ctypes.c_int32, ctypes.c_int32, _P],
    "qmv_pack_bytes": [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                       ctypes.POINTER(ctypes.c_int64)],
    "qmv_pack_weights": [ctypes.POINTER(Packed), ctypes.POINTER(QTensor), _P],
    "qmv_gemm_q8_packed": [_P, ctypes.POINTER(Packed), ctypes.POINTER(QTensor), ctypes.c_int32, ctypes.c_int32, _P],
    "qmv_gemm_q4_packed": [_P, ctypes.POINTER(Packed), ctypes.POINTER(QTensor), ctypes.c_int32, ctypes.c_int32, _P],
    "qmv_quantize_q8_b128": [ctypes.POINTER(QAct), _P, ctypes.c_int64, _P],
    "qmv_matvec_zp_fx": [_P, ctypes.POINTER(ZpTensor), _P, ctypes.POINTER(QAct), ctypes.c_int32, ctypes.c_int32, _P],
    "qmv_quantize_q8_b256": [ctypes.POINTER(QAct), _P, ctypes.c_int64, _P],
    "qmv_matvec_q4k_fx": [_P, ctypes.POINTER(Q4kTensor), _P, ctypes.POINTER(QAct), ctypes.c_int32, ctypes.c_int32,
                          _P],
    "qmv_device_check": [],
    "qmv_rmsnorm": [_P, _P, _P, ctypes.c_int64, ctypes.c_float, _P],
    "qmv_silu_mul": [_P, _P, _P, ctypes.c_int64, _P],
    "qmv_ceiling_stream_read": [_P, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P],
    "qmv_ceiling_mfma_i8": [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P],
}


def lib() -> ctypes.CDLL:
    """Load the in-tree libqmv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_quantized_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.qmv_status_str.argtypes = [ctypes.c_int]
        L.qmv_status_str.restype = ctypes.c_char_p
        L.qmv_last_kernel.argtypes = []
        L.qmv_last_kernel.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(code: int, where: str):
    if code != 0:
        raise QmvError(code, where)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, dtype=None):
    if not t.is_cuda:
        raise ValueError("libqmv takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libqmv takes contiguous tensors")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"expected {dtype}, got {t.dtype}")
    return t


def qtensor(q: torch.Tensor, d: torch.Tensor, qtype: int) -> QTensor:
    """Describe a device Q4_0/Q8_0 matrix (q, d) for the C ABI."""
    _dev(q, (torch.int8, torch.uint8))
    _dev(d, torch.float32)
    rows = d.shape[0]
    cols = d.shape[-1] * QK
    return QTensor(q.data_ptr(), d.data_ptr(), rows, cols, qtype)


def last_kernel() -> str:
    return lib().qmv_last_kernel().decode()


def status_str(code: int) -> str:
    return lib().qmv_status_str(code).decode()


def qmv_device_check() -> None:
    _check(lib().qmv_device_check(), "qmv_device_check")


def qmv_quantize_q8(x: torch.Tensor, q: torch.Tensor | None = None, d: torch.Tensor | None = None):
    """Q8_0-quantize a float32 device tensor whose last dim is a multiple of
    32.  Returns (q int8 like x, d float32 [..., K/32])."""
    _dev(x, torch.float32)
    if q is None:
        q = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    if d is None:
        d = torch.empty(x.shape[:-1] + (x.shape[-1] // QK,), dtype=torch.float32, device=x.device)
    act = QAct(q.data_ptr(), d.data_ptr(), 0)
    _check(lib().qmv_quantize_q8(ctypes.byref(act), x.data_ptr(), x.numel(), _stream()), "qmv_quantize_q8")
    return q, d


def qmv_quantize_weights(w: torch.Tensor, qtype: int, q: torch.Tensor | None = None,
                         d: torch.Tensor | None = None):
    """Quantize a float32 [rows, K] device matrix to Q4_0 or Q8_0."""
    _dev(w, torch.float32)
    rows, cols = w.shape
    if q is None:
        q = torch.empty((rows, cols // 2 if qtype == QMV_Q4_0 else cols),
                        dtype=torch.uint8 if qtype == QMV_Q4_0 else torch.int8, device=w.device)
    if d is None:
        d = torch.empty((rows, cols // QK), dtype=torch.float32, device=w.device)
    W = QTensor(q.data_ptr(), d.data_ptr(), rows, cols, qtype)
    _check(lib().qmv_quantize_weights(ctypes.byref(W), w.data_ptr(), _stream()), "qmv_quantize_weights")
    return q, d


def _out(y, n, like):
    if y is None:
        return torch.zeros(n, dtype=torch.float32, device=like.device)
    _dev(y, torch.float32)
    return y


def _matvec(qtype, fname, wq, wd, xq, xd, r0, r1, y):
    W = qtensor(wq, wd, qtype)
    _dev(xq, torch.int8)
    _dev(xd, torch.float32)
    r0 = 0 if r0 is None else r0
    r1 = W.rows if r1 is None else r1
    y = _out(y, W.rows, wd)
    act = QAct(xq.data_ptr(), xd.data_ptr(), xq.numel())
    _check(getattr(lib(), fname)(y.data_ptr(), ctypes.byref(W), ctypes.byref(act), r0, r1, _stream()), fname)
    return y


def qmv_matvec_q8(wq, wd, xq, xd, r0=None, r1=None, y=None):
    return _matvec(QMV_Q8_0, "qmv_matvec_q8", wq, wd, xq, xd, r0, r1, y)


def qmv_matvec_q4(wq, wd, xq, xd, r0=None, r1=None, y=None):
    return _matvec(QMV_Q4_0, "qmv_matvec_q4", wq, wd, xq, xd, r0, r1, y)


def _matvec_fx(qtype, fname, wq, wd, x, r0, r1, y, xq_out):
    W = qtensor(wq, wd, qtype)
    _dev(x, torch.float32)
    r0 = 0 if r0 is None else r0
    r1 = W.rows if r1 is None else r1
    y = _out(y, W.rows, wd)
    act = None
    if xq_out is not None:
        q, d = xq_out
        _dev(q, torch.int8)
        _dev(d, torch.float32)
        act = QAct(q.data_ptr(), d.data_ptr(), 0)
    code = getattr(lib(), fname)(y.data_ptr(), ctypes.byref(W), x.data_ptr(),
                                 ctypes.byref(act) if act is not None else None, r0, r1, _stream())
    _check(code, fname)
    return y


def qmv_matvec_q8_fx(wq, wd, x, r0=None, r1=None, y=None, xq_out=None):
    """y = W x with x float32 quantized inside the kernel.  xq_out, if given,
    is a (q int8 [K], d float32 [K/32]) pair receiving the quantized x."""
    return _matvec_fx(QMV_Q8_0, "qmv_matvec_q8_fx", wq, wd, x, r0, r1, y, xq_out)


def qmv_matvec_q4_fx(wq, wd, x, r0=None, r1=None, y=None, xq_out=None):
    return _matvec_fx(QMV_Q4_0, "qmv_matvec_q4_fx", wq, wd, x, r0, r1, y, xq_out)


def _matvec_fx_rmsnorm(qtype, fname, wq, wd, x, w_norm, eps, r0, r1, y, xq_out):
    W = qtensor(wq, wd, qtype)
    _dev(x, torch.float32)
    _dev(w_norm, torch.float32)
    r0 = 0 if r0 is None else r0
    r1 = W.rows if r1 is None else r1
    y = _out(y, W.rows, wd)
    act = None
    if xq_out is not None:
        q, d = xq_out
        _dev(q, torch.int8)
        _dev(d, torch.float32)
        act = QAct(q.data_ptr(), d.data_ptr(), 0)
    code = getattr(lib(), fname)(y.data_ptr(), ctypes.byref(W), x.data_ptr(), w_norm.data_ptr(), float(eps),
                                 ctypes.byref(act) if act is not None else None, r0, r1, _stream())
    _check(code, fname)
    return y


def qmv_matvec_q8_fx_rmsnorm(wq, wd, x, w_norm, eps, r0=None, r1=None, y=None, xq_out=None):
    """y = W q8(rmsnorm(x) * w_norm) in one launch (see include/qmv.h)."""
    return _matvec_fx_rmsnorm(QMV_Q8_0, "qmv_matvec_q8_fx_rmsnorm", wq, wd, x, w_norm, eps, r0, r1, y, xq_out)


def qmv_matvec_q4_fx_rmsnorm(wq, wd, x, w_norm, eps, r0=None, r1=None, y=None, xq_out=None):
    return _matvec_fx_rmsnorm(QMV_Q4_0, "qmv_matvec_q4_fx_rmsnorm", wq, wd, x, w_norm, eps, r0, r1, y, xq_out)


def _matvec_fx_silu_mul(qtype, fname, wq, wd, g, u, r0, r1, y, xq_out):
    W = qtensor(wq, wd, qtype)
    _dev(g, torch.float32)
    _dev(u, torch.float32)
    r0 = 0 if r0 is None else r0
    r1 = W.rows if r1 is None else r1
    y = _out(y, W.rows, wd)
    act = None
    if xq_out is not None:
        q, d = xq_out
        _dev(q, torch.int8)
        _dev(d, torch.float32)
        act = QAct(q.data_ptr(), d.data_ptr(), 0)
    code = getattr(lib(), fname)(y.data_ptr(), ctypes.byref(W), g.data_ptr(), u.data_ptr(),
                                 ctypes.byref(act) if act is not None else None, r0, r1, _stream())
    _check(code, fname)
    return y


def qmv_matvec_q8_fx_silu_mul(wq, wd, g, u, r0=None, r1=None, y=None, xq_out=None):
    """y = W q8(silu(g) * u) in one launch (see include/qmv.h)."""
    return _matvec_fx_silu_mul(QMV_Q8_0, "qmv_matvec_q8_fx_silu_mul", wq, wd, g, u, r0, r1, y, xq_out)


def qmv_matvec_q4_fx_silu_mul(wq, wd, g, u, r0=None, r1=None, y=None, xq_out=None):
    return _matvec_fx_silu_mul(QMV_Q4_0, "qmv_matvec_q4_fx_silu_mul", wq, wd, g, u, r0, r1, y, xq_out)


def _gemm(qtype, fname, wq, wd, xq, xd, r0, r1, Y):
    W = qtensor(wq, wd, qtype)
    X = qtensor(xq, xd, QMV_Q8_0)
    r0 = 0 if r0 is None else r0
    r1 = W.rows if r1 is None else r1
    if Y is None:
        Y = torch.zeros((X.rows, W.rows), dtype=torch.float32, device=wd.device)
    _dev(Y, torch.float32)
    _check(getattr(lib(), fname)(Y.data_ptr(), ctypes.byref(W), ctypes.byref(X), r0, r1, _stream()), fname)
    return Y


def qmv_gemm_q8(wq, wd, xq, xd, r0=None, r1=None, Y=None):
    """Y[m, r] for all M rows of the Q8_0 activation (xq [M, K], xd [M, K/32])."""
    return _gemm(QMV_Q8_0, "qmv_gemm_q8", wq, wd, xq, xd, r0, r1, Y)


def qmv_gemm_q4(wq, wd, xq, xd, r0=None, r1=None, Y=None):
    return _gemm(QMV_Q4_0, "qmv_gemm_q4", wq, wd, xq, xd, r0, r1, Y)


def qmv_pack_bytes(qtype: int, rows: int, cols: int) -> tuple[int, int]:
    """Bytes of the packed quants and scales of a rows x cols matrix (host only)."""
    qb, db = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().qmv_pack_bytes(qtype, rows, cols, ctypes.byref(qb), ctypes.byref(db)), "qmv_pack_bytes")
    return qb.value, db.value


class PackedWeights:
    """Device weights in the pack-once layout (q: uint8 [q_bytes], d: float32
    [d_bytes / 4]) with their shape; desc is the qmv_packed descriptor."""

    def __init__(self, q: torch.Tensor, d: torch.Tensor, rows: int, cols: int, qtype: int):
        self.q, self.d, self.rows, self.cols, self.qtype = q, d, rows, cols, qtype
        self.desc = Packed(q.data_ptr(), d.data_ptr(), rows, cols, qtype)


def qmv_pack_weights(wq, wd, qtype: int, q: torch.Tensor | None = None,
                     d: torch.Tensor | None = None) -> PackedWeights:
    """Pack a row-major Q4_0 / Q8_0 device matrix (wq, wd) once (see include/qmv.h)."""
    W = qtensor(wq, wd, qtype)
    qb, db = qmv_pack_bytes(qtype, W.rows, W.cols)
    if q is None:
        q = torch.empty(max(qb, 16), dtype=torch.uint8, device=wd.device)
    if d is None:
        d = torch.empty(max(db // 4, 4), dtype=torch.float32, device=wd.device)
    _dev(q, (torch.uint8, torch.int8))
    _dev(d, torch.float32)
    if q.numel() < qb or d.numel() * 4 < db:
        raise ValueError(f"packed buffers too small: need {qb} and {db} bytes")
    P = Packed(q.data_ptr(), d.data_ptr(), 0, 0, 0)
    _check(lib().qmv_pack_weights(ctypes.byref(P), ctypes.byref(W), _stream()), "qmv_pack_weights")
    return PackedWeights(q, d, P.rows, P.cols, P.type)


def _gemm_packed(qtype, fname, P: PackedWeights, xq, xd, r0, r1, Y):
    X = qtensor(xq, xd, QMV_Q8_0)
    r0 = 0 if r0 is None else r0
    r1 = P.rows if r1 is None else r1
    if Y is None:
        Y = torch.zeros((X.rows, P.rows), dtype=torch.float32, device=xd.device)
    _dev(Y, torch.float32)
    _check(getattr(lib(), fname)(Y.data_ptr(), ctypes.byref(P.desc), ctypes.byref(X), r0, r1, _stream()), fname)
    return Y


def qmv_gemm_q8_packed(P: PackedWeights, xq, xd, r0=None, r1=None, Y=None):
    """qmv_gemm_q8 on packed weights (r0 a multiple of 16)."""
    return _gemm_packed(QMV_Q8_0, "qmv_gemm_q8_packed", P, xq, xd, r0, r1, Y)


def qmv_gemm_q4_packed(P: PackedWeights, xq, xd, r0=None, r1=None, Y=None):
    return _gemm_packed(QMV_Q4_0, "qmv_gemm_q4_packed", P, xq, xd, r0, r1, Y)


ZP_BLOCK = 128


def zptensor(q: torch.Tensor, d: torch.Tensor, zp: torch.Tensor | None, bits: int) -> ZpTensor:
    """Describe a device matrix of the 128-block zero-point format: q uint8
    [rows, K] (bits 8) or [rows, K/2] (bits 4), d float32 [rows, K/128], zp
    uint8 [rows, K/128] or None."""
    _dev(q, (torch.uint8, torch.int8))
    _dev(d, torch.float32)
    if zp is not None:
        _dev(zp, (torch.uint8, torch.int8))
    rows = d.shape[0]
    cols = d.shape[-1] * ZP_BLOCK
    return ZpTensor(q.data_ptr(), d.data_ptr(), None if zp is None else zp.data_ptr(), rows, cols, bits)


def qmv_quantize_q8_b128(x: torch.Tensor):
    """The Q8_0 rule on 128-element blocks: (q int8 like x, d float32 [..., K/128])."""
    _dev(x, torch.float32)
    q = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    d = torch.empty(x.shape[:-1] + (x.shape[-1] // ZP_BLOCK,), dtype=torch.float32, device=x.device)
    act = QAct(q.data_ptr(), d.data_ptr(), 0)
    _check(lib().qmv_quantize_q8_b128(ctypes.byref(act), x.data_ptr(), x.numel(), _stream()), "qmv_quantize_q8_b128")
    return q, d


def qmv_matvec_zp_fx(wq, wd, wzp, bits, x, r0=None, r1=None, y=None, xq_out=None):
    """y = W q8_b128(x) on the 128-block zero-point format (see include/qmv.h)."""
    W = zptensor(wq, wd, wzp, bits)
    _dev(x, torch.float32)
    r0 = 0 if r0 is None else r0
    r1 = W.rows if r1 is None else r1
    if y is None:
        y = torch.zeros(W.rows, dtype=torch.float32, device=x.device)
    _dev(y, torch.float32)
    act = None
    if xq_out is not None:
        q, d = xq_out
        act = QAct(_dev(q, torch.int8).data_ptr(), _dev(d, torch.float32).data_ptr(), 0)
    code = lib().qmv_matvec_zp_fx(y.data_ptr(), ctypes.byref(W), x.data_ptr(),
                                  ctypes.byref(act) if act is not None else None, r0, r1, _stream())
    _check(code, "qmv_matvec_zp_fx")
    return y


Q4K_BLOCK = 256


def q4ktensor(q, sc, mn, d, dmin) -> Q4kTensor:
    """Describe a device K-quant matrix: q uint8 [rows, K/2], sc and mn uint8
    [rows, K/32], d and dmin float32 [rows, K/256]."""
    for t in (q, sc, mn):
        _dev(t, (torch.uint8, torch.int8))
    _dev(d, torch.float32)
    _dev(dmin, torch.float32)
    rows = sc.shape[0]
    cols = sc.shape[-1] * QK
    return Q4kTensor(q.data_ptr(), sc.data_ptr(), mn.data_ptr(), d.data_ptr(), dmin.data_ptr(), rows, cols)


def qmv_quantize_q8_b256(x: torch.Tensor):
    """The Q8_0 rule on 256-element blocks: (q int8 like x, d float32 [..., K/256])."""
    _dev(x, torch.float32)
    q = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    d = torch.empty(x.shape[:-1] + (x.shape[-1] // Q4K_BLOCK,), dtype=torch.float32, device=x.device)
    act = QAct(q.data_ptr(), d.data_ptr(), 0)
    _check(lib().qmv_quantize_q8_b256(ctypes.byref(act), x.data_ptr(), x.numel(), _stream()), "qmv_quantize_q8_b256")
    return q, d


def qmv_matvec_q4k_fx(q, sc, mn, d, dmin, x, r0=None, r1=None, y=None, xq_out=None):
    """y = W q8_b256(x) on K-quant super-blocks (see include/qmv.h)."""
    W = q4ktensor(q, sc, mn, d, dmin)
    _dev(x, torch.float32)
    r0 = 0 if r0 is None else r0
    r1 = W.rows if r1 is None else r1
    if y is None:
        y = torch.zeros(W.rows, dtype=torch.float32, device=x.device)
    _dev(y, torch.float32)
    act = None
    if xq_out is not None:
        xq, xd = xq_out
        act = QAct(_dev(xq, torch.int8).data_ptr(), _dev(xd, torch.float32).data_ptr(), 0)
    code = lib().qmv_matvec_q4k_fx(y.data_ptr(), ctypes.byref(W), x.data_ptr(),
                                   ctypes.byref(act) if act is not None else None, r0, r1, _stream())
    _check(code, "qmv_matvec_q4k_fx")
    return y


class Prepared:
    """A libqmv call with its arguments marshalled once: calling it costs one
    ctypes call (on the stream current at preparation time unless another
    is given), so host overhead does not starve the GPU between launches and
    the call can be captured in a HIP graph.  The tensors must stay alive and
    keep their storage while the object is used."""

    def __init__(self, fname: str, args: list, keep: list, stream=None):
        self._f = getattr(lib(), fname)
        self._fname = fname
        self._args = args
        self._keep = keep
        self._stream = stream

    def __call__(self, stream=None):
        s = stream if stream is not None else (self._stream if self._stream is not None else _stream())
        code = self._f(*self._args, s)
        if code != 0:
            raise QmvError(code, self._fname)


def prepare_matvec_fx(qtype, wq, wd, x, y, r0=None, r1=None, xq_out=None, stream=None) -> Prepared:
    """Prepared qmv_matvec_q4_fx / qmv_matvec_q8_fx (same arguments as those)."""
    W = qtensor(wq, wd, qtype)
    _dev(x, torch.float32)
    _dev(y, torch.float32)
    r0 = 0 if r0 is None else r0
    r1 = W.rows if r1 is None else r1
    act = None
    if xq_out is not None:
        q, d = xq_out
        act = QAct(_dev(q, torch.int8).data_ptr(), _dev(d, torch.float32).data_ptr(), 0)
    fname = "qmv_matvec_q4_fx" if qtype == QMV_Q4_0 else "qmv_matvec_q8_fx"
    args = [y.data_ptr(), ctypes.byref(W), x.data_ptr(), ctypes.byref(act) if act is not None else None, r0, r1]
    return Prepared(fname, args, [W, act, wq, wd, x, y, xq_out], stream)


def prepare_matvec_fx_rmsnorm(qtype, wq, wd, x, w_norm, eps, y, r0=None, r1=None, xq_out=None,
                              stream=None) -> Prepared:
    """Prepared qmv_matvec_q4_fx_rmsnorm / qmv_matvec_q8_fx_rmsnorm."""
    W = qtensor(wq, wd, qtype)
    _dev(x, torch.float32)
    _dev(w_norm, torch.float32)
    _dev(y, torch.float32)
    r0 = 0 if r0 is None else r0
    r1 = W.rows if r1 is None else r1
    act = None
    if xq_out is not None:
        q, d = xq_out
        act = QAct(_dev(q, torch.int8).data_ptr(), _dev(d, torch.float32).data_ptr(), 0)
    fname = "qmv_matvec_q4_fx_rmsnorm" if qtype == QMV_Q4_0 else "qmv_matvec_q8_fx_rmsnorm"
    args = [y.data_ptr(), ctypes.byref(W), x.data_ptr(), w_norm.data_ptr(), ctypes.c_float(eps),
            ctypes.byref(act) if act is not None else None, r0, r1]
    return Prepared(fname, args, [W, act, wq, wd, x, w_norm, y, xq_out], stream)


def _swiglu_args(qtype, wq, wd, x, w_norm, eps, a, y, p0, p1, xq_out):
    W = qtensor(wq, wd, qtype)
    if W.rows % 2:
        raise ValueError("the stacked gate|up matrix needs an even row count")
    _dev(x, torch.float32)
    if w_norm is not None:
        _dev(w_norm, torch.float32)
    p0 = 0 if p0 is None else p0
    p1 = W.rows // 2 if p1 is None else p1
    y = _out(y, W.rows, wd)
    a = _out(a, W.rows // 2, wd)
    act = None
    if xq_out is not None:
        q, d = xq_out
        act = QAct(_dev(q, torch.int8).data_ptr(), _dev(d, torch.float32).data_ptr(), 0)
    fname = "qmv_matvec_q4_fx_swiglu" if qtype == QMV_Q4_0 else "qmv_matvec_q8_fx_swiglu"
    args = [a.data_ptr(), y.data_ptr(), ctypes.byref(W), x.data_ptr(),
            w_norm.data_ptr() if w_norm is not None else None, ctypes.c_float(eps),
            ctypes.byref(act) if act is not None else None, p0, p1]
    return fname, args, [W, act, wq, wd, x, w_norm, a, y, xq_out], a, y


def qmv_matvec_fx_swiglu(qtype, wq, wd, x, w_norm=None, eps=0.0, p0=None, p1=None, a=None, y=None, xq_out=None):
    """Stacked gate|up product with the gate applied: returns (a, y), y = W h
    (h = x, or rmsnorm(x) * w_norm) and a = silu(y[:F]) * y[F:] (include/qmv.h)."""
    fname, args, _keep, a, y = _swiglu_args(qtype, wq, wd, x, w_norm, eps, a, y, p0, p1, xq_out)
    _check(getattr(lib(), fname)(*args, _stream()), fname)
    return a, y


def prepare_matvec_fx_swiglu(qtype, wq, wd, x, a, y, w_norm=None, eps=0.0, p0=None, p1=None, xq_out=None,
                             stream=None) -> Prepared:
    """Prepared qmv_matvec_q4_fx_swiglu / qmv_matvec_q8_fx_swiglu."""
    fname, args, keep, _a, _y = _swiglu_args(qtype, wq, wd, x, w_norm, eps, a, y, p0, p1, xq_out)
    return Prepared(fname, args, keep, stream)


def prepare_matvec_fx_silu_mul(qtype, wq, wd, g, u, y, r0=None, r1=None, xq_out=None, stream=None) -> Prepared:
    """Prepared qmv_matvec_q4_fx_silu_mul / qmv_matvec_q8_fx_silu_mul."""
    W = qtensor(wq, wd, qtype)
    _dev(g, torch.float32)
    _dev(u, torch.float32)
    _dev(y, torch.float32)
    r0 = 0 if r0 is None else r0
    r1 = W.rows if r1 is None else r1
    act = None
    if xq_out is not None:
        q, d = xq_out
        act = QAct(_dev(q, torch.int8).data_ptr(), _dev(d, torch.float32).data_ptr(), 0)
    fname = "qmv_matvec_q4_fx_silu_mul" if qtype == QMV_Q4_0 else "qmv_matvec_q8_fx_silu_mul"
    args = [y.data_ptr(), ctypes.byref(W), g.data_ptr(), u.data_ptr(),
            ctypes.byref(act) if act is not None else None, r0, r1]
    return Prepared(fname, args, [W, act, wq, wd, g, u, y, xq_out], stream)


def prepare_gemm(qtype, wq, wd, xq, xd, Y, r0=None, r1=None, stream=None) -> Prepared:
    """Prepared qmv_gemm_q4 / qmv_gemm_q8."""
    W = qtensor(wq, wd, qtype)
    X = qtensor(xq, xd, QMV_Q8_0)
    _dev(Y, torch.float32)
    r0 = 0 if r0 is None else r0
    r1 = W.rows if r1 is None else r1
    fname = "qmv_gemm_q4" if qtype == QMV_Q4_0 else "qmv_gemm_q8"
    args = [Y.data_ptr(), ctypes.byref(W), ctypes.byref(X), r0, r1]
    return Prepared(fname, args, [W, X, wq, wd, xq, xd, Y], stream)


def prepare_gemm_packed(P: PackedWeights, xq, xd, Y, r0=None, r1=None, stream=None) -> Prepared:
    """Prepared qmv_gemm_q4_packed / qmv_gemm_q8_packed."""
    X = qtensor(xq, xd, QMV_Q8_0)
    _dev(Y, torch.float32)
    r0 = 0 if r0 is None else r0
    r1 = P.rows if r1 is None else r1
    fname = "qmv_gemm_q4_packed" if P.qtype == QMV_Q4_0 else "qmv_gemm_q8_packed"
    args = [Y.data_ptr(), ctypes.byref(P.desc), ctypes.byref(X), r0, r1]
    return Prepared(fname, args, [P, X, xq, xd, Y], stream)


def prepare_matvec_zp_fx(wq, wd, wzp, bits, x, y, r0=None, r1=None, stream=None) -> Prepared:
    """Prepared qmv_matvec_zp_fx."""
    W = zptensor(wq, wd, wzp, bits)
    _dev(x, torch.float32)
    _dev(y, torch.float32)
    r0 = 0 if r0 is None else r0
    r1 = W.rows if r1 is None else r1
    args = [y.data_ptr(), ctypes.byref(W), x.data_ptr(), None, r0, r1]
    return Prepared("qmv_matvec_zp_fx", args, [W, wq, wd, wzp, x, y], stream)


def prepare_matvec_q4k_fx(q, sc, mn, d, dmin, x, y, r0=None, r1=None, stream=None) -> Prepared:
    """Prepared qmv_matvec_q4k_fx."""
    W = q4ktensor(q, sc, mn, d, dmin)
    _dev(x, torch.float32)
    _dev(y, torch.float32)
    r0 = 0 if r0 is None else r0
    r1 = W.rows if r1 is None else r1
    args = [y.data_ptr(), ctypes.byref(W), x.data_ptr(), None, r0, r1]
    return Prepared("qmv_matvec_q4k_fx", args, [W, q, sc, mn, d, dmin, x, y], stream)


def qmv_rmsnorm(x: torch.Tensor, w: torch.Tensor, eps: float, o: torch.Tensor | None = None):
    """o = w * (x / rms(x)) as qmv_rmsnorm computes it (one launch)."""
    _dev(x, torch.float32)
    _dev(w, torch.float32)
    o = torch.empty_like(x) if o is None else _dev(o, torch.float32)
    _check(lib().qmv_rmsnorm(o.data_ptr(), x.data_ptr(), w.data_ptr(), x.numel(), float(eps), _stream()),
           "qmv_rmsnorm")
    return o


def qmv_silu_mul(g: torch.Tensor, u: torch.Tensor, o: torch.Tensor | None = None):
    """o = silu(g) * u as qmv_silu_mul computes it (one launch)."""
    _dev(g, torch.float32)
    _dev(u, torch.float32)
    o = torch.empty_like(g) if o is None else _dev(o, torch.float32)
    _check(lib().qmv_silu_mul(o.data_ptr(), g.data_ptr(), u.data_ptr(), g.numel(), _stream()), "qmv_silu_mul")
    return o


def prepare_rmsnorm(x, w, eps, o, stream=None) -> "Prepared":
    return Prepared("qmv_rmsnorm", [o.data_ptr(), x.data_ptr(), w.data_ptr(), x.numel(), ctypes.c_float(eps)],
                    [o, x, w], stream)


def prepare_silu_mul(g, u, o, stream=None) -> "Prepared":
    return Prepared("qmv_silu_mul", [o.data_ptr(), g.data_ptr(), u.data_ptr(), g.numel()], [o, g, u], stream)


# ---- measurement helpers (not on the product path)

def qmv_ceiling_stream_read(buf: torch.Tensor, sink: torch.Tensor, workgroups: int, depth: int = 4,
                            stream=None) -> None:
    """Stream-read every byte of the device tensor buf (uint32 sink of
    `workgroups` entries receives per-workgroup XORs of its 32-bit words)."""
    _dev(buf)
    _dev(sink, (torch.int32, torch.uint32))
    _check(lib().qmv_ceiling_stream_read(sink.data_ptr(), buf.data_ptr(), buf.numel() * buf.element_size(),
                                         workgroups, depth, _stream() if stream is None else stream),
           "qmv_ceiling_stream_read")


def qmv_ceiling_mfma_i8(sink: torch.Tensor, shape: int, iters: int, workgroups: int, a: int = 1, b: int = 1,
                        stream=None) -> None:
    """Chains of int8 matrix-core instructions (shape 0: 16x16x32, 1:
    16x16x64, 2: 32x32x32); sink (4 * workgroups int32) receives per-wavefront
    sums of the results."""
    _dev(sink, (torch.int32, torch.uint32))
    _check(lib().qmv_ceiling_mfma_i8(sink.data_ptr(), shape, iters, workgroups, a, b,
                                     _stream() if stream is None else stream), "qmv_ceiling_mfma_i8")
