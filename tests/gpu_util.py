"""Helpers shared by the GPU parity tests (host <-> device copies and the
tolerance check).  No arithmetic of the method lives here."""
import concurrent.futures as cf
import os
import sys

import numpy as np
import torch

from oracle import oracle as orc

DEV = "cuda:0"


def announce(msg: str):
    """Name the case about to run on the GPU (flushed first, so that a fault
    in it is attributable from the log)."""
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_close(qtype, y_gpu, y_ref, wq, wd, xq, xd, r0=None, r1=None, what=""):
    """|y - y_ref| <= 1e-5 * sum_b |sumi * dw * dx| + 1e-6 for every row."""
    tol = orc.tolerance(qtype, wq, wd, xq, xd, r0, r1)
    r0 = 0 if r0 is None else r0
    r1 = len(y_ref) if r1 is None else r1
    err = np.abs(y_gpu[r0:r1].astype(np.float64) - y_ref[r0:r1].astype(np.float64))
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, (f"{what}: {bad.size} rows out of tolerance, first row {r0 + bad[0]}: "
                           f"gpu {y_gpu[r0 + bad[0]]!r} ref {y_ref[r0 + bad[0]]!r} tol {tol[bad[0]]:.3g}")
    return float((err / tol).max()) if err.size else 0.0


# ---- every output of a full-size case against the oracle, rows split over
# host threads (the oracle's own [r0, r1) contract; ctypes releases the GIL
# inside each oracle call, so the chunks run in parallel)

def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunks(r0: int, r1: int, n: int):
    n = max(1, min(n * 4, r1 - r0))
    b = np.linspace(r0, r1, n + 1).astype(int)
    return [(int(b[i]), int(b[i + 1])) for i in range(n) if b[i + 1] > b[i]]


def _par(fn, r0, r1):
    with cf.ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(lambda ab: fn(*ab), _chunks(r0, r1, _threads())))


def _verdict(parts, what):
    worst = max((w for w, _ in parts), default=0.0)
    bad = [b for _, b in parts if b is not None]
    assert not bad, f"{what}: {sum(n for n, _ in bad)} outputs out of tolerance, first {bad[0][1]}"
    return worst


def check_gemm_all(qtype, Y, wq, wd, xq, xd, r0=0, r1=None, what=""):
    """Every Y[m, r], m < M, r in [r0, r1), within 1e-5 * sum_b |sumi * dw *
    dx| + 1e-6 of the oracle's gemm."""
    r1 = wd.shape[0] if r1 is None else r1
    m = xq.shape[0]

    def part(a, b):
        Yref = orc.gemm(qtype, wq, wd, xq, xd, a, b)
        worst, bad = 0.0, None
        for i in range(m):
            tol = orc.tolerance(qtype, wq, wd, xq[i], xd[i], a, b)
            err = np.abs(Y[i, a:b].astype(np.float64) - Yref[i, a:b].astype(np.float64))
            worst = max(worst, float((err / tol).max()))
            nb_ = int((err > tol).sum())
            if nb_ and bad is None:
                r = a + int(np.argmax(err > tol))
                bad = (nb_, f"m={i} r={r} gpu {Y[i, r]!r} ref {Yref[i, r]!r}")
        return worst, bad

    return _verdict(_par(part, r0, r1), what)


def check_zp_all(bits, y, wq, wd, wzp, xq, xd, r0=0, r1=None, what=""):
    """Every y[r], r in [r0, r1), of the 128-block zero-point product."""
    r1 = wd.shape[0] if r1 is None else r1

    def part(a, b):
        yref = orc.matvec_zp(bits, wq, wd, wzp, xq, xd, a, b)
        tol = orc.tolerance_zp(bits, wq, wd, wzp, xq, xd, a, b)
        err = np.abs(y[a:b].astype(np.float64) - yref[a:b].astype(np.float64))
        nb_ = int((err > tol).sum())
        bad = (nb_, f"r={a + int(np.argmax(err > tol))}") if nb_ else None
        return float((err / tol).max()), bad

    return _verdict(_par(part, r0, r1), what)


def check_q4k_all(y, w, xq, xd, r0=0, r1=None, what=""):
    """Every y[r], r in [r0, r1), of the K-quant super-block product."""
    r1 = w[0].shape[0] if r1 is None else r1

    def part(a, b):
        yref = orc.matvec_q4k(*w, xq, xd, a, b)
        tol = orc.tolerance_q4k(*w, xq, xd, a, b)
        err = np.abs(y[a:b].astype(np.float64) - yref[a:b].astype(np.float64))
        nb_ = int((err > tol).sum())
        bad = (nb_, f"r={a + int(np.argmax(err > tol))}") if nb_ else None
        return float((err / tol).max()), bad

    return _verdict(_par(part, r0, r1), what)
