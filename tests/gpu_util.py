"""Helpers shared by the GPU parity tests (host <-> device copies and the
tolerance check).  No arithmetic of the method lives here."""
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
