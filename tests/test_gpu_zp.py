"""The 128-element-block zero-point format (qmv_matvec_zp_fx,
qmv_quantize_q8_b128) on the GPU against the oracle (oracle.quantize_q8_b128,
oracle.matvec_zp).

The activation is quantized inside the kernel: its codes and block scales
(returned through xq) must equal the oracle's bit for bit, and y must be
within |y - y_ref| <= 1e-5 * sum_b |sumi * dw * dx| + 1e-6 of the oracle's
product on those codes.  With unit scales (integer activations whose block
maxima are 127, so dx = 1 and q = x; dw = 1) y is the exact integer sum.
Cases span the kernel's configurations: rows of 4 .. 8 chunks (16-lane
groups), up to 32 chunks (32-lane groups), 1 .. 8 chunks per lane and
several windows per row; zero points given or the default; row ranges that
start and end anywhere; the Qwen2.5-0.5B and Llama-7B shapes at full size."""
import numpy as np
import pytest
import torch

import pins
from block_quantized_decode_amd import qmv, synth
from gpu_util import announce, dev, host
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

SENTINEL = np.float32(-12345.5)


def _run(bits, wq, wd, wzp, x, r0=None, r1=None, y=None):
    k = x.size
    qo = torch.full((k,), 99, dtype=torch.int8, device="cuda:0")
    do = torch.full((k // 128,), -1.0, dtype=torch.float32, device="cuda:0")
    y = qmv.qmv_matvec_zp_fx(dev(wq), dev(wd), None if wzp is None else dev(wzp), bits, dev(x), r0, r1, y,
                             xq_out=(qo, do))
    return host(y), host(qo), host(do)


def _check(bits, y, wq, wd, wzp, xq, xd, r0, r1, what):
    yref = orc.matvec_zp(bits, wq, wd, wzp, xq, xd, r0, r1)
    tol = orc.tolerance_zp(bits, wq, wd, wzp, xq, xd, r0, r1)
    err = np.abs(y[r0:r1].astype(np.float64) - yref[r0:r1].astype(np.float64))
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, f"{what}: {bad.size} rows out of tolerance, first {r0 + bad[0]}"


def _x(rng, k):
    x = synth.normal(rng, (k,))
    x[rng.choice(k, size=max(1, k // 100), replace=False)] *= np.float32(20.0)
    return x


# K: 128 (one block: 16-lane groups for both widths), 256, 512 and 1024
# (32-lane groups for one width), 896 (Qwen hidden), 2048, 4096, 4864 (Qwen
# FFN), 8192 (8 chunks per lane, 8 bits), 11008 (two windows), 65536 (the
# largest K)
SHAPES = [(5, 128), (33, 256), (77, 512), (301, 896), (19, 1024), (130, 2048), (257, 4096), (64, 4864),
          (21, 8192), (40, 11008), (9, 65536)]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("rows,k", SHAPES)
@pytest.mark.parametrize("with_zp", [True, False])
def test_zp_matches_oracle(bits, rows, k, with_zp):
    announce(f"zp{bits} {rows}x{k} zp={with_zp}")
    rng = np.random.default_rng(5000 + rows + k + bits + with_zp)
    wq, wd, wzp = synth.raw_zp(rng, bits, rows, k, with_zp)
    x = _x(rng, k)
    xq, xd = orc.quantize_q8_b128(x)
    y, qo, do = _run(bits, wq, wd, wzp, x)
    assert qmv.last_kernel().startswith(f"zp{bits}_"), qmv.last_kernel()
    assert np.array_equal(qo, xq), "activation codes"
    assert np.array_equal(do.view(np.uint32), xd.view(np.uint32)), "activation scales"
    _check(bits, y, wq, wd, wzp, xq, xd, 0, rows, f"zp{bits} {rows}x{k}")
    y2, _, _ = _run(bits, wq, wd, wzp, x)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "same inputs, same bits"


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("k", [128, 896, 4864])
def test_zp_exact_unit_scales(bits, k):
    """dw = 1, integer activations with a 127 in every block (dx = 1, q = x):
    y is the exact sum of the block sums."""
    announce(f"zp{bits} unit scales K={k}")
    rng = np.random.default_rng(5100 + k + bits)
    rows = 70
    wq, _, wzp = synth.raw_zp(rng, bits, rows, k)
    x = rng.integers(-20, 21, size=k).astype(np.float32)
    x[::128] = 127.0
    wd = np.ones((rows, k // 128), np.float32)
    y, qo, do = _run(bits, wq, wd, wzp, x)
    assert np.array_equal(qo, x.astype(np.int8)) and np.all(do == 1.0)
    want = (pins.zp_values(bits, wq, wzp) * x.astype(np.int64)).sum(axis=1)
    assert np.abs(want).max() < 2 ** 24
    assert np.array_equal(y.astype(np.int64), want)


@pytest.mark.parametrize("bits", [4, 8])
def test_zp_row_ranges(bits):
    rng = np.random.default_rng(5200 + bits)
    rows, k = 1333, 896
    wq, wd, wzp = synth.raw_zp(rng, bits, rows, k)
    x = _x(rng, k)
    xq, xd = orc.quantize_q8_b128(x)
    for r0, r1 in ((0, rows), (1, 2), (17, 1300), (1329, 1333), (640, 640)):
        announce(f"zp{bits} rows [{r0},{r1})")
        yd = torch.full((rows,), float(SENTINEL), dtype=torch.float32, device="cuda:0")
        y, qo, _ = _run(bits, wq, wd, wzp, x, r0, r1, yd)
        assert np.all(y[:r0] == SENTINEL) and np.all(y[r1:] == SENTINEL), (r0, r1)
        assert np.array_equal(qo, xq)  # the activation is returned even for an empty range
        if r1 > r0:
            _check(bits, y, wq, wd, wzp, xq, xd, r0, r1, f"[{r0},{r1})")


@pytest.mark.parametrize("k", [128, 4096, 65536 - 128])
def test_quantize_b128(k):
    """The standalone 128-block quantization equals the oracle's, bit for bit
    (zero blocks and single-element blocks included)."""
    announce(f"quantize b128 K={k}")
    rng = np.random.default_rng(5300 + k)
    x = synth.normal(rng, (3, k))
    x[1, :128] = 0.0
    x[2, 128 * (k // 256):128 * (k // 256 + 1)] = 0.0
    x[2, 128 * (k // 256) + 5] = -3.0
    q, d = qmv.qmv_quantize_q8_b128(dev(x))
    assert qmv.last_kernel() == "quant_q8_b128"
    qr, dr = orc.quantize_q8_b128(x)
    assert np.array_equal(host(q), qr)
    assert np.array_equal(host(d).view(np.uint32), dr.view(np.uint32))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("rows,k", [(4864, 896), (896, 4864), (151936, 896), (11008, 4096), (4096, 11008)])
def test_zp_full_size(bits, rows, k):
    """The bench's shapes (Qwen2.5-0.5B W_gate / W_up, W_down and lm_head;
    Llama-7B W_up and W_down) at full size: codes bit-exact, sampled row
    ranges within tolerance of the oracle."""
    announce(f"zp{bits} full size {rows}x{k}")
    rng = np.random.default_rng(5400 + rows + k + bits)
    wq, wd, wzp = synth.raw_zp(rng, bits, rows, k, with_zp=(rows != 151936))
    x = _x(rng, k)
    xq, xd = orc.quantize_q8_b128(x)
    y, qo, do = _run(bits, wq, wd, wzp, x)
    assert np.array_equal(qo, xq) and np.array_equal(do.view(np.uint32), xd.view(np.uint32))
    for r0 in (0, rows // 2 - 5, rows - 11):
        _check(bits, y, wq, wd, wzp, xq, xd, r0, r0 + 11, f"full {rows}x{k} [{r0},{r0 + 11})")
