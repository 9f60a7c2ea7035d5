"""The fused M = 1 matvec (float32 activation quantized inside the kernel)
on the GPU against the oracle, over the shapes that exercise both modes of
the fused kernel: small K (K / 32 <= 32, whole rows per wavefront: rows
interleaved over the wavefronts, partial last rounds) and split K (ragged
slices with K / 32 not a multiple of the wavefront count, partial last
passes, the largest slice K = 16384), the K on either side of each mode
(handled by the row-streaming kernel), row sub-ranges, and row counts that
hit the rows-per-workgroup cap.

Block sums are checked bit for bit through the fused entry point itself:
an activation of integers in [-127, 127] with a +-127 in every block
quantizes to exactly itself with scale 1, so with unit weight scales y is
the exact sum of the block sums (while |sum| < 2^24)."""
import numpy as np
import pytest
import torch

import pins
from block_quantized_decode_amd import qmv, synth
from gpu_util import announce, check_close, dev, host
from oracle import oracle as orc

pytestmark = pytest.mark.gpu


def _fx(qtype):
    return qmv.qmv_matvec_q4_fx if qtype == 4 else qmv.qmv_matvec_q8_fx


def _weights(rng, qtype, rows, k):
    w = synth.normal(rng, (rows, k), 0.02)
    return orc.quantize_q4(w) if qtype == 4 else orc.quantize_q8(w)


def _unit_activation(rng, k, lim):
    """Integers in [-lim, lim] with one +-127 per 32-element block: Q8_0
    turns each block into itself with d = 1 exactly."""
    x = rng.integers(-lim, lim + 1, size=k).astype(np.float32)
    pos = rng.integers(0, 32, size=k // 32) + 32 * np.arange(k // 32)
    x[pos] = np.where(rng.random(k // 32) < 0.5, -127.0, 127.0).astype(np.float32)
    return x


# (rows, K): K / 32 = 1, 16, 28 (Qwen2.5-0.5B hidden), 32 (whole rows per
# wavefront; 33 beyond: row-streaming kernel), 64 (smallest split), 65 and
# 66 (ragged slices, a last wavefront with 2 or 3 blocks), 128, 172, 344
# (Llama-7B W_down), 512 (the largest slice), 513 (beyond: row-streaming
# kernel); rows with partial last passes and fewer rows than compute units
SHAPES = [(1, 32), (33, 512), (600, 512), (7, 896), (4871, 896), (77, 1024), (19, 1056),
          (5, 2048), (257, 2080), (3, 2112), (1031, 4096), (64, 5504), (37, 11008), (130, 16384), (9, 16416)]


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("rows,k", SHAPES)
def test_fx_exact_block_sums(qtype, rows, k):
    announce(f"fx exact sums q{qtype} {rows}x{k}")
    rng = np.random.default_rng(900 + rows + k)
    wq, _ = synth.raw_q4(rng, rows, k) if qtype == 4 else synth.raw_q8(rng, rows, k)
    lim = 15 if qtype == 4 else 3    # keeps sum_b |sumi| below 2^24
    x = _unit_activation(rng, k, lim)
    xq, xd = orc.quantize_q8(x)
    assert np.all(xd == 1.0) and np.array_equal(xq.astype(np.float32), x)
    want = (pins.w_values(qtype, wq) * xq.astype(np.int64)[None, :]).sum(axis=1)
    assert np.all(np.abs(orc.block_sums(qtype, wq, xq)).astype(np.int64).sum(axis=1) < 2 ** 24)
    ones_w = np.ones((rows, k // 32), np.float32)
    y = host(_fx(qtype)(dev(wq), dev(ones_w), dev(x)))
    assert np.array_equal(y.astype(np.int64), want)


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("rows,k", SHAPES)
def test_fx_tolerance_and_quantized_copy(qtype, rows, k):
    announce(f"fx q{qtype} {rows}x{k}")
    rng = np.random.default_rng(1000 + rows + k)
    wq, wd = _weights(rng, qtype, rows, k)
    x = synth.normal(rng, (k,))
    x[rng.choice(k, size=max(1, k // 100), replace=False)] *= np.float32(20.0)
    xq, xd = orc.quantize_q8(x)
    yref = orc.matvec(qtype, wq, wd, xq, xd)
    qo = torch.full((k,), 99, dtype=torch.int8, device="cuda:0")
    do = torch.full((k // 32,), -1.0, dtype=torch.float32, device="cuda:0")
    y = host(_fx(qtype)(dev(wq), dev(wd), dev(x), xq_out=(qo, do)))
    assert np.array_equal(host(qo), xq), "fused quantization differs from the oracle's"
    assert np.array_equal(host(do).view(np.uint32), xd.view(np.uint32))
    check_close(qtype, y, yref, wq, wd, xq, xd, what=f"fx q{qtype} {rows}x{k}")
    y2 = host(_fx(qtype)(dev(wq), dev(wd), dev(x)))
    assert np.array_equal(y, y2), "same inputs, same bits"


@pytest.mark.parametrize("qtype", [4, 8])
def test_fx_row_ranges(qtype):
    announce(f"fx row ranges q{qtype}")
    rng = np.random.default_rng(1100)
    rows, k = 1333, 11008
    wq, wd = _weights(rng, qtype, rows, k)
    x = synth.normal(rng, (k,))
    xq, xd = orc.quantize_q8(x)
    yref = orc.matvec(qtype, wq, wd, xq, xd)
    for r0, r1 in ((0, rows), (1, 2), (3, 11), (17, 1300), (1329, 1333), (640, 640)):
        ydev = torch.full((rows,), -7.5, dtype=torch.float32, device="cuda:0")
        y = host(_fx(qtype)(dev(wq), dev(wd), dev(x), r0, r1, ydev))
        assert np.all(y[:r0] == -7.5) and np.all(y[r1:] == -7.5), f"rows outside [{r0},{r1}) written"
        if r1 > r0:
            check_close(qtype, y, yref, wq, wd, xq, xd, r0, r1, what=f"[{r0},{r1})")
    # whole-row mode (K / 32 = 28)
    rows, k = 3001, 896
    wq, wd = _weights(rng, qtype, rows, k)
    x = synth.normal(rng, (k,))
    xq, xd = orc.quantize_q8(x)
    yref = orc.matvec(qtype, wq, wd, xq, xd)
    for r0, r1 in ((0, rows), (2, 3), (5, 70), (999, 3001), (2990, 2999)):
        ydev = torch.full((rows,), -7.5, dtype=torch.float32, device="cuda:0")
        y = host(_fx(qtype)(dev(wq), dev(wd), dev(x), r0, r1, ydev))
        assert np.all(y[:r0] == -7.5) and np.all(y[r1:] == -7.5), f"rows outside [{r0},{r1}) written"
        if r1 > r0:
            check_close(qtype, y, yref, wq, wd, xq, xd, r0, r1, what=f"[{r0},{r1})")


def test_fx_rows_per_workgroup_cap():
    """More rows than 1024 per compute unit: the grid grows beyond one
    workgroup per compute unit; every row is still written once."""
    announce("fx many rows q4 270000x2048")
    rng = np.random.default_rng(1200)
    rows, k = 270000, 2048
    wq, wd = synth.raw_q4(rng, rows, k)
    x = synth.normal(rng, (k,))
    xq, xd = orc.quantize_q8(x)
    yref = orc.matvec(4, wq, wd, xq, xd)
    y = host(qmv.qmv_matvec_q4_fx(dev(wq), dev(wd), dev(x)))
    check_close(4, y, yref, wq, wd, xq, xd, what="270000 rows")


def test_fx_kernel_choice():
    """K / 32 <= 32 and K / 32 in [64, 512] run the fused kernel (whole-row
    and split-K modes), other K the row kernel."""
    announce("fx kernel choice")
    rng = np.random.default_rng(1300)
    for k, want in ((32, "fx_"), (1024, "fx_"), (1056, "rows_"), (2016, "rows_"), (2048, "fx_"), (16384, "fx_"),
                    (16416, "rows_")):
        wq, wd = _weights(rng, 4, 8, k)
        qmv.qmv_matvec_q4_fx(dev(wq), dev(wd), dev(synth.normal(rng, (k,))))
        torch.cuda.synchronize()
        assert qmv.last_kernel().startswith(want), (k, qmv.last_kernel())
