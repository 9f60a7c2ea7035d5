"""The matrix-core product (M > 8 activation rows) on the GPU against the
oracle.

Cases span the tile edges of the kernel: activation rows around multiples
of 16 and 32 and past the 64 rows of one pass, weight rows that leave a
ragged last tile, K from one block up to the 131072 limit with block counts
that do not divide evenly among the wavefronts, row ranges that start and
end inside a tile, and the extreme quant values.

Block sums are checked bit for bit with unit scales (Y = sum of the block
sums, exact in fp32 while every partial sum stays below 2^24) and with a
one-hot activation scale (Y = one block's sum); outputs with real scales
are checked against the oracle within
|y - y_ref| <= 1e-5 * sum_b |sumi * dw * dx| + 1e-6."""
import numpy as np
import pytest
import torch

import pins
from block_quantized_decode_amd import qmv, synth
from gpu_util import announce, check_close, check_gemm_all, dev, host
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

SENTINEL = np.float32(-12345.5)


def _f(qtype):
    return qmv.qmv_gemm_q4 if qtype == 4 else qmv.qmv_gemm_q8


def _weights(rng, qtype, rows, k):
    return synth.raw_q4(rng, rows, k) if qtype == 4 else synth.raw_q8(rng, rows, k)


def _act(rng, m, k):
    return orc.quantize_q8(synth.normal(rng, (m, k)))


def _sums(qtype, wq, xq):
    """Exact int32 block sums [m, rows, nb] from the oracle."""
    return np.stack([orc.block_sums(qtype, wq, xq[i]) for i in range(xq.shape[0])])


def _check_all(qtype, Y, wq, wd, xq, xd, r0, r1, what):
    Yref = orc.gemm(qtype, wq, wd, xq, xd, r0, r1)
    worst = 0.0
    for i in range(xq.shape[0]):
        worst = max(worst, check_close(qtype, Y[i], Yref[i], wq, wd, xq[i], xd[i], r0, r1, what=f"{what} row {i}"))
    return worst


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("m", [9, 15, 16, 17, 31, 32, 33, 47, 48, 63, 64, 65, 100, 129])
def test_gemm_mfma_rows(qtype, m):
    announce(f"gemm mfma q{qtype} m={m} rows=77 k=2080")
    rng = np.random.default_rng(900 + m + 1000 * qtype)
    rows, k = 77, 2080  # 65 blocks: uneven split over the wavefronts; last row tile ragged
    wq, wd = _weights(rng, qtype, rows, k)
    xq, xd = _act(rng, m, k)
    Y = host(_f(qtype)(dev(wq), dev(wd), dev(xq), dev(xd)))
    _check_all(qtype, Y, wq, wd, xq, xd, 0, rows, f"q{qtype} m={m}")


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("rows,k", [(1, 32), (16, 32), (17, 64), (33, 96), (5, 256), (300, 512), (64, 4128),
                                    (48, 11008), (20, 16384), (3, 131072)])
def test_gemm_mfma_shapes(qtype, rows, k):
    m = 40
    announce(f"gemm mfma q{qtype} m={m} rows={rows} k={k}")
    rng = np.random.default_rng(rows * 7 + k + qtype)
    wq, wd = _weights(rng, qtype, rows, k)
    xq, xd = _act(rng, m, k)
    Y = host(_f(qtype)(dev(wq), dev(wd), dev(xq), dev(xd)))
    _check_all(qtype, Y, wq, wd, xq, xd, 0, rows, f"q{qtype} {rows}x{k}")


@pytest.mark.parametrize("qtype", [4, 8])
def test_gemm_mfma_row_ranges(qtype):
    rng = np.random.default_rng(31 + qtype)
    rows, k, m = 150, 1024, 37
    wq, wd = _weights(rng, qtype, rows, k)
    xq, xd = _act(rng, m, k)
    for r0, r1 in [(0, 150), (5, 70), (16, 48), (149, 150), (33, 33), (1, 149)]:
        announce(f"gemm mfma q{qtype} m={m} r0={r0} r1={r1}")
        Y0 = np.full((m, rows), SENTINEL, np.float32)
        Y = host(_f(qtype)(dev(wq), dev(wd), dev(xq), dev(xd), r0, r1, dev(Y0)))
        outside = np.ones(rows, bool)
        outside[r0:r1] = False
        assert np.all(Y[:, outside] == SENTINEL), f"rows outside [{r0}, {r1}) were written"
        if r1 > r0:
            _check_all(qtype, Y, wq, wd, xq, xd, r0, r1, f"q{qtype} [{r0},{r1})")


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("m", [16, 64, 70])
def test_gemm_mfma_exact_unit_scales(qtype, m):
    announce(f"gemm mfma unit scales q{qtype} m={m}")
    rng = np.random.default_rng(55 + m + qtype)
    rows, k = 96, 4096
    wq, _ = _weights(rng, qtype, rows, k)
    xq, _ = _act(rng, m, k)
    xs = (xq // 8).astype(np.int8)  # |x| <= 16 keeps every partial sum below 2^24
    ones_w = np.ones((rows, k // 32), np.float32)
    ones_x = np.ones((m, k // 32), np.float32)
    w64 = pins.w_values(qtype, wq)
    assert np.abs(w64).sum(axis=1).max() * 16 < 2 ** 24
    Y = host(_f(qtype)(dev(wq), dev(ones_w), dev(xs), dev(ones_x)))
    want = (w64 @ xs.astype(np.int64).T).T
    assert np.array_equal(Y.astype(np.int64), want)


@pytest.mark.parametrize("qtype", [4, 8])
def test_gemm_mfma_exact_one_hot(qtype):
    """dx one-hot at block b (dw = 1): Y[m, r] is exactly sumi(m, r, b)."""
    rng = np.random.default_rng(77 + qtype)
    rows, k, m = 40, 2048, 33
    nb = k // 32
    wq, _ = _weights(rng, qtype, rows, k)
    xq, _ = _act(rng, m, k)
    ones_w = np.ones((rows, nb), np.float32)
    sums = _sums(qtype, wq, xq)
    for b in [0, 1, nb // 2, nb - 1]:
        announce(f"gemm mfma one-hot q{qtype} block {b}")
        dx = np.zeros((m, nb), np.float32)
        dx[:, b] = 1.0
        Y = host(_f(qtype)(dev(wq), dev(ones_w), dev(xq), dev(dx)))
        assert np.array_equal(Y.astype(np.int64), sums[:, :, b].astype(np.int64)), f"block {b}"


@pytest.mark.parametrize("qtype", [4, 8])
def test_gemm_mfma_extreme_quants(qtype):
    """Largest |sumi|: weights at their extreme codes against x = +-127."""
    announce(f"gemm mfma extreme quants q{qtype}")
    rows, k, m = 32, 1024, 20
    nb = k // 32
    rng = np.random.default_rng(5)
    if qtype == 4:
        # nibble 0 -> -8 and 15 -> 7, in both halves of the byte
        codes = rng.choice(np.array([0x00, 0xFF, 0x0F, 0xF0], np.uint8), size=(rows, k // 2))
        wq = codes
    else:
        wq = rng.choice(np.array([-127, 127], np.int8), size=(rows, k))
    xq = rng.choice(np.array([-127, 127], np.int8), size=(m, k))
    wd = np.ones((rows, nb), np.float32)
    sums = _sums(qtype, wq, xq)
    b = 3
    dx = np.zeros((m, nb), np.float32)
    dx[:, b] = 1.0
    Y = host(_f(qtype)(dev(wq), dev(wd), dev(xq), dev(dx)))
    assert np.array_equal(Y.astype(np.int64), sums[:, :, b].astype(np.int64))
    # real scales at the extremes, every block
    wd = np.abs(synth.normal(rng, (rows, nb), 0.01)).astype(np.float32) + np.float32(1e-3)
    xd = np.abs(synth.normal(rng, (m, nb), 0.05)).astype(np.float32) + np.float32(1e-3)
    Y = host(_f(qtype)(dev(wq), dev(wd), dev(xq), dev(xd)))
    _check_all(qtype, Y, wq, wd, xq, xd, 0, rows, f"extreme q{qtype}")


@pytest.mark.parametrize("qtype", [4, 8])
def test_gemm_mfma_deterministic(qtype):
    announce(f"gemm mfma repeat q{qtype}")
    rng = np.random.default_rng(9)
    rows, k, m = 200, 4096, 64
    wq, wd = _weights(rng, qtype, rows, k)
    xq, xd = _act(rng, m, k)
    args = (dev(wq), dev(wd), dev(xq), dev(xd))
    Y1 = host(_f(qtype)(*args))
    Y2 = host(_f(qtype)(*args))
    assert np.array_equal(Y1.view(np.uint32), Y2.view(np.uint32))


@pytest.mark.parametrize("qtype", [4, 8])
def test_gemm_k_limit(qtype):
    """Sizes beyond the limits are refused (status, nothing launched):
    M * K > 131072 for M <= 8, K > 131072 for M > 8."""
    rng = np.random.default_rng(3)
    for m, k in ((4, 32800), (8, 16416), (9, 131104), (64, 131104)):
        wq, wd = _weights(rng, qtype, 2, k)
        xq, xd = _act(rng, m, k)
        with pytest.raises(qmv.QmvError, match="QMV_E_SHAPE"):
            _f(qtype)(dev(wq), dev(wd), dev(xq), dev(xd))


ROW_TILE_CASES = [(8187, 256, 20, "mt2_rt2_"), (11000, 512, 64, "mt4_rt3_"), (16387, 128, 33, "mt4_rt4_"),
                  (10000, 8192, 40, "mt4_rt3_w8_d2_t"), (13000, 8192, 64, "mt4_rt4_w8_d2_t")]


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("rows,k,m,form", ROW_TILE_CASES, ids=[f"{r}x{k}-m{m}" for r, k, m, _ in ROW_TILE_CASES])
def test_gemm_mfma_row_tiles(qtype, rows, k, m, form):
    """Weight-row counts that give a workgroup 2, 3 and 4 tiles of 16 rows
    (more tiles than compute units), with a ragged last tile; 16387 rows
    also need more workgroups than compute units.  The last two take the
    stage loop with a guarded tail at 3 and 4 tiles with four activation
    tiles, the forms whose registers spill to scratch (the 4-tile one for
    both formats, the 3-tile one for Q8_0)."""
    announce(f"gemm mfma q{qtype} m={m} rows={rows} k={k}")
    rng = np.random.default_rng(rows + k + m + qtype)
    wq, wd = _weights(rng, qtype, rows, k)
    xq, xd = _act(rng, m, k)
    Y = host(_f(qtype)(dev(wq), dev(wd), dev(xq), dev(xd)))
    kname = qmv.last_kernel()
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert kname.startswith(f"mm_q{qtype}_{form}"), kname
    _check_all(qtype, Y, wq, wd, xq, xd, 0, rows, f"q{qtype} {rows}x{k} m={m}")


# One activation tile (9 .. 16 rows): stages per wavefront 4 (K = 4096), 8
# (8192), 11 (11008), 16 (16384); 1 .. 4 weight tiles per workgroup; a ragged
# last tile and a partial last stage (K = 4128).
ONE_TILE_CASES = [(4096, 4096, 16, 1), (4090, 8192, 9, 1), (4096, 11008, 16, 1), (3001, 16384, 12, 1),
                  (8000, 4096, 16, 2), (11008, 4096, 16, 3), (11000, 8192, 13, 3), (16000, 4128, 16, 4),
                  (16001, 8192, 10, 4)]


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("rows,k,m,rt", ONE_TILE_CASES, ids=[f"{r}x{k}-m{m}-rt{t}" for r, k, m, t in ONE_TILE_CASES])
def test_gemm_one_activation_tile(qtype, rows, k, m, rt):
    """Every output against the oracle, and the launch shape (weight tiles
    per workgroup) on a 256-compute-unit MI355X."""
    announce(f"gemm one tile q{qtype} {rows}x{k} m={m}")
    rng = np.random.default_rng(9000 + rows + k + m + qtype)
    wq, wd = _weights(rng, qtype, rows, k)
    xq, xd = _act(rng, m, k)
    Y = host(_f(qtype)(dev(wq), dev(wd), dev(xq), dev(xd)))
    kname = qmv.last_kernel()
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert kname.startswith(f"mm_q{qtype}_mt1_rt{rt}_"), kname
    worst = check_gemm_all(qtype, Y, wq, wd, xq, xd, what=f"q{qtype} {rows}x{k} m={m}")
    print(f"  {kname}: max |err| / tol = {worst:.4f}")
    Y2 = host(_f(qtype)(dev(wq), dev(wd), dev(xq), dev(xd)))
    assert np.array_equal(Y.view(np.uint32), Y2.view(np.uint32)), "same inputs, same bits"
