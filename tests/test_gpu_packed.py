"""The pack-once weight layout and the matrix-core product on it, on the GPU.

qmv_pack_weights is a permutation of the stored bytes and scales.  Its
output is compared byte for byte with the layout written out here in numpy
from the header's description: units of 16 rows x 4 blocks, lane
l = 16 g + i holding elements 8 g .. 8 g + 7 of row i, Q4_0 nibbles
re-paired as (8 g + j, 8 g + 4 + j), scales [row][block], padding value 0
with scale 0.

The packed product adds the same terms in the same order as the row-major
matrix-core product, so for M > 8 it must give the same bits as qmv_gemm_*
on the unpacked weights; it is also checked against the oracle (tolerance
|y - y_ref| <= 1e-5 * sum_b |sumi * dw * dx| + 1e-6, and exactly with unit
scales).  For M <= 8 (the row-major call takes another path there) it is
checked against the oracle only."""
import numpy as np
import pytest
import torch

import pins
from block_quantized_decode_amd import qmv, synth
from gpu_util import announce, check_close, check_gemm_all, dev, host
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

SENTINEL = np.float32(-12345.5)


def _weights(rng, qtype, rows, k):
    return synth.raw_q4(rng, rows, k) if qtype == 4 else synth.raw_q8(rng, rows, k)


def _act(rng, m, k):
    return orc.quantize_q8(synth.normal(rng, (m, k)))


def _gemm(qtype):
    return qmv.qmv_gemm_q4 if qtype == 4 else qmv.qmv_gemm_q8


def _gemm_packed(qtype):
    return qmv.qmv_gemm_q4_packed if qtype == 4 else qmv.qmv_gemm_q8_packed


def pack_layout(qtype, wq, wd):
    """The packed bytes and scales as the header describes them."""
    rows, nb = wd.shape
    nt, nq = (rows + 15) // 16, (nb + 3) // 4
    if qtype == 4:
        b = wq.view(np.uint8).reshape(rows, nb, 16)
        elem = np.concatenate([b & 0x0F, b >> 4], axis=2)         # stored nibble of element e
        full = np.full((nt * 16, nq * 4, 32), 8, np.uint8)         # value 0 = nibble 8
        full[:rows, :nb] = elem
        t = full.reshape(nt, 16, nq, 4, 4, 8)                      # [T, i, Q, u, g, e]
        t = (t[..., 0:4] | (t[..., 4:8] << 4)).astype(np.uint8)   # byte j: (8 g + j, 8 g + 4 + j)
    else:
        full = np.zeros((nt * 16, nq * 4, 32), np.uint8)
        full[:rows, :nb] = wq.view(np.uint8).reshape(rows, nb, 32)
        t = full.reshape(nt, 16, nq, 2, 2, 4, 8)                   # [T, i, Q, u / 2, u % 2, g, e]
        q = t.transpose(0, 2, 3, 5, 1, 4, 6).reshape(-1)           # [T, Q, u / 2, g, i, u % 2, bytes]
    if qtype == 4:
        q = t.transpose(0, 2, 4, 1, 3, 5).reshape(-1)              # [T, Q, g, i, u, bytes]
    d = np.zeros((nt * 16, nq * 4), np.float32)
    d[:rows, :nb] = wd
    d = d.reshape(nt, 16, nq, 4).transpose(0, 2, 1, 3).reshape(-1)  # [T, Q, row, block]
    return q, d


def _pack(qtype, wq, wd):
    return qmv.qmv_pack_weights(dev(wq), dev(wd), qtype)


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("rows,k", [(1, 32), (16, 128), (17, 160), (45, 4128), (300, 512), (33, 11008)])
def test_pack_layout(qtype, rows, k):
    announce(f"pack layout q{qtype} {rows}x{k}")
    rng = np.random.default_rng(4000 + rows + k + qtype)
    wq, wd = _weights(rng, qtype, rows, k)
    P = _pack(qtype, wq, wd)
    assert (P.rows, P.cols, P.qtype) == (rows, k, qtype)
    assert qmv.last_kernel() == f"pack_q{qtype}"
    qref, dref = pack_layout(qtype, wq, wd)
    qb, db = qmv.qmv_pack_bytes(qtype, rows, k)
    assert (qref.size, dref.size * 4) == (qb, db)
    assert np.array_equal(host(P.q)[:qb], qref)
    assert np.array_equal(host(P.d)[:db // 4].view(np.uint32), dref.view(np.uint32))


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("m", [9, 16, 17, 33, 64, 65, 100])
def test_packed_equals_row_major(qtype, m):
    """Same bits as the row-major matrix-core product; within tolerance of
    the oracle.  K = 4128 (129 blocks: a last quad of one block)."""
    announce(f"packed gemm q{qtype} m={m}")
    rng = np.random.default_rng(4100 + m + qtype)
    rows, k = 300, 4128
    wq, wd = _weights(rng, qtype, rows, k)
    xq, xd = _act(rng, m, k)
    P = _pack(qtype, wq, wd)
    Yp = host(_gemm_packed(qtype)(P, dev(xq), dev(xd)))
    assert qmv.last_kernel().startswith("mmp_"), qmv.last_kernel()
    Y = host(_gemm(qtype)(dev(wq), dev(wd), dev(xq), dev(xd)))
    assert qmv.last_kernel().startswith("mm_"), qmv.last_kernel()
    assert np.array_equal(Yp.view(np.uint32), Y.view(np.uint32))
    Yref = orc.gemm(qtype, wq, wd, xq, xd)
    for i in range(m):
        check_close(qtype, Yp[i], Yref[i], wq, wd, xq[i], xd[i], what=f"packed q{qtype} m={m} row {i}")


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("m", [1, 4, 8])
def test_packed_few_rows(qtype, m):
    announce(f"packed gemm few rows q{qtype} m={m}")
    rng = np.random.default_rng(4200 + m + qtype)
    rows, k = 77, 2080
    wq, wd = _weights(rng, qtype, rows, k)
    xq, xd = _act(rng, m, k)
    Yp = host(_gemm_packed(qtype)(_pack(qtype, wq, wd), dev(xq), dev(xd)))
    Yref = orc.gemm(qtype, wq, wd, xq, xd)
    for i in range(m):
        check_close(qtype, Yp[i], Yref[i], wq, wd, xq[i], xd[i], what=f"packed q{qtype} m={m} row {i}")


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("rows,k", [(16, 32), (17, 64), (33, 96), (5, 256)])
def test_packed_small_shapes(qtype, rows, k):
    """One block, part of a quad, fewer rows than a tile."""
    announce(f"packed gemm q{qtype} {rows}x{k}")
    rng = np.random.default_rng(4300 + rows + k + qtype)
    m = 20
    wq, wd = _weights(rng, qtype, rows, k)
    xq, xd = _act(rng, m, k)
    Yp = host(_gemm_packed(qtype)(_pack(qtype, wq, wd), dev(xq), dev(xd)))
    Y = host(_gemm(qtype)(dev(wq), dev(wd), dev(xq), dev(xd)))
    assert np.array_equal(Yp.view(np.uint32), Y.view(np.uint32))
    Yref = orc.gemm(qtype, wq, wd, xq, xd)
    for i in range(m):
        check_close(qtype, Yp[i], Yref[i], wq, wd, xq[i], xd[i], what=f"packed q{qtype} row {i}")


@pytest.mark.parametrize("qtype", [4, 8])
def test_packed_row_ranges(qtype):
    """r0 a multiple of 16, r1 anywhere: only rows [r0, r1) are written, and
    they equal the row-major product's."""
    rng = np.random.default_rng(4400 + qtype)
    rows, k, m = 1333, 1024, 24
    wq, wd = _weights(rng, qtype, rows, k)
    xq, xd = _act(rng, m, k)
    P = _pack(qtype, wq, wd)
    Y = host(_gemm(qtype)(dev(wq), dev(wd), dev(xq), dev(xd)))
    for r0, r1 in ((0, rows), (16, 17), (32, 1300), (1328, 1333), (640, 640), (0, 5)):
        announce(f"packed gemm q{qtype} rows [{r0},{r1})")
        Yd = torch.full((m, rows), float(SENTINEL), dtype=torch.float32, device="cuda:0")
        Yp = host(_gemm_packed(qtype)(P, dev(xq), dev(xd), r0, r1, Yd))
        assert np.all(Yp[:, :r0] == SENTINEL) and np.all(Yp[:, r1:] == SENTINEL), (r0, r1)
        assert np.array_equal(Yp[:, r0:r1].view(np.uint32), Y[:, r0:r1].view(np.uint32)), (r0, r1)
    with pytest.raises(qmv.QmvError, match="QMV_E_SHAPE"):
        _gemm_packed(qtype)(P, dev(xq), dev(xd), 8, 40)


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("m", [16, 64])
def test_packed_exact_unit_scales(qtype, m):
    """dw = dx = 1 and |x| <= 16: Y is the exact integer sum of the block sums."""
    announce(f"packed gemm unit scales q{qtype} m={m}")
    rng = np.random.default_rng(4500 + m + qtype)
    rows, k = 96, 4096
    wq, _ = _weights(rng, qtype, rows, k)
    xq, _ = _act(rng, m, k)
    xs = (xq // 8).astype(np.int8)
    w64 = pins.w_values(qtype, wq)
    assert np.abs(w64).sum(axis=1).max() * 16 < 2 ** 24
    P = _pack(qtype, wq, np.ones((rows, k // 32), np.float32))
    Y = host(_gemm_packed(qtype)(P, dev(xs), dev(np.ones((m, k // 32), np.float32))))
    assert np.array_equal(Y.astype(np.int64), (w64 @ xs.astype(np.int64).T).T)


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("rows,k,m", [(11008, 4096, 16), (11008, 4096, 64), (4096, 11008, 64), (16387, 128, 33)])
def test_packed_full_size(qtype, rows, k, m):
    """The bench's batched shapes (Llama-7B W_up and W_down at 16 and 64
    activation rows) and a case with more workgroups than compute units:
    the same bits as the row-major product, and every output within
    tolerance of the oracle."""
    announce(f"packed gemm full size q{qtype} {rows}x{k} m={m}")
    rng = np.random.default_rng(4600 + rows + k + m + qtype)
    wq, wd = _weights(rng, qtype, rows, k)
    xq, xd = _act(rng, m, k)
    Yp = host(_gemm_packed(qtype)(_pack(qtype, wq, wd), dev(xq), dev(xd)))
    Y = host(_gemm(qtype)(dev(wq), dev(wd), dev(xq), dev(xd)))
    assert np.array_equal(Yp.view(np.uint32), Y.view(np.uint32))
    worst = check_gemm_all(qtype, Yp, wq, wd, xq, xd, what=f"packed q{qtype} {rows}x{k} m={m}")
    print(f"  all {m} x {rows} outputs, max |err| / tol = {worst:.4f}")
