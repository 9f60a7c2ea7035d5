"""Matvec / small-batch products on the GPU against the oracle.

Block sums are checked bit for bit through the public entry points with
unit scales (y = sum of block sums, exact in fp32 while |sum| < 2^24) and
with a one-hot activation scale (y = one block's sum, at any K); fp32
outputs with real scales are checked against the oracle within
|y - y_ref| <= 1e-5 * sum_b |sumi * dw * dx| + 1e-6."""
import numpy as np
import pytest
import torch

import pins
from block_quantized_decode_amd import qmv, synth
from gpu_util import announce, check_close, dev, host
from oracle import oracle as orc

pytestmark = pytest.mark.gpu


def _weights(rng, qtype, rows, k, raw=True):
    if raw:
        return synth.raw_q4(rng, rows, k) if qtype == 4 else synth.raw_q8(rng, rows, k)
    w = synth.normal(rng, (rows, k), 0.02)
    return orc.quantize_q4(w) if qtype == 4 else orc.quantize_q8(w)


def _mv(qtype, wq, wd, xq, xd, r0=None, r1=None, y=None):
    f = qmv.qmv_matvec_q4 if qtype == 4 else qmv.qmv_matvec_q8
    return f(dev(wq), dev(wd), dev(xq), dev(xd), r0, r1, y)


SHAPES = [(1, 32), (3, 32), (4, 64), (7, 96), (64, 4096), (129, 2048), (37, 11008), (10, 896), (5, 32 * 65)]


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("rows,k", SHAPES)
def test_block_sums_exact_unit_scales(qtype, rows, k):
    announce(f"unit-scale matvec q{qtype} {rows}x{k}")
    rng = np.random.default_rng(200 + rows + k)
    wq, _ = _weights(rng, qtype, rows, k)
    xq = synth.raw_q8(rng, 1, k)[0].reshape(-1)
    ones_w = np.ones((rows, k // 32), np.float32)
    ones_x = np.ones(k // 32, np.float32)
    if k > 1024:   # keep |sum| < 2^24 so the fp32 result is exact: shrink the activation
        xq = (xq // 8).astype(np.int8)
    want = (pins.w_values(qtype, wq) * xq.astype(np.int64)[None, :]).sum(axis=1)
    # every partial sum the kernel can form is bounded by sum_b |sumi|: keep it below 2^24
    assert np.all(np.abs(orc.block_sums(qtype, wq, xq)).astype(np.int64).sum(axis=1) < 2 ** 24)
    y = host(_mv(qtype, wq, ones_w, xq, ones_x))
    assert np.array_equal(y.astype(np.int64), want)


@pytest.mark.parametrize("qtype", [4, 8])
def test_block_sums_exact_one_hot(qtype):
    announce(f"one-hot matvec q{qtype}")
    rng = np.random.default_rng(210)
    rows, k = 67, 11008
    wq, _ = _weights(rng, qtype, rows, k)
    xq = synth.raw_q8(rng, 1, k)[0].reshape(-1)
    ones_w = np.ones((rows, k // 32), np.float32)
    sums = orc.block_sums(qtype, wq, xq)
    for b in (0, 1, 63, 64, 200, k // 32 - 1):
        oh = np.zeros(k // 32, np.float32)
        oh[b] = 1.0
        y = host(_mv(qtype, wq, ones_w, xq, oh))
        assert np.array_equal(y.astype(np.int64), sums[:, b].astype(np.int64)), f"block {b}"


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("rows,k", SHAPES)
def test_matvec_tolerance(qtype, rows, k):
    announce(f"matvec q{qtype} {rows}x{k}")
    rng = np.random.default_rng(300 + rows + k)
    wq, wd = _weights(rng, qtype, rows, k)
    x = synth.normal(rng, (k,))
    xq, xd = orc.quantize_q8(x)
    yref = orc.matvec(qtype, wq, wd, xq, xd)
    y = host(_mv(qtype, wq, wd, xq, xd))
    check_close(qtype, y, yref, wq, wd, xq, xd, what=f"q{qtype} {rows}x{k}")


@pytest.mark.parametrize("qtype", [4, 8])
def test_row_ranges(qtype):
    announce(f"row ranges q{qtype}")
    rng = np.random.default_rng(400)
    rows, k = 103, 4096
    wq, wd = _weights(rng, qtype, rows, k)
    xq, xd = orc.quantize_q8(synth.normal(rng, (k,)))
    yref = orc.matvec(qtype, wq, wd, xq, xd)
    for r0, r1 in ((0, 103), (1, 2), (5, 9), (17, 103), (100, 103), (0, 4), (50, 50)):
        ydev = torch.full((rows,), -7.5, dtype=torch.float32, device="cuda:0")
        y = host(_mv(qtype, wq, wd, xq, xd, r0, r1, ydev))
        assert np.all(y[:r0] == -7.5) and np.all(y[r1:] == -7.5), f"rows outside [{r0},{r1}) written"
        if r1 > r0:
            check_close(qtype, y, yref, wq, wd, xq, xd, r0, r1, what=f"[{r0},{r1})")


@pytest.mark.parametrize("qtype", [4, 8])
def test_extreme_quants(qtype):
    """Q4_0: every byte value (nibble 0 = -8 included); Q8_0: -128, -127, 127."""
    announce(f"extreme quants q{qtype}")
    rng = np.random.default_rng(500)
    rows, k = 64, 2048
    if qtype == 4:
        wq = np.tile(np.arange(256, dtype=np.uint8), rows * (k // 2) // 256).reshape(rows, k // 2)
    else:
        wq = rng.choice(np.array([-128, -127, 127, 0, 1, -1], np.int8), size=(rows, k))
    wd = synth.raw_scales(rng, (rows, k // 32))
    xq = rng.choice(np.array([-127, 127, -1, 0], np.int8), size=k)
    xd = synth.raw_scales(rng, (k // 32,))
    ones_w = np.ones_like(wd)
    sums = orc.block_sums(qtype, wq, xq)
    oh = np.zeros(k // 32, np.float32)
    oh[3] = 1.0
    y = host(_mv(qtype, wq, ones_w, xq, oh))
    assert np.array_equal(y.astype(np.int64), sums[:, 3].astype(np.int64))
    yref = orc.matvec(qtype, wq, wd, xq, xd)
    y = host(_mv(qtype, wq, wd, xq, xd))
    check_close(qtype, y, yref, wq, wd, xq, xd, what="extremes")


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("rows,k", [(1, 32), (9, 64), (256, 512), (300, 4096), (41, 11008)])
def test_matvec_fx(qtype, rows, k):
    announce(f"matvec_fx q{qtype} {rows}x{k}")
    rng = np.random.default_rng(600 + rows)
    wq, wd = _weights(rng, qtype, rows, k, raw=False)
    x = synth.normal(rng, (k,))
    x[::50] *= np.float32(20.0)
    xq, xd = orc.quantize_q8(x)
    yref = orc.matvec(qtype, wq, wd, xq, xd)
    qo = torch.zeros(k, dtype=torch.int8, device="cuda:0")
    do = torch.zeros(k // 32, dtype=torch.float32, device="cuda:0")
    f = qmv.qmv_matvec_q4_fx if qtype == 4 else qmv.qmv_matvec_q8_fx
    y = host(f(dev(wq), dev(wd), dev(x), xq_out=(qo, do)))
    assert np.array_equal(host(qo), xq), "fused quantization differs from the oracle's"
    assert np.array_equal(host(do).view(np.uint32), xd.view(np.uint32))
    check_close(qtype, y, yref, wq, wd, xq, xd, what="fx")
    y2 = host(f(dev(wq), dev(wd), dev(x)))
    assert np.array_equal(y, y2), "same inputs, same bits (no atomics, fixed order)"


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 11, 16])
def test_gemm(qtype, m):
    announce(f"gemm q{qtype} m={m}")
    rng = np.random.default_rng(700 + m)
    rows, k = 77, 2048
    wq, wd = _weights(rng, qtype, rows, k)
    X = synth.normal(rng, (m, k))
    xq, xd = orc.quantize_q8(X)
    Yref = orc.gemm(qtype, wq, wd, xq, xd)
    f = qmv.qmv_gemm_q4 if qtype == 4 else qmv.qmv_gemm_q8
    Y = host(f(dev(wq), dev(wd), dev(xq), dev(xd)))
    for i in range(m):
        check_close(qtype, Y[i], Yref[i], wq, wd, xq[i], xd[i], what=f"gemm row {i}")
    # unit scales: exact block sums for every activation row
    ones_w = np.ones_like(wd)
    ones_x = np.ones_like(xd)
    xs = (xq // 8).astype(np.int8)
    Y = host(f(dev(wq), dev(ones_w), dev(xs), dev(ones_x)))
    want = pins.w_values(qtype, wq) @ xs.astype(np.int64).T
    assert np.array_equal(Y.astype(np.int64), want.T)


def test_prepared_calls_and_graph_replay():
    """Prepared calls captured in a HIP graph: every replay, with eager work
    and synchronisations in between, gives the eager result bit for bit
    (the kernels are deterministic: fixed summation order, no atomics)."""
    announce("graph replay")
    rng = np.random.default_rng(800)
    dev_ = "cuda:0"
    cases = []
    for qtype, rows, k in ((4, 300, 4096), (4, 77, 11008), (8, 129, 896)):
        wq, wd = _weights(rng, qtype, rows, k, raw=False)
        x = synth.normal(rng, (k,))
        cases.append((qtype, dev(wq), dev(wd), dev(x), torch.zeros(rows, dtype=torch.float32, device=dev_),
                      orc.matvec(qtype, wq, wd, *orc.quantize_q8(x)), (wq, wd, x)))
    stream = torch.cuda.Stream()
    calls = [qmv.prepare_matvec_fx(qt, q, d, x, y, stream=stream.cuda_stream) for qt, q, d, x, y, _, _ in cases]
    with torch.cuda.stream(stream):
        for c in calls:
            c()
    torch.cuda.synchronize()
    eager = [host(y).copy() for *_, y, _, _ in [(c[0], c[1], c[2], c[3], c[4], c[5], c[6]) for c in cases]]
    for (qt, _, _, _, _, yref, (wq, wd, x)), ye in zip(cases, eager):
        xq, xd = orc.quantize_q8(x)
        check_close(qt, ye, yref, wq, wd, xq, xd, what="prepared eager")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for c in calls:
            c()
    for rep in range(3):
        for *_, y, _, _ in cases:
            y.fill_(-1.0)                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (*_, y, _, _), ye in zip(cases, eager):
            assert np.array_equal(host(y), ye), f"replay {rep} differs from the eager result"
