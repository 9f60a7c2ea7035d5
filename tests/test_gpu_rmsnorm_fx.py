"""The fused rmsnorm + Q8_0 quantization + product (qmv_matvec_q4_fx_rmsnorm /
_q8_) on the GPU against the oracle (oracle.rmsnorm, then quantize_q8, then
matvec).  Every operation of the normalization is correctly rounded in
binary32 and its sum of squares has a fixed pairwise order, so the quantized
normalized activation must equal the oracle's bit for bit -- codes and block
scales -- and y must be within the product's tolerance of the oracle's on
those codes.

Besides random activations (with 1% outliers x20), the cases include
activations built so that the order of the sum of squares decides its
rounding: each block holds one element of magnitude s and 31 of magnitude
s * 2^-12, with s a different power of two per block.  Pairwise summation
gives a block sum s^2 (1 + 15 * 2^-23) where a left-to-right sum gives s^2,
and block sums of very different size lose different bits depending on the
order they are combined in; a kernel with another order changes inv by
several ulps, which changes the block maxima of h and hence the scales."""
import numpy as np
import pytest
import torch

from block_quantized_decode_amd import qmv, synth
from gpu_util import announce, check_close, dev, host
from oracle import oracle as orc

pytestmark = pytest.mark.gpu


def _fxn(qtype):
    return qmv.qmv_matvec_q4_fx_rmsnorm if qtype == 4 else qmv.qmv_matvec_q8_fx_rmsnorm


def _weights(rng, qtype, rows, k):
    w = synth.normal(rng, (rows, k), 0.02)
    return orc.quantize_q4(w) if qtype == 4 else orc.quantize_q8(w)


def _order_sensitive(rng, k):
    nb = k // 32
    s = np.float32(2.0) ** rng.integers(-6, 7, size=nb).astype(np.float32)
    sign = np.where(rng.random(k) < 0.5, -1.0, 1.0).astype(np.float32)
    x = np.repeat(s * np.float32(2.0 ** -12), 32).astype(np.float32)
    x[::32] = s
    return x * sign


def _run(qtype, wq, wd, x, wn, eps, r0=None, r1=None, y=None):
    k = x.size
    qo = torch.full((k,), 99, dtype=torch.int8, device="cuda:0")
    do = torch.full((k // 32,), -1.0, dtype=torch.float32, device="cuda:0")
    y = _fxn(qtype)(dev(wq), dev(wd), dev(x), dev(wn), eps, r0, r1, y, xq_out=(qo, do))
    return host(y), host(qo), host(do)


# (rows, K): K / 32 = 1, 16, 28 and 32 (whole rows per wavefront), 64 (the
# smallest split), 65 (ragged slices, block count not a power of two), 128,
# 160 (Llama-13B hidden), 344, 512 (the largest)
SHAPES = [(3, 32), (33, 512), (301, 896), (77, 1024), (5, 2048), (257, 2080), (1031, 4096), (19, 5120),
          (37, 11008), (45, 9216), (130, 16384)]


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("rows,k", SHAPES)
@pytest.mark.parametrize("kind", ["normal", "order"])
def test_rmsnorm_fx_matches_oracle(qtype, rows, k, kind):
    announce(f"rmsnorm fx q{qtype} {rows}x{k} {kind}")
    rng = np.random.default_rng(2000 + rows + k + (7 if kind == "order" else 0))
    wq, wd = _weights(rng, qtype, rows, k)
    if kind == "normal":
        x = synth.normal(rng, (k,))
        x[rng.choice(k, size=max(1, k // 100), replace=False)] *= np.float32(20.0)
        eps = 1e-5
    else:
        x = _order_sensitive(rng, k)
        eps = 1e-6
    wn = (1.0 + 0.1 * rng.standard_normal(k)).astype(np.float32)
    h = orc.rmsnorm(x, wn, eps)
    xq, xd = orc.quantize_q8(h)
    yref = orc.matvec(qtype, wq, wd, xq, xd)
    y, qo, do = _run(qtype, wq, wd, x, wn, eps)
    assert qmv.last_kernel().startswith("fxn_"), qmv.last_kernel()
    assert np.array_equal(do.view(np.uint32), xd.view(np.uint32)), "block scales of the normalized activation"
    assert np.array_equal(qo, xq), "codes of the normalized activation"
    check_close(qtype, y, yref, wq, wd, xq, xd, what=f"rmsnorm fx q{qtype} {rows}x{k} {kind}")
    y2, _, _ = _run(qtype, wq, wd, x, wn, eps)
    assert np.array_equal(y, y2), "same inputs, same bits"


@pytest.mark.parametrize("qtype", [4, 8])
def test_rmsnorm_fx_row_ranges_and_scaling(qtype):
    """Row sub-ranges write only their rows; scaling x by a power of two with
    eps = 0 leaves the normalized activation, hence y, unchanged bit for bit."""
    announce(f"rmsnorm fx row ranges q{qtype}")
    rng = np.random.default_rng(2100)
    rows, k = 1333, 4096
    wq, wd = _weights(rng, qtype, rows, k)
    x = synth.normal(rng, (k,))
    wn = (1.0 + 0.1 * rng.standard_normal(k)).astype(np.float32)
    h = orc.rmsnorm(x, wn, 1e-5)
    xq, xd = orc.quantize_q8(h)
    yref = orc.matvec(qtype, wq, wd, xq, xd)
    for r0, r1 in ((0, rows), (1, 2), (17, 1300), (1329, 1333), (640, 640)):
        ydev = torch.full((rows,), -7.5, dtype=torch.float32, device="cuda:0")
        y, _, _ = _run(qtype, wq, wd, x, wn, 1e-5, r0, r1, ydev)
        assert np.all(y[:r0] == -7.5) and np.all(y[r1:] == -7.5), f"rows outside [{r0},{r1}) written"
        if r1 > r0:
            check_close(qtype, y, yref, wq, wd, xq, xd, r0, r1, what=f"[{r0},{r1})")
    y0, q0, d0 = _run(qtype, wq, wd, x, wn, 0.0)
    for e in (-4, 6):
        y1, q1, d1 = _run(qtype, wq, wd, x * np.float32(2.0 ** e), wn, 0.0)
        assert np.array_equal(q1, q0) and np.array_equal(d1, d0) and np.array_equal(y1, y0), e


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("rows,k", [(2560, 2048), (11264, 2048), (11008, 4096)])
def test_rmsnorm_fx_full_size_launches(qtype, rows, k):
    """The launches the bench's fusion section times, at full size: rmsnorm
    ahead of the concatenated TinyLlama-1.1B projections (W_q|W_k|W_v 2560 x
    2048, W_gate|W_up 11264 x 2048) and of the Llama-7B W_up."""
    announce(f"rmsnorm fx full size q{qtype} {rows}x{k}")
    rng = np.random.default_rng(3000 + rows + k)
    wq, wd = _weights(rng, qtype, rows, k)
    x = synth.normal(rng, (k,))
    wn = (1.0 + 0.1 * rng.standard_normal(k)).astype(np.float32)
    xq, xd = orc.quantize_q8(orc.rmsnorm(x, wn, 1e-5))
    yref = orc.matvec(qtype, wq, wd, xq, xd)
    y, qo, do = _run(qtype, wq, wd, x, wn, 1e-5)
    assert np.array_equal(qo, xq) and np.array_equal(do.view(np.uint32), xd.view(np.uint32))
    check_close(qtype, y, yref, wq, wd, xq, xd, what=f"full size {rows}x{k}")


def test_fused_forms_graph_replay():
    """Prepared calls of the rmsnorm and FFN-gate forms and of the 4-row
    matrix-core product captured in one HIP graph, chained as in a decode
    layer (the gate form reads the halves of the gate|up output the rmsnorm
    form wrote): every replay, with eager work and synchronisations in
    between, gives the eager result bit for bit."""
    announce("fused forms graph replay")
    rng = np.random.default_rng(3200)
    k, hidden = 2048, 5632
    stream = torch.cuda.Stream()
    s = stream.cuda_stream
    wgu_q, wgu_d = _weights(rng, 4, 2 * hidden, k)
    wdn_q, wdn_d = _weights(rng, 4, k, hidden)
    x = dev(synth.normal(rng, (k,)))
    wn = dev((1.0 + 0.1 * rng.standard_normal(k)).astype(np.float32))
    y_gu = torch.zeros(2 * hidden, dtype=torch.float32, device="cuda:0")
    y_dn = torch.zeros(k, dtype=torch.float32, device="cuda:0")
    X4 = synth.normal(rng, (4, k))
    x4q, x4d = orc.quantize_q8(X4)
    Y4 = torch.zeros((4, 2 * hidden), dtype=torch.float32, device="cuda:0")
    gq, gd = dev(wgu_q), dev(wgu_d)
    calls = [qmv.prepare_matvec_fx_rmsnorm(4, gq, gd, x, wn, 1e-5, y_gu, stream=s),
             qmv.prepare_matvec_fx_silu_mul(4, dev(wdn_q), dev(wdn_d), y_gu[:hidden], y_gu[hidden:], y_dn, stream=s),
             qmv.prepare_gemm(4, gq, gd, dev(x4q), dev(x4d), Y4, stream=s)]
    with torch.cuda.stream(stream):
        for c in calls:
            c()
    torch.cuda.synchronize()
    eager = [host(t).copy() for t in (y_gu, y_dn, Y4)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in calls:
            c()
    for rep in range(3):
        for t in (y_gu, y_dn, Y4):
            t.fill_(-1.0)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip((y_gu, y_dn, Y4), eager):
            assert np.array_equal(host(t), e), f"replay {rep} differs from the eager result"
    # the eager chain itself against the oracle
    h = orc.rmsnorm(host(x), host(wn), 1e-5)
    hq, hd = orc.quantize_q8(h)
    check_close(4, eager[0], orc.matvec(4, wgu_q, wgu_d, hq, hd), wgu_q, wgu_d, hq, hd, what="rmsnorm + gate|up")
    Y4ref = orc.gemm(4, wgu_q, wgu_d, x4q, x4d)
    for i in range(4):
        check_close(4, eager[2][i], Y4ref[i], wgu_q, wgu_d, x4q[i], x4d[i], what=f"4-row product row {i}")
