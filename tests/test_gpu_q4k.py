"""K-quant super-blocks with the integer-folded sub-block scales
(qmv_matvec_q4k_fx, qmv_quantize_q8_b256) on the GPU against the oracle
(oracle.quantize_q8_b256, oracle.matvec_q4k, oracle.superblock_sums_q4k).

The activation is quantized inside the kernel: its codes and block scales
must equal the oracle's bit for bit, and y must be within
|y - y_ref| <= 1e-5 * sum_k |dx| (|S1 d| + |S2 dmin|) + 1e-6 of the oracle's
product on those codes.  With d = dmin = 1 and an activation whose block
maxima are 127 (dx = 1, q = x), y is the exact sum of S1 - S2 (kept below
2^24).  Cases span the kernel's configurations (rows of 8, 16 and 32
sub-blocks on 16- and 32-lane groups, 1 .. 8 chunks per lane and several
windows on 64-lane groups, wavefront teams for few rows), ragged row
ranges, and the TinyLlama-1.1B and Llama-7B shapes at full size."""
import numpy as np
import pytest
import torch

import pins
from block_quantized_decode_amd import qmv, synth
from gpu_util import announce, check_q4k_all, dev, host
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

SENTINEL = np.float32(-12345.5)


def _run(w, x, r0=None, r1=None, y=None):
    k = x.size
    qo = torch.full((k,), 99, dtype=torch.int8, device="cuda:0")
    do = torch.full((k // 256,), -1.0, dtype=torch.float32, device="cuda:0")
    y = qmv.qmv_matvec_q4k_fx(*[dev(a) for a in w], dev(x), r0, r1, y, xq_out=(qo, do))
    return host(y), host(qo), host(do)


def _check(y, w, xq, xd, r0, r1, what):
    yref = orc.matvec_q4k(*w, xq, xd, r0, r1)
    tol = orc.tolerance_q4k(*w, xq, xd, r0, r1)
    err = np.abs(y[r0:r1].astype(np.float64) - yref[r0:r1].astype(np.float64))
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, f"{what}: {bad.size} rows out of tolerance, first {r0 + bad[0]}"


def _x(rng, k):
    x = synth.normal(rng, (k,))
    x[rng.choice(k, size=max(1, k // 100), replace=False)] *= np.float32(20.0)
    return x


# K = 256 and 512 (16-lane groups), 1024 (32-lane), 2048 (TinyLlama hidden),
# 4096, 5632 (TinyLlama FFN), 11008 (Llama-7B FFN), 16384 and 65536 (the
# largest K)
SHAPES = [(5, 256), (33, 512), (77, 1024), (301, 2048), (130, 4096), (64, 5632), (40, 11008), (19, 16384),
          (9, 65536)]


@pytest.mark.parametrize("rows,k", SHAPES)
def test_q4k_matches_oracle(rows, k):
    announce(f"q4k {rows}x{k}")
    rng = np.random.default_rng(6000 + rows + k)
    w = synth.raw_q4k(rng, rows, k)
    x = _x(rng, k)
    xq, xd = orc.quantize_q8_b256(x)
    y, qo, do = _run(w, x)
    assert qmv.last_kernel().startswith(("q4k_", "gs_q4k_")), qmv.last_kernel()
    assert np.array_equal(qo, xq), "activation codes"
    assert np.array_equal(do.view(np.uint32), xd.view(np.uint32)), "activation scales"
    _check(y, w, xq, xd, 0, rows, f"q4k {rows}x{k}")
    y2, _, _ = _run(w, x)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "same inputs, same bits"


@pytest.mark.parametrize("k", [256, 2048, 5632])
def test_q4k_exact_unit_scales(k):
    """d = dmin = 1 and integer activations with a 127 in every block
    (dx = 1, q = x): y is the exact sum of S1 - S2 over the super-blocks."""
    announce(f"q4k unit scales K={k}")
    rng = np.random.default_rng(6100 + k)
    rows = 70
    q, sc, mn, _, _ = synth.raw_q4k(rng, rows, k)
    sc = (sc % 4).astype(np.uint8)  # keeps every S1 below 2^24
    one = np.ones((rows, k // 256), np.float32)
    x = rng.integers(-20, 21, size=k).astype(np.float32)
    x[::256] = 127.0
    w = (q, sc, mn, one, one)
    y, qo, do = _run(w, x)
    assert np.array_equal(qo, x.astype(np.int8)) and np.all(do == 1.0)
    s1, s2 = orc.superblock_sums_q4k(q, sc, mn, x.astype(np.int8))
    assert np.abs(s1).max() < 2 ** 24
    want = (s1.astype(np.int64) - s2).sum(axis=1)
    b1, b2 = pins._q4k_brute_sums(q, sc, mn, x.astype(np.int8))
    assert np.array_equal(want, (b1 - b2).sum(axis=1))
    assert np.array_equal(y.astype(np.int64), want)


def test_q4k_extreme_fold():
    """The page's bound: nibbles 15, scales 63, activation 127 everywhere give
    S1 = 8*63*32*127*15 per super-block; with d = 2^-10, dmin = 0 and dx = 1
    every y is that times the number of super-blocks times 2^-10, exactly."""
    announce("q4k extreme fold")
    rows, k = 40, 2048
    nk = k // 256
    q = np.full((rows, k // 2), 0xFF, np.uint8)
    sc = np.full((rows, k // 32), 63, np.uint8)
    mn = np.full((rows, k // 32), 63, np.uint8)
    d = np.full((rows, nk), 2.0 ** -10, np.float32)
    dmin = np.zeros((rows, nk), np.float32)
    x = np.full(k, 127.0, np.float32)
    y, qo, do = _run((q, sc, mn, d, dmin), x)
    bound = pins.golden("q4k_fold_bound.json")["fold_bound"]
    assert np.all(do == 1.0) and np.all(qo == 127)
    assert np.all(y == np.float32(np.float32(bound) * np.float32(2.0 ** -10) * nk))


def test_q4k_row_ranges():
    rng = np.random.default_rng(6200)
    rows, k = 1333, 2048
    w = synth.raw_q4k(rng, rows, k)
    x = _x(rng, k)
    xq, xd = orc.quantize_q8_b256(x)
    for r0, r1 in ((0, rows), (1, 2), (17, 1300), (1329, 1333), (640, 640)):
        announce(f"q4k rows [{r0},{r1})")
        yd = torch.full((rows,), float(SENTINEL), dtype=torch.float32, device="cuda:0")
        y, qo, _ = _run(w, x, r0, r1, yd)
        assert np.all(y[:r0] == SENTINEL) and np.all(y[r1:] == SENTINEL), (r0, r1)
        assert np.array_equal(qo, xq)
        if r1 > r0:
            _check(y, w, xq, xd, r0, r1, f"[{r0},{r1})")


@pytest.mark.parametrize("k", [256, 4096, 65536 - 256])
def test_quantize_b256(k):
    announce(f"quantize b256 K={k}")
    rng = np.random.default_rng(6300 + k)
    x = synth.normal(rng, (3, k))
    x[1, :256] = 0.0
    q, d = qmv.qmv_quantize_q8_b256(dev(x))
    assert qmv.last_kernel() == "quant_q8_b256"
    qr, dr = orc.quantize_q8_b256(x)
    assert np.array_equal(host(q), qr)
    assert np.array_equal(host(d).view(np.uint32), dr.view(np.uint32))


@pytest.mark.parametrize("rows,k", [(2048, 2048), (256, 2048), (5632, 2048), (2048, 5632), (11008, 4096),
                                    (4096, 11008)])
def test_q4k_full_size(rows, k):
    """TinyLlama-1.1B (W_q/W_o, W_k/W_v, W_gate/W_up, W_down) and Llama-7B
    (W_up, W_down) at full size: codes bit-exact, every row within tolerance
    of the oracle."""
    announce(f"q4k full size {rows}x{k}")
    rng = np.random.default_rng(6400 + rows + k)
    w = synth.raw_q4k(rng, rows, k)
    x = _x(rng, k)
    xq, xd = orc.quantize_q8_b256(x)
    y, qo, do = _run(w, x)
    assert np.array_equal(qo, xq) and np.array_equal(do.view(np.uint32), xd.view(np.uint32))
    worst = check_q4k_all(y, w, xq, xd, what=f"full {rows}x{k}")
    print(f"  {qmv.last_kernel()}: all {rows} rows, max |err| / tol = {worst:.4f}")


def test_q4k_graph_replay():
    """Prepared K-quant matvecs in one HIP graph: every replay, with eager
    work in between, gives the eager result bit for bit."""
    announce("q4k graph replay")
    rng = np.random.default_rng(6500)
    stream = torch.cuda.Stream()
    s = stream.cuda_stream
    wa = [dev(a) for a in synth.raw_q4k(rng, 5632, 2048)]
    wb = [dev(a) for a in synth.raw_q4k(rng, 2048, 5632)]
    xa, xb = dev(_x(rng, 2048)), dev(_x(rng, 5632))
    ya = torch.zeros(5632, dtype=torch.float32, device="cuda:0")
    yb = torch.zeros(2048, dtype=torch.float32, device="cuda:0")
    calls = [qmv.prepare_matvec_q4k_fx(*wa, xa, ya, stream=s), qmv.prepare_matvec_q4k_fx(*wb, xb, yb, stream=s)]
    with torch.cuda.stream(stream):
        for c in calls:
            c()
    torch.cuda.synchronize()
    eager = [host(ya).copy(), host(yb).copy()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in calls:
            c()
    for rep in range(3):
        ya.fill_(-1.0)
        yb.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(ya), eager[0]) and np.array_equal(host(yb), eager[1]), rep
    xq, xd = orc.quantize_q8_b256(host(xa))
    _check(eager[0], [host(a) for a in wa], xq, xd, 0, 5632, "graph q4k")
