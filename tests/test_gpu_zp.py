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
from gpu_util import announce, check_zp_all, dev, host
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
    assert qmv.last_kernel().startswith((f"zp{bits}_", "gs_zp4_" if bits == 4 else "zp8_")), qmv.last_kernel()
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


# Full-size shapes and the launch each one takes on a 256-compute-unit
# MI355X (names: lanes per row l, chunks per lane j, ring depth d, team of p
# wavefronts, w wavefronts per workgroup), so that a change of dispatch shows:
#   - the bench's shapes: Qwen2.5-0.5B W_gate / W_up, W_down and lm_head,
#     Llama-7B W_up and W_down;
#   - rows in [2048, 4096) at K = 11008, where teams take more wavefronts
#     until a ring turn takes one scale load (p = 4);
#   - one wavefront per row with two windows per row, the accumulator
#     carried across items (8-bit K = 16384 and 4-bit K = 32768 at 8192 rows);
#   - the split-K kernel for 4-bit codes (gs_: n units per lane and pass,
#     ring depth d, w wavefronts) on the Llama-7B shapes (8 wavefronts) and
#     the Qwen2.5-0.5B W_down (4 wavefronts: fewer rows).
FULL = [
    (4, 4864, 896, "zp4_l32_j1_d3_p1_w8"), (8, 4864, 896, "zp8_l64_j1_d3_p1_w8"),
    (4, 896, 4864, "gs_zp4_n3_d4_w4"), (8, 896, 4864, "zp8_l64_j2_d3_p4_w16"),
    (4, 151936, 896, "zp4_l32_j1_d3_p1_w8"), (8, 151936, 896, "zp8_l64_j1_d3_p1_w8"),
    (4, 11008, 4096, "gs_zp4_n1_d4_w8"), (8, 11008, 4096, "zp8_l64_j4_d2_p1_w16"),
    (4, 4096, 11008, "gs_zp4_n2_d4_w11"), (8, 4096, 11008, "zp8_l64_j3_d2_p4_w16"),
    (4, 2048, 11008, "zp4_l64_j2_d2_p4_w16"), (8, 2048, 11008, "zp8_l64_j3_d2_p4_w16"),
    (4, 3001, 11008, "zp4_l64_j2_d2_p4_w16"), (8, 3001, 11008, "zp8_l64_j3_d2_p4_w16"),
    (8, 8192, 16384, "zp8_l64_j8_d2_p1_w16"), (4, 8192, 32768, "zp4_l64_j8_d2_p1_w16"),
]


@pytest.mark.parametrize("bits,rows,k,kernel", FULL, ids=[f"zp{b}-{r}x{k}" for b, r, k, _ in FULL])
def test_zp_full_size(bits, rows, k, kernel):
    """Full size: codes bit-exact, every row within tolerance of the oracle,
    and the launch shape named above."""
    announce(f"zp{bits} full size {rows}x{k}")
    rng = np.random.default_rng(5400 + rows + k + bits)
    wq, wd, wzp = synth.raw_zp(rng, bits, rows, k, with_zp=(rows != 151936))
    x = _x(rng, k)
    xq, xd = orc.quantize_q8_b128(x)
    y, qo, do = _run(bits, wq, wd, wzp, x)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert qmv.last_kernel() == kernel, qmv.last_kernel()
    assert np.array_equal(qo, xq) and np.array_equal(do.view(np.uint32), xd.view(np.uint32))
    worst = check_zp_all(bits, y, wq, wd, wzp, xq, xd, what=f"full {rows}x{k}")
    print(f"  {qmv.last_kernel()}: all {rows} rows, max |err| / tol = {worst:.4f}")


def test_zp_and_packed_graph_replay():
    """Prepared zero-point matvecs (8- and 4-bit) and a packed matrix-core
    product captured in one HIP graph: every replay, with eager work and
    synchronisations in between, gives the eager result bit for bit."""
    announce("zp and packed graph replay")
    rng = np.random.default_rng(5500)
    stream = torch.cuda.Stream()
    s = stream.cuda_stream
    k8, n8 = 896, 4864
    q8, d8, z8 = synth.raw_zp(rng, 8, n8, k8)
    k4, n4 = 4864, 896
    q4, d4, _ = synth.raw_zp(rng, 4, n4, k4, with_zp=False)
    x8 = dev(_x(rng, k8))
    x4 = dev(_x(rng, k4))
    y8 = torch.zeros(n8, dtype=torch.float32, device="cuda:0")
    y4 = torch.zeros(n4, dtype=torch.float32, device="cuda:0")
    wq, wd = synth.raw_q4(rng, 300, 2048)
    xq, xd = orc.quantize_q8(synth.normal(rng, (24, 2048)))
    P = qmv.qmv_pack_weights(dev(wq), dev(wd), 4)
    Y = torch.zeros((24, 300), dtype=torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    calls = [qmv.prepare_matvec_zp_fx(dev(q8), dev(d8), dev(z8), 8, x8, y8, stream=s),
             qmv.prepare_matvec_zp_fx(dev(q4), dev(d4), None, 4, x4, y4, stream=s),
             qmv.prepare_gemm_packed(P, dev(xq), dev(xd), Y, stream=s)]
    with torch.cuda.stream(stream):
        for c in calls:
            c()
    torch.cuda.synchronize()
    outs = (y8, y4, Y)
    eager = [host(t).copy() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in calls:
            c()
    for rep in range(3):
        for t in outs:
            t.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(outs, eager):
            assert np.array_equal(host(t), e), f"replay {rep} differs from the eager result"
    # the eager results against the oracle
    xq8, xd8 = orc.quantize_q8_b128(host(x8))
    _check(8, eager[0], q8, d8, z8, xq8, xd8, 0, n8, "graph zp8")
    xq4, xd4 = orc.quantize_q8_b128(host(x4))
    _check(4, eager[1], q4, d4, None, xq4, xd4, 0, n4, "graph zp4")
    Yref = orc.gemm(4, wq, wd, xq, xd)
    tol = np.stack([orc.tolerance(4, wq, wd, xq[i], xd[i]) for i in range(24)])
    assert np.all(np.abs(eager[2].astype(np.float64) - Yref) <= tol), "graph packed product"


@pytest.mark.parametrize("bits", [4, 8])
def test_zp_and_packed_empty(bits):
    """Zero-row matrices and empty ranges: nothing is written to y, the
    activation output is still produced, packing zero rows is a no-op.  The
    zero-row tensors have null data pointers (torch gives empty tensors
    none), which the calls accept for matrices without rows."""
    announce(f"zp{bits} and packed, empty cases")
    rng = np.random.default_rng(5600 + bits)
    k = 896
    wq = torch.zeros((0, k if bits == 8 else k // 2), dtype=torch.uint8, device="cuda:0")
    wd = torch.zeros((0, k // 128), dtype=torch.float32, device="cuda:0")
    x = _x(rng, k)
    qo = torch.full((k,), 99, dtype=torch.int8, device="cuda:0")
    do = torch.full((k // 128,), -1.0, dtype=torch.float32, device="cuda:0")
    y = torch.full((4,), float(SENTINEL), dtype=torch.float32, device="cuda:0")
    qmv.qmv_matvec_zp_fx(wq, wd, None, bits, dev(x), 0, 0, y, xq_out=(qo, do))
    xq, xd = orc.quantize_q8_b128(x)
    assert np.array_equal(host(qo), xq) and np.array_equal(host(do).view(np.uint32), xd.view(np.uint32))
    assert np.all(host(y) == SENTINEL)
    q4 = torch.zeros((0, 1024), dtype=torch.uint8, device="cuda:0")
    d4 = torch.zeros((0, 64), dtype=torch.float32, device="cuda:0")
    P = qmv.qmv_pack_weights(q4, d4, 4)
    assert (P.rows, P.cols) == (0, 2048)
    wq4, wd4 = synth.raw_q4(rng, 40, 2048)
    P = qmv.qmv_pack_weights(dev(wq4), dev(wd4), 4)
    xq2, xd2 = orc.quantize_q8(synth.normal(rng, (20, 2048)))
    Y = torch.full((20, 40), float(SENTINEL), dtype=torch.float32, device="cuda:0")
    qmv.qmv_gemm_q4_packed(P, dev(xq2), dev(xd2), 16, 16, Y)
    assert np.all(host(Y) == SENTINEL)
