"""A seeded sweep of random shapes through every product entry point (GPU),
each checked on every output against the oracle.

The shapes are drawn once from a fixed seed: row counts 1 .. 9000 and row
sub-ranges that start and end anywhere, K any multiple of the format's block
(up to the entry point's limit), 1 .. 70 activation rows for the batched
product, with and without zero points, so that every launcher choice
(split K or whole rows, row-streaming kernels, matrix-core tiles, the
split-K form of the exported formats, ragged tails) is reached with sizes
the hand-picked cases do not use.  A second draw covers the fused
neighbour forms (rmsnorm, the FFN gate, stacked gate|up pairs) and the
packed-weight product the same way.  Weights are raw random codes and
scales (every code value occurs; quantized normal weights for the fused
neighbour forms), activations normal with 1% outliers x20."""
import numpy as np
import pytest
import torch

from block_quantized_decode_amd import qmv, synth
from gpu_util import announce, check_gemm_all, check_q4k_all, check_zp_all, dev, host
from oracle import oracle as orc
from test_gpu_neighbours import _swiglu_case, _swiglu_check
from test_gpu_silu_fx import _check_activation

pytestmark = pytest.mark.gpu

SENTINEL = np.float32(-12345.5)
_R = np.random.default_rng(20251202)


def _k(rng, block, lo, hi):
    return int(rng.integers(lo // block, hi // block + 1)) * block


def _range(rng, rows):
    if rows < 8 or rng.random() < 0.5:
        return 0, rows
    a = int(rng.integers(0, rows // 2))
    b = int(rng.integers(a + 1, rows + 1))
    return a, b


def _x(rng, m, k):
    x = synth.normal(rng, (m, k))
    flat = x.reshape(-1)
    flat[rng.choice(flat.size, size=max(1, flat.size // 100), replace=False)] *= np.float32(20.0)
    return x


FX = [(int(_R.integers(1, 9000)), _k(_R, 32, 32, 30720), int(q)) for q in _R.choice([4, 8], size=14)]
GEMM = [(int(_R.integers(1, 6000)), _k(_R, 32, 32, 16384), int(_R.integers(2, 71)), int(q))
        for q in _R.choice([4, 8], size=12)]
ZP = [(int(_R.integers(1, 9000)), _k(_R, 128, 128, 16384), int(b), bool(z))
      for b, z in zip(_R.choice([4, 8], size=10), _R.random(10) < 0.7)]
Q4K = [(int(_R.integers(1, 9000)), _k(_R, 256, 256, 16384)) for _ in range(8)]

# the second draw (its own generator, so the shapes above stay as they were)
_R2 = np.random.default_rng(20261202)
RMS = [(int(_R2.integers(1, 9000)), _k(_R2, 32, 32, 30208), int(q)) for q in _R2.choice([4, 8], size=10)]
SILU = [(int(_R2.integers(1, 9000)), _k(_R2, 32, 32, 30720), int(q)) for q in _R2.choice([4, 8], size=8)]
SWIGLU = [(int(_R2.integers(1, 5000)), _k(_R2, 32, 32, 16384), int(q), bool(n))
          for q, n in zip(_R2.choice([4, 8], size=8), _R2.random(8) < 0.5)]
PACKED = [(int(_R2.integers(1, 6000)), _k(_R2, 32, 32, 16384), int(_R2.integers(1, 71)), int(q))
          for q in _R2.choice([4, 8], size=10)]


@pytest.mark.parametrize("rows,k,qtype", FX, ids=[f"q{q}-{r}x{k}" for r, k, q in FX])
def test_random_fused_matvec(rows, k, qtype):
    announce(f"random fx q{qtype} {rows}x{k}")
    rng = np.random.default_rng(rows * 7919 + k)
    wq, wd = synth.raw_q4(rng, rows, k) if qtype == 4 else synth.raw_q8(rng, rows, k)
    x = _x(rng, 1, k).reshape(-1)
    r0, r1 = _range(rng, rows)
    xq, xd = orc.quantize_q8(x)
    ydev = torch.full((rows,), float(SENTINEL), dtype=torch.float32, device="cuda:0")
    qo = torch.zeros(k, dtype=torch.int8, device="cuda:0")
    do = torch.zeros(k // 32, dtype=torch.float32, device="cuda:0")
    f = qmv.qmv_matvec_q4_fx if qtype == 4 else qmv.qmv_matvec_q8_fx
    y = host(f(dev(wq), dev(wd), dev(x), r0, r1, ydev, xq_out=(qo, do)))
    kname = qmv.last_kernel()
    assert np.array_equal(host(qo), xq) and np.array_equal(host(do).view(np.uint32), xd.view(np.uint32))
    assert np.all(y[:r0] == SENTINEL) and np.all(y[r1:] == SENTINEL)
    worst = check_gemm_all(qtype, y.reshape(1, -1), wq, wd, xq.reshape(1, -1), xd.reshape(1, -1), r0, r1,
                           what=f"fx q{qtype} {rows}x{k} [{r0},{r1})")
    print(f"  {kname} [{r0},{r1}): max |err| / tol = {worst:.4f}")


@pytest.mark.parametrize("rows,k,m,qtype", GEMM, ids=[f"q{q}-{r}x{k}-m{m}" for r, k, m, q in GEMM])
def test_random_gemm(rows, k, m, qtype):
    announce(f"random gemm q{qtype} {rows}x{k} m={m}")
    rng = np.random.default_rng(rows * 104729 + k + m)
    wq, wd = synth.raw_q4(rng, rows, k) if qtype == 4 else synth.raw_q8(rng, rows, k)
    xq, xd = orc.quantize_q8(_x(rng, m, k))
    r0, r1 = _range(rng, rows)
    Ydev = torch.full((m, rows), float(SENTINEL), dtype=torch.float32, device="cuda:0")
    f = qmv.qmv_gemm_q4 if qtype == 4 else qmv.qmv_gemm_q8
    Y = host(f(dev(wq), dev(wd), dev(xq), dev(xd), r0, r1, Ydev))
    kname = qmv.last_kernel()
    assert np.all(Y[:, :r0] == SENTINEL) and np.all(Y[:, r1:] == SENTINEL)
    worst = check_gemm_all(qtype, Y, wq, wd, xq, xd, r0, r1, what=f"gemm q{qtype} {rows}x{k} m={m}")
    print(f"  {kname} [{r0},{r1}): max |err| / tol = {worst:.4f}")


@pytest.mark.parametrize("rows,k,bits,with_zp", ZP, ids=[f"zp{b}-{r}x{k}-{z}" for r, k, b, z in ZP])
def test_random_zero_point(rows, k, bits, with_zp):
    announce(f"random zp{bits} {rows}x{k} zp={with_zp}")
    rng = np.random.default_rng(rows * 15485863 + k + bits)
    wq, wd, wzp = synth.raw_zp(rng, bits, rows, k, with_zp)
    x = _x(rng, 1, k).reshape(-1)
    r0, r1 = _range(rng, rows)
    xq, xd = orc.quantize_q8_b128(x)
    ydev = torch.full((rows,), float(SENTINEL), dtype=torch.float32, device="cuda:0")
    qo = torch.zeros(k, dtype=torch.int8, device="cuda:0")
    do = torch.zeros(k // 128, dtype=torch.float32, device="cuda:0")
    y = host(qmv.qmv_matvec_zp_fx(dev(wq), dev(wd), None if wzp is None else dev(wzp), bits, dev(x), r0, r1,
                                  ydev, xq_out=(qo, do)))
    kname = qmv.last_kernel()
    if r1 > r0:
        assert np.array_equal(host(qo), xq) and np.array_equal(host(do).view(np.uint32), xd.view(np.uint32))
    assert np.all(y[:r0] == SENTINEL) and np.all(y[r1:] == SENTINEL)
    worst = check_zp_all(bits, y, wq, wd, wzp, xq, xd, r0, r1, what=f"zp{bits} {rows}x{k}")
    print(f"  {kname} [{r0},{r1}): max |err| / tol = {worst:.4f}")


@pytest.mark.parametrize("rows,k", Q4K, ids=[f"{r}x{k}" for r, k in Q4K])
def test_random_k_quant(rows, k):
    announce(f"random q4k {rows}x{k}")
    rng = np.random.default_rng(rows * 32452843 + k)
    w = synth.raw_q4k(rng, rows, k)
    x = _x(rng, 1, k).reshape(-1)
    r0, r1 = _range(rng, rows)
    xq, xd = orc.quantize_q8_b256(x)
    ydev = torch.full((rows,), float(SENTINEL), dtype=torch.float32, device="cuda:0")
    qo = torch.zeros(k, dtype=torch.int8, device="cuda:0")
    do = torch.zeros(k // 256, dtype=torch.float32, device="cuda:0")
    y = host(qmv.qmv_matvec_q4k_fx(*[dev(a) for a in w], dev(x), r0, r1, ydev, xq_out=(qo, do)))
    kname = qmv.last_kernel()
    if r1 > r0:
        assert np.array_equal(host(qo), xq) and np.array_equal(host(do).view(np.uint32), xd.view(np.uint32))
    assert np.all(y[:r0] == SENTINEL) and np.all(y[r1:] == SENTINEL)
    worst = check_q4k_all(y, w, xq, xd, r0, r1, what=f"q4k {rows}x{k}")
    print(f"  {kname} [{r0},{r1}): max |err| / tol = {worst:.4f}")


def _qweights(rng, qtype, rows, k):
    w = synth.normal(rng, (rows, k), 0.02)
    return orc.quantize_q4(w) if qtype == 4 else orc.quantize_q8(w)


def _acts(k):
    qo = torch.full((k,), 99, dtype=torch.int8, device="cuda:0")
    do = torch.full((k // 32,), -1.0, dtype=torch.float32, device="cuda:0")
    return qo, do


@pytest.mark.parametrize("rows,k,qtype", RMS, ids=[f"q{q}-{r}x{k}" for r, k, q in RMS])
def test_random_rmsnorm_fused(rows, k, qtype):
    """rmsnorm + quantization + product: the quantized normalized activation
    bit for bit, every output in the row range within tolerance."""
    announce(f"random rmsnorm fx q{qtype} {rows}x{k}")
    rng = np.random.default_rng(rows * 6151 + k)
    wq, wd = _qweights(rng, qtype, rows, k)
    x = _x(rng, 1, k).reshape(-1)
    wn = (1.0 + 0.1 * rng.standard_normal(k)).astype(np.float32)
    r0, r1 = _range(rng, rows)
    hq, hd = orc.quantize_q8(orc.rmsnorm(x, wn, 1e-5))
    ydev = torch.full((rows,), float(SENTINEL), dtype=torch.float32, device="cuda:0")
    qo, do = _acts(k)
    f = qmv.qmv_matvec_q4_fx_rmsnorm if qtype == 4 else qmv.qmv_matvec_q8_fx_rmsnorm
    y = host(f(dev(wq), dev(wd), dev(x), dev(wn), 1e-5, r0, r1, ydev, xq_out=(qo, do)))
    kname = qmv.last_kernel()
    if r1 > r0:
        assert np.array_equal(host(qo), hq) and np.array_equal(host(do).view(np.uint32), hd.view(np.uint32))
    assert np.all(y[:r0] == SENTINEL) and np.all(y[r1:] == SENTINEL)
    worst = check_gemm_all(qtype, y.reshape(1, -1), wq, wd, hq.reshape(1, -1), hd.reshape(1, -1), r0, r1,
                           what=f"rmsnorm fx q{qtype} {rows}x{k}")
    print(f"  {kname} [{r0},{r1}): max |err| / tol = {worst:.4f}")


@pytest.mark.parametrize("rows,k,qtype", SILU, ids=[f"q{q}-{r}x{k}" for r, k, q in SILU])
def test_random_silu_mul_fused(rows, k, qtype):
    """The FFN gate + quantization + product: the quantized gate within the
    exp bound of the oracle's, every output within tolerance of the oracle's
    product on the kernel's own codes."""
    announce(f"random silu fx q{qtype} {rows}x{k}")
    rng = np.random.default_rng(rows * 7723 + k)
    wq, wd = _qweights(rng, qtype, rows, k)
    g = (_x(rng, 1, k).reshape(-1) * np.float32(2.0)).astype(np.float32)
    u = _x(rng, 1, k).reshape(-1)
    r0, r1 = _range(rng, rows)
    ydev = torch.full((rows,), float(SENTINEL), dtype=torch.float32, device="cuda:0")
    qo, do = _acts(k)
    f = qmv.qmv_matvec_q4_fx_silu_mul if qtype == 4 else qmv.qmv_matvec_q8_fx_silu_mul
    y = host(f(dev(wq), dev(wd), dev(g), dev(u), r0, r1, ydev, xq_out=(qo, do)))
    kname = qmv.last_kernel()
    qo, do = host(qo), host(do)
    if r1 > r0:
        _check_activation(orc.silu_mul(g, u), qo, do)
    assert np.all(y[:r0] == SENTINEL) and np.all(y[r1:] == SENTINEL)
    worst = check_gemm_all(qtype, y.reshape(1, -1), wq, wd, qo.reshape(1, -1), do.reshape(1, -1), r0, r1,
                           what=f"silu fx q{qtype} {rows}x{k}")
    print(f"  {kname} [{r0},{r1}): max |err| / tol = {worst:.4f}")


@pytest.mark.parametrize("F,k,qtype,norm", SWIGLU, ids=[f"q{q}-F{f}x{k}-{n}" for f, k, q, n in SWIGLU])
def test_random_swiglu(F, k, qtype, norm):
    """Stacked gate|up pairs over a random pair range."""
    announce(f"random swiglu q{qtype} F={F} K={k} norm={norm}")
    wq, wd, x, wn = _swiglu_case(qtype, F, k, F * 3253 + k, norm)
    p0, p1 = _range(np.random.default_rng(F + k), F)
    kname = _swiglu_check(qtype, wq, wd, x, wn, p0, p1)
    print(f"  {kname} pairs [{p0},{p1})")


@pytest.mark.parametrize("rows,k,m,qtype", PACKED, ids=[f"q{q}-{r}x{k}-m{m}" for r, k, m, q in PACKED])
def test_random_packed_gemm(rows, k, m, qtype):
    """The packed-weight product over a row range starting on a 16-row tile:
    every output within tolerance of the oracle, and for 9 or more
    activation rows the same bits as the row-major product."""
    announce(f"random packed gemm q{qtype} {rows}x{k} m={m}")
    rng = np.random.default_rng(rows * 92821 + k + m)
    wq, wd = synth.raw_q4(rng, rows, k) if qtype == 4 else synth.raw_q8(rng, rows, k)
    xq, xd = orc.quantize_q8(_x(rng, m, k))
    r0, r1 = _range(rng, rows)
    r0 -= r0 % 16
    P = qmv.qmv_pack_weights(dev(wq), dev(wd), qtype)
    Yd = torch.full((m, rows), float(SENTINEL), dtype=torch.float32, device="cuda:0")
    fp = qmv.qmv_gemm_q4_packed if qtype == 4 else qmv.qmv_gemm_q8_packed
    Yp = host(fp(P, dev(xq), dev(xd), r0, r1, Yd))
    kname = qmv.last_kernel()
    assert np.all(Yp[:, :r0] == SENTINEL) and np.all(Yp[:, r1:] == SENTINEL)
    if m >= 9:
        f = qmv.qmv_gemm_q4 if qtype == 4 else qmv.qmv_gemm_q8
        Y = host(f(dev(wq), dev(wd), dev(xq), dev(xd)))
        assert np.array_equal(Yp[:, r0:r1].view(np.uint32), Y[:, r0:r1].view(np.uint32))
    worst = check_gemm_all(qtype, Yp, wq, wd, xq, xd, r0, r1, what=f"packed q{qtype} {rows}x{k} m={m}")
    print(f"  {kname} [{r0},{r1}): max |err| / tol = {worst:.4f}")
