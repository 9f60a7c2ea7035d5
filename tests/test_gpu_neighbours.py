"""The decode-step neighbours of the product (GPU): the standalone rmsnorm
and silu_mul launches, the fused forms at every K the LDS budget allows
(the row-streaming kernel takes K / 32 in 33 .. 63 and above 512), and the
stacked gate|up product with the gate applied (qmv_matvec_q*_fx_swiglu).

  * qmv_rmsnorm: every operation correctly rounded in binary32 with the sum
    of squares in a fixed pairwise order, so it must equal oracle.rmsnorm
    bit for bit (order-sensitive inputs included).
  * qmv_silu_mul: exp is the device's single-precision exp, so within the
    spec's 1e-6 relative bound of oracle.silu_mul (C library expf).
  * a standalone neighbour followed by the plain fused product gives the
    fused form's bits (codes, scales and y), whichever kernel runs.
  * swiglu: y bit-identical to the plain (or rmsnorm) fused product of the
    same stacked matrix, a bit-identical to qmv_silu_mul on that y, and y
    within the product's tolerance of the oracle's."""
import numpy as np
import pytest
import torch

from block_quantized_decode_amd import qmv, synth
from gpu_util import announce, check_close, dev, host
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

REL = 2e-6   # twice the spec's exp bound


def _weights(rng, qtype, rows, k):
    w = synth.normal(rng, (rows, k), 0.02)
    return orc.quantize_q4(w) if qtype == 4 else orc.quantize_q8(w)


def _order_sensitive(rng, k):
    """One element of magnitude s and 31 of s * 2^-12 per block, s a random
    power of two per block: the summation order decides the rounding of the
    sum of squares."""
    nb = k // 32
    s = np.float32(2.0) ** rng.integers(-6, 7, size=nb).astype(np.float32)
    sign = np.where(rng.random(k) < 0.5, -1.0, 1.0).astype(np.float32)
    x = np.repeat(s * np.float32(2.0 ** -12), 32).astype(np.float32)
    x[::32] = s
    return x * sign


@pytest.mark.parametrize("n", [32, 64, 96, 2048, 2080, 4096, 5120, 11008, 16384, 30720, 131072])
@pytest.mark.parametrize("kind", ["normal", "order"])
def test_rmsnorm_matches_oracle(n, kind):
    announce(f"rmsnorm n={n} {kind}")
    rng = np.random.default_rng(4000 + n + (1 if kind == "order" else 0))
    x = synth.normal(rng, (n,)) if kind == "normal" else _order_sensitive(rng, n)
    w = (1.0 + 0.1 * rng.standard_normal(n)).astype(np.float32)
    for eps in (1e-5, 0.0):
        ref = orc.rmsnorm(x, w, eps)
        o = host(qmv.qmv_rmsnorm(dev(x), dev(w), eps))
        assert qmv.last_kernel() == "rmsnorm"
        assert np.array_equal(o.view(np.uint32), ref.view(np.uint32)), f"eps={eps}"
    # in place: o = x
    xd = dev(x)
    qmv.qmv_rmsnorm(xd, dev(w), 1e-5, o=xd)
    assert np.array_equal(host(xd).view(np.uint32), orc.rmsnorm(x, w, 1e-5).view(np.uint32)), "in place"


@pytest.mark.parametrize("n", [0, 1, 3, 5, 4096, 5632, 11008, 1000003])
def test_silu_mul_matches_oracle(n):
    announce(f"silu_mul n={n}")
    rng = np.random.default_rng(4100 + n)
    g = (synth.normal(rng, (max(n, 1),)) * np.float32(3.0)).astype(np.float32)[:n]
    u = synth.normal(rng, (max(n, 1),))[:n]
    if n > 100:
        g[rng.choice(n, size=n // 100, replace=False)] *= np.float32(30.0)   # saturated gates, both signs
    ref = orc.silu_mul(g, u).astype(np.float64)
    gd, ud = dev(g), dev(u)
    o = host(qmv.qmv_silu_mul(gd, ud))
    if n == 0:
        return
    err = np.abs(o.astype(np.float64) - ref)
    # for g below about -87.3 the logistic factor 1 / (1 + exp(-g)) is
    # subnormal in binary32; the device's reciprocal may flush it to zero,
    # an absolute difference of at most |g u| 2^-126
    tol = REL * np.abs(ref) + np.abs(g.astype(np.float64) * u) * 2.0 ** -126
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, f"{bad.size} outside; first g={g[bad[0]]!r} u={u[bad[0]]!r} gpu={o[bad[0]]!r} ref={ref[bad[0]]!r}"
    # in place over g: the same bits
    qmv.qmv_silu_mul(gd, ud, o=gd)
    assert np.array_equal(host(gd), o)


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("rows,k", [(40, 32 * 33), (7, 32 * 40), (129, 32 * 63), (33, 32 * 520),
                                    (65, 32 * 800), (9, 30208)])
def test_fused_forms_every_k(qtype, rows, k):
    """K / 32 outside the split-K range: the row-streaming kernel's fused
    forms, against the oracle and against standalone neighbour + plain
    fused product (same bits)."""
    announce(f"fused forms every K q{qtype} {rows}x{k}")
    rng = np.random.default_rng(4200 + rows + k)
    wq, wd = _weights(rng, qtype, rows, k)
    wqd, wdd = dev(wq), dev(wd)
    x = synth.normal(rng, (k,))
    wn = (1.0 + 0.1 * rng.standard_normal(k)).astype(np.float32)
    fxn = qmv.qmv_matvec_q4_fx_rmsnorm if qtype == 4 else qmv.qmv_matvec_q8_fx_rmsnorm
    fxs = qmv.qmv_matvec_q4_fx_silu_mul if qtype == 4 else qmv.qmv_matvec_q8_fx_silu_mul
    fx = qmv.qmv_matvec_q4_fx if qtype == 4 else qmv.qmv_matvec_q8_fx

    def run(f, *args):
        qo = torch.full((k,), 99, dtype=torch.int8, device="cuda:0")
        do = torch.full((k // 32,), -1.0, dtype=torch.float32, device="cuda:0")
        y = host(f(wqd, wdd, *args, xq_out=(qo, do)))
        return y, host(qo), host(do), qmv.last_kernel()

    # rmsnorm form: codes bit-exact against the oracle
    y, qo, do, kname = run(fxn, dev(x), dev(wn), 1e-5)
    assert kname.startswith("rows_") and "_fxn" in kname, kname
    hq, hd = orc.quantize_q8(orc.rmsnorm(x, wn, 1e-5))
    assert np.array_equal(qo, hq) and np.array_equal(do.view(np.uint32), hd.view(np.uint32))
    check_close(qtype, y, orc.matvec(qtype, wq, wd, hq, hd), wq, wd, hq, hd, what="rmsnorm form")
    h = qmv.qmv_rmsnorm(dev(x), dev(wn), 1e-5)
    y2, qo2, do2, _ = run(fx, h)
    assert np.array_equal(y2, y) and np.array_equal(qo2, qo) and np.array_equal(do2, do), "rmsnorm + plain"
    # silu form: the activation within the exp bound, y on the kernel's own codes
    if k <= 30720:
        g = (synth.normal(rng, (k,)) * np.float32(2.0)).astype(np.float32)
        y, qo, do, kname = run(fxs, dev(g), dev(x))
        assert kname.startswith("rows_") and "_fxs" in kname, kname
        aq, ad = orc.quantize_q8(orc.silu_mul(g, x))
        assert np.all(np.abs(do.astype(np.float64) - ad) <= REL * ad), "silu form scales"
        assert np.all(np.abs(qo.astype(np.int32) - aq.astype(np.int32)) <= 1), "silu form codes"
        check_close(qtype, y, orc.matvec(qtype, wq, wd, qo, do), wq, wd, qo, do, what="silu form")
        a = qmv.qmv_silu_mul(dev(g), dev(x))
        y2, qo2, do2, _ = run(fx, a)
        assert np.array_equal(y2, y) and np.array_equal(qo2, qo) and np.array_equal(do2, do), "silu_mul + plain"


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("k", [2048, 4096])
def test_split_k_forms_equal_standalone_chain(qtype, k):
    """In the split-K range too, standalone neighbour + plain fused product
    = the fused form, bit for bit."""
    announce(f"split-K fused = chain q{qtype} K={k}")
    rng = np.random.default_rng(4300 + k)
    rows = 1000
    wq, wd = _weights(rng, qtype, rows, k)
    wqd, wdd = dev(wq), dev(wd)
    x, g = synth.normal(rng, (k,)), synth.normal(rng, (k,))
    wn = (1.0 + 0.1 * rng.standard_normal(k)).astype(np.float32)
    fxn = qmv.qmv_matvec_q4_fx_rmsnorm if qtype == 4 else qmv.qmv_matvec_q8_fx_rmsnorm
    fxs = qmv.qmv_matvec_q4_fx_silu_mul if qtype == 4 else qmv.qmv_matvec_q8_fx_silu_mul
    fx = qmv.qmv_matvec_q4_fx if qtype == 4 else qmv.qmv_matvec_q8_fx
    y1 = host(fxn(wqd, wdd, dev(x), dev(wn), 1e-5))
    assert qmv.last_kernel().startswith("fxn_")
    y2 = host(fx(wqd, wdd, qmv.qmv_rmsnorm(dev(x), dev(wn), 1e-5)))
    assert np.array_equal(y1, y2)
    y1 = host(fxs(wqd, wdd, dev(g), dev(x)))
    assert qmv.last_kernel().startswith("fxs_")
    y2 = host(fx(wqd, wdd, qmv.qmv_silu_mul(dev(g), dev(x))))
    assert np.array_equal(y1, y2)


def _swiglu_case(qtype, F, k, seed, norm):
    rng = np.random.default_rng(seed)
    wq, wd = _weights(rng, qtype, 2 * F, k)
    x = synth.normal(rng, (k,))
    wn = (1.0 + 0.1 * rng.standard_normal(k)).astype(np.float32) if norm else None
    return wq, wd, x, wn


def _swiglu_check(qtype, wq, wd, x, wn, p0=None, p1=None, expect_fused=None):
    F = wq.shape[0] // 2
    k = x.size
    p0 = 0 if p0 is None else p0
    p1 = F if p1 is None else p1
    wqd, wdd = dev(wq), dev(wd)
    wnd = dev(wn) if wn is not None else None
    qo = torch.full((k,), 99, dtype=torch.int8, device="cuda:0")
    do = torch.full((k // 32,), -1.0, dtype=torch.float32, device="cuda:0")
    a = torch.full((F,), -7.5, dtype=torch.float32, device="cuda:0")
    y = torch.full((2 * F,), -7.5, dtype=torch.float32, device="cuda:0")
    qmv.qmv_matvec_fx_swiglu(qtype, wqd, wdd, dev(x), wnd, 1e-5, p0, p1, a=a, y=y, xq_out=(qo, do))
    kname = qmv.last_kernel()
    if expect_fused is not None:
        assert kname.endswith("_gu") == expect_fused, kname
    a, y, qo, do = host(a), host(y), host(qo), host(do)
    # untouched outside the pair range
    assert np.all(a[:p0] == -7.5) and np.all(a[p1:] == -7.5)
    assert np.all(y[:p0] == -7.5) and np.all(y[p1:F + p0] == -7.5) and np.all(y[F + p1:] == -7.5)
    # the quantized activation against the oracle, and y against the oracle
    h = orc.rmsnorm(x, wn, 1e-5) if wn is not None else x
    hq, hd = orc.quantize_q8(h)
    if p1 > p0:   # (an empty range launches nothing, as every product entry point)
        assert np.array_equal(qo, hq) and np.array_equal(do.view(np.uint32), hd.view(np.uint32))
    yref = orc.matvec(qtype, wq, wd, hq, hd)
    if p1 > p0:
        check_close(qtype, y, yref, wq, wd, hq, hd, p0, p1, what="gate rows")
        check_close(qtype, y, yref, wq, wd, hq, hd, F + p0, F + p1, what="up rows")
    # y = the plain fused product of the stacked matrix, bit for bit
    if wn is not None:
        f = qmv.qmv_matvec_q4_fx_rmsnorm if qtype == 4 else qmv.qmv_matvec_q8_fx_rmsnorm
        yp = host(f(wqd, wdd, dev(x), wnd, 1e-5))
    else:
        f = qmv.qmv_matvec_q4_fx if qtype == 4 else qmv.qmv_matvec_q8_fx
        yp = host(f(wqd, wdd, dev(x)))
    assert np.array_equal(y[p0:p1], yp[p0:p1]) and np.array_equal(y[F + p0:F + p1], yp[F + p0:F + p1])
    # a = qmv_silu_mul on that y bit for bit, and the oracle's silu_mul within the exp bound
    if p1 > p0:
        ag = host(qmv.qmv_silu_mul(dev(y[p0:p1]), dev(y[F + p0:F + p1])))
        assert np.array_equal(a[p0:p1], ag), "gate differs from qmv_silu_mul on the same y"
        ar = orc.silu_mul(y[p0:p1], y[F + p0:F + p1]).astype(np.float64)
        gu = np.abs(y[p0:p1].astype(np.float64) * y[F + p0:F + p1])
        assert np.all(np.abs(a[p0:p1] - ar) <= REL * np.abs(ar) + gu * 2.0 ** -126)
    return kname


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("F,k,fused", [(1, 2048, True), (3, 2048, True), (5, 2048, True), (257, 2080, True),
                                       (1031, 4096, True), (61, 5632, True), (130, 16384, True),
                                       (33, 512, False), (7, 1280, False), (40, 32 * 520, False)])
@pytest.mark.parametrize("norm", [False, True])
def test_swiglu_matches_oracle(qtype, F, k, fused, norm):
    announce(f"swiglu q{qtype} F={F} K={k} norm={norm}")
    wq, wd, x, wn = _swiglu_case(qtype, F, k, 4400 + F + k, norm)
    _swiglu_check(qtype, wq, wd, x, wn, expect_fused=fused)


@pytest.mark.parametrize("qtype", [4, 8])
def test_swiglu_pair_ranges(qtype):
    announce(f"swiglu pair ranges q{qtype}")
    F, k = 1333, 4096
    wq, wd, x, wn = _swiglu_case(qtype, F, k, 4500, True)
    for p0, p1 in ((0, F), (1, 2), (17, 1300), (1329, 1333), (640, 640), (0, 4)):
        _swiglu_check(qtype, wq, wd, x, wn, p0, p1)
    # fallback path: the gate launch on views 12 bytes past 16-byte alignment (its scalar form)
    wq, wd, x, wn = _swiglu_case(qtype, 99, 1280, 4501, False)
    for p0, p1 in ((3, 98), (1, 2)):
        _swiglu_check(qtype, wq, wd, x, wn, p0, p1, expect_fused=False)


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("F,k", [(5632, 2048), (11008, 4096)])
def test_swiglu_full_size(qtype, F, k):
    """TinyLlama-1.1B (W_gate|W_up 11264 x 2048) and Llama-7B (22016 x 4096)."""
    announce(f"swiglu full size q{qtype} F={F} K={k}")
    wq, wd, x, wn = _swiglu_case(qtype, F, k, 4600 + F, True)
    _swiglu_check(qtype, wq, wd, x, wn, expect_fused=True)


def test_swiglu_graph_replay():
    """rmsnorm+gate|up+gate, then the down projection on the gate's output,
    captured in one HIP graph: every replay equals the eager result."""
    announce("swiglu graph replay")
    rng = np.random.default_rng(4700)
    k, F = 2048, 5632
    stream = torch.cuda.Stream()
    s = stream.cuda_stream
    gq, gd = (dev(t) for t in _weights(rng, 4, 2 * F, k))
    dq, dd = (dev(t) for t in _weights(rng, 4, k, F))
    x = dev(synth.normal(rng, (k,)))
    wn = dev((1.0 + 0.1 * rng.standard_normal(k)).astype(np.float32))
    a = torch.zeros(F, dtype=torch.float32, device="cuda:0")
    y = torch.zeros(2 * F, dtype=torch.float32, device="cuda:0")
    out = torch.zeros(k, dtype=torch.float32, device="cuda:0")
    calls = [qmv.prepare_matvec_fx_swiglu(4, gq, gd, x, a, y, w_norm=wn, eps=1e-5, stream=s),
             qmv.prepare_matvec_fx(4, dq, dd, a, out, stream=s)]
    with torch.cuda.stream(stream):
        for c in calls:
            c()
    torch.cuda.synchronize()
    eager = [host(t).copy() for t in (a, y, out)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for c in calls:
            c()
    for rep in range(3):
        for t in (a, y, out):
            t.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, e in zip((a, y, out), eager):
            assert np.array_equal(host(t), e), f"replay {rep}"
