"""The split-K form of the 4-bit zero-point and K-quant products
(kernels_gs.hip) on the GPU against the oracle: 8 wavefronts per workgroup
for rows of at least 128 units of 32 elements and at least 16 rows per
compute unit, 4 wavefronts for fewer rows of at least 64 units (slices of at
most 64 units either way).

The activation codes and scales must equal the oracle's bit for bit and
every row must be within the oracle's tolerance, as for the row-streaming
kernels.  The cases cover each units-per-lane count (K = 4096: 1 unit per
lane and pass, 8192: 2 on 8 wavefronts, 12288 and 11008: 2 on 12 and 11,
16384: 4), with and without
zero points, K-quant super-blocks, row counts that leave a
ragged last pass and a short last workgroup, row sub-ranges, repeated calls
(same bits) and unit scales (the exact integer sums).  8-bit zero-point
codes keep the row-streaming kernel (test_gpu_zp.py)."""
import numpy as np
import pytest
import torch

from block_quantized_decode_amd import qmv, synth
from gpu_util import announce, check_q4k_all, check_zp_all, dev, host
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

SENTINEL = np.float32(-12345.5)


def _x(rng, k):
    x = synth.normal(rng, (k,))
    x[rng.choice(k, size=max(1, k // 100), replace=False)] *= np.float32(20.0)
    return x


def _zp(bits, wq, wd, wzp, x, r0=None, r1=None, y=None):
    k = x.size
    qo = torch.full((k,), 99, dtype=torch.int8, device="cuda:0")
    do = torch.full((k // 128,), -1.0, dtype=torch.float32, device="cuda:0")
    y = qmv.qmv_matvec_zp_fx(dev(wq), dev(wd), None if wzp is None else dev(wzp), bits, dev(x), r0, r1, y,
                             xq_out=(qo, do))
    return host(y), host(qo), host(do), qmv.last_kernel()


def _q4k(w, x, r0=None, r1=None, y=None):
    k = x.size
    qo = torch.full((k,), 99, dtype=torch.int8, device="cuda:0")
    do = torch.full((k // 256,), -1.0, dtype=torch.float32, device="cuda:0")
    y = qmv.qmv_matvec_q4k_fx(*[dev(a) for a in w], dev(x), r0, r1, y, xq_out=(qo, do))
    return host(y), host(qo), host(do), qmv.last_kernel()


def _nc(k, g, w=8):
    """Units per lane and pass the launcher picks (w wavefronts, 16 lanes a row).
    With 8 wavefronts, rows of 257 .. 384 units whose nu / 32 wavefronts
    (9 .. 12) hold 2 units per lane with at most 5% of the slots empty take
    those instead (K = 11008 on 11, 12288 on 12)."""
    nu = k // 32
    w2 = -(-nu // 32)
    if w == 8 and 256 < nu and w2 <= 12 and 20 * nu >= 19 * 32 * w2 and -(-(nu // g) // w2) * g == 32:
        return 2
    s = -(-(nu // g) // w) * g
    return -(-s // 16)


ZP_SHAPES = [(4096, 4096), (4099, 4096), (5003, 8192), (4096, 12288), (4100, 11008), (11008, 4096),
             (4096, 11008), (4097, 16384)]


@pytest.mark.parametrize("bits", [4])
@pytest.mark.parametrize("rows,k", ZP_SHAPES)
@pytest.mark.parametrize("with_zp", [True, False])
def test_gs_zp_matches_oracle(bits, rows, k, with_zp):
    announce(f"gs zp{bits} {rows}x{k} zp={with_zp}")
    rng = np.random.default_rng(7000 + rows + k + bits + with_zp)
    wq, wd, wzp = synth.raw_zp(rng, bits, rows, k, with_zp)
    x = _x(rng, k)
    xq, xd = orc.quantize_q8_b128(x)
    y, qo, do, kname = _zp(bits, wq, wd, wzp, x)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert kname.startswith(f"gs_zp{bits}_n{_nc(k, 4)}_"), kname
    assert np.array_equal(qo, xq), "activation codes"
    assert np.array_equal(do.view(np.uint32), xd.view(np.uint32)), "activation scales"
    worst = check_zp_all(bits, y, wq, wd, wzp, xq, xd, what=f"gs zp{bits} {rows}x{k}")
    print(f"  {kname}: max |err| / tol = {worst:.4f}")
    y2, _, _, _ = _zp(bits, wq, wd, wzp, x)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "same inputs, same bits"


Q4K_SHAPES = [(4096, 4096), (4099, 4096), (5003, 8192), (4096, 12288), (4100, 11008), (11008, 4096),
              (4096, 11008), (4097, 16384)]


@pytest.mark.parametrize("rows,k", Q4K_SHAPES)
def test_gs_q4k_matches_oracle(rows, k):
    announce(f"gs q4k {rows}x{k}")
    rng = np.random.default_rng(7100 + rows + k)
    w = synth.raw_q4k(rng, rows, k)
    x = _x(rng, k)
    xq, xd = orc.quantize_q8_b256(x)
    y, qo, do, kname = _q4k(w, x)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert kname.startswith(f"gs_q4k_n{_nc(k, 8)}_"), kname
    assert np.array_equal(qo, xq) and np.array_equal(do.view(np.uint32), xd.view(np.uint32))
    worst = check_q4k_all(y, w, xq, xd, what=f"gs q4k {rows}x{k}")
    print(f"  {kname}: max |err| / tol = {worst:.4f}")
    y2, _, _, _ = _q4k(w, x)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "same inputs, same bits"


@pytest.mark.parametrize("fmt", ["zp4", "q4k"])
def test_gs_row_ranges(fmt):
    """Sub-ranges of rows (at least 16 per compute unit, so the split-K
    form runs) write exactly their rows."""
    announce(f"gs row ranges {fmt}")
    rng = np.random.default_rng(7200)
    rows, k = 9001, 11008
    x = _x(rng, k)
    if fmt == "q4k":
        w = synth.raw_q4k(rng, rows, k)
        xq, xd = orc.quantize_q8_b256(x)
    else:
        bits = int(fmt[2])
        wq, wd, wzp = synth.raw_zp(rng, bits, rows, k, True)
        xq, xd = orc.quantize_q8_b128(x)
    for r0, r1 in ((0, rows), (3, 4099 + 3), (4901, rows), (17, 8207)):
        ydev = torch.full((rows,), float(SENTINEL), dtype=torch.float32, device="cuda:0")
        if fmt == "q4k":
            y, _, _, kname = _q4k(w, x, r0, r1, ydev)
            check_q4k_all(y, w, xq, xd, r0, r1, what=f"[{r0},{r1})")
        else:
            y, _, _, kname = _zp(bits, wq, wd, wzp, x, r0, r1, ydev)
            check_zp_all(bits, y, wq, wd, wzp, xq, xd, r0, r1, what=f"[{r0},{r1})")
        if torch.cuda.get_device_properties(0).multi_processor_count == 256:
            assert kname.startswith("gs_"), kname
        assert np.all(y[:r0] == SENTINEL) and np.all(y[r1:] == SENTINEL), f"rows outside [{r0},{r1}) written"


@pytest.mark.parametrize("bits", [4])
def test_gs_zp_unit_scales_exact(bits):
    """Integer activation with block maxima 127 (dx = 1, q = x) and dw = 1:
    y is the exact integer sum of (B - zp) * q over the row, extreme codes
    and zero points included."""
    announce(f"gs zp{bits} unit scales")
    rng = np.random.default_rng(7300 + bits)
    rows, k = 4104, 8192
    top = (1 << bits) - 1
    B = rng.integers(0, top + 1, size=(rows, k)).astype(np.int64)
    B[0, :] = top
    B[1, :] = 0
    zp = rng.integers(0, top + 1, size=(rows, k // 128)).astype(np.int64)
    zp[0, :] = 0
    zp[1, :] = top
    x = rng.integers(-3, 4, size=k).astype(np.float32)
    x[::128] = 127.0                       # every block's maximum is 127
    if bits == 8:
        wq = B.astype(np.uint8)
    else:
        wq = (B[:, 0::2] | (B[:, 1::2] << 4)).astype(np.uint8)
    wd = np.ones((rows, k // 128), np.float32)
    y, qo, do, kname = _zp(bits, wq, wd, zp.astype(np.uint8), x)
    assert np.array_equal(qo, x.astype(np.int8)) and np.all(do == 1.0)
    blk = ((B - np.repeat(zp, 128, axis=1)) * x.astype(np.int64)).reshape(rows, k // 128, 128).sum(axis=2)
    # every partial sum of block sums is an integer below 2^24: exact in fp32 in any order
    assert np.all(np.abs(blk).sum(axis=1) < 2 ** 24)
    assert np.array_equal(y.astype(np.int64), blk.sum(axis=1)), kname


def test_gs_q4k_unit_scales_exact():
    """d = dmin = 1 with integer activation (dx = 1): y = sum_b sc_b * dot_b -
    mn_b * sum q_b over the row, exactly (|y| < 2^24 here)."""
    announce("gs q4k unit scales")
    rng = np.random.default_rng(7400)
    rows, k = 4104, 4096
    nsub = k // 32
    wv = rng.integers(0, 16, size=(rows, k)).astype(np.int64)
    sc = rng.integers(0, 64, size=(rows, nsub)).astype(np.int64)
    mn = rng.integers(0, 64, size=(rows, nsub)).astype(np.int64)
    wv[0, :] = 15
    sc[0, :] = 63
    mn[1, :] = 63
    # the spec's Q4_0 nibble order within each sub-block: byte j = element j | element j + 16 << 4
    sub = wv.reshape(rows, nsub, 32)
    q = (sub[:, :, :16] | (sub[:, :, 16:] << 4)).astype(np.uint8).reshape(rows, k // 2)
    x = rng.integers(-3, 4, size=k).astype(np.float32)
    x[::256] = 127.0
    d = np.ones((rows, k // 256), np.float32)
    dmin = np.ones((rows, k // 256), np.float32)
    w = (q, sc.astype(np.uint8), mn.astype(np.uint8), d, dmin)
    y, qo, do, kname = _q4k(w, x)
    assert np.array_equal(qo, x.astype(np.int8)) and np.all(do == 1.0)
    xs = x.astype(np.int64).reshape(nsub, 32)
    dots = (sub * xs[None]).sum(axis=2)
    s1 = (sc * dots).reshape(rows, k // 256, 8).sum(axis=2)
    s2 = (mn * xs.sum(axis=1)[None]).reshape(rows, k // 256, 8).sum(axis=2)
    # every partial sum is an integer below 2^24: exact in fp32 in any order
    assert np.all((np.abs(s1) + np.abs(s2)).sum(axis=1) < 2 ** 24)
    assert np.array_equal(y.astype(np.int64), (s1 - s2).sum(axis=1)), kname


# Fewer than 16 rows per compute unit: 4 wavefronts, 1 .. 4 units per lane and
# pass (K = 2048: 1; 4096: 2; 4864 and 5632: 3; 8192: 4), a ragged last pass,
# a workgroup of fewer rows than a pass, and the most rows below the 8-wavefront form.
W4_SHAPES = [(3, 2048), (256, 2048), (2048, 2048), (4095, 4096), (896, 4864), (2049, 5632), (1000, 8192)]


@pytest.mark.parametrize("fmt", ["zp4", "q4k"])
@pytest.mark.parametrize("rows,k", W4_SHAPES)
def test_gs_four_wavefronts(fmt, rows, k):
    announce(f"gs {fmt} four wavefronts {rows}x{k}")
    rng = np.random.default_rng(7400 + rows + k)
    x = _x(rng, k)
    if fmt == "q4k":
        w = synth.raw_q4k(rng, rows, k)
        xq, xd = orc.quantize_q8_b256(x)
        y, qo, do, kname = _q4k(w, x)
        worst = check_q4k_all(y, w, xq, xd, what=f"gs q4k {rows}x{k}")
        y2 = _q4k(w, x)[0]
    else:
        wq, wd, wzp = synth.raw_zp(rng, 4, rows, k, True)
        xq, xd = orc.quantize_q8_b128(x)
        y, qo, do, kname = _zp(4, wq, wd, wzp, x)
        worst = check_zp_all(4, y, wq, wd, wzp, xq, xd, what=f"gs zp4 {rows}x{k}")
        y2 = _zp(4, wq, wd, wzp, x)[0]
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        nc = _nc(k, 8 if fmt == 'q4k' else 4, 4)
        assert kname == f"gs_{fmt}_n{nc}_d{3 if fmt == 'q4k' and nc >= 2 else 4}_w4", kname
    assert np.array_equal(qo, xq) and np.array_equal(do.view(np.uint32), xd.view(np.uint32))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "same inputs, same bits"
    print(f"  {kname}: max |err| / tol = {worst:.4f}")


@pytest.mark.parametrize("fmt", ["zp4", "q4k"])
def test_gs_four_wavefronts_row_ranges(fmt):
    """Sub-ranges of a 3001-row matrix (the 4-wavefront form) write exactly
    their rows."""
    announce(f"gs four wavefronts row ranges {fmt}")
    rng = np.random.default_rng(7500)
    rows, k = 3001, 5632
    x = _x(rng, k)
    if fmt == "q4k":
        w = synth.raw_q4k(rng, rows, k)
        xq, xd = orc.quantize_q8_b256(x)
    else:
        wq, wd, wzp = synth.raw_zp(rng, 4, rows, k, True)
        xq, xd = orc.quantize_q8_b128(x)
    for r0, r1 in ((0, rows), (1, 2), (5, 1029), (2990, rows)):
        ydev = torch.full((rows,), float(SENTINEL), dtype=torch.float32, device="cuda:0")
        if fmt == "q4k":
            y, _, _, kname = _q4k(w, x, r0, r1, ydev)
            check_q4k_all(y, w, xq, xd, r0, r1, what=f"[{r0},{r1})")
        else:
            y, _, _, kname = _zp(4, wq, wd, wzp, x, r0, r1, ydev)
            check_zp_all(4, y, wq, wd, wzp, xq, xd, r0, r1, what=f"[{r0},{r1})")
        if torch.cuda.get_device_properties(0).multi_processor_count == 256:
            assert kname.endswith("_w4") and kname.startswith("gs_"), kname
        assert np.all(y[:r0] == SENTINEL) and np.all(y[r1:] == SENTINEL), f"rows outside [{r0},{r1}) written"
