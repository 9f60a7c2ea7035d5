"""Every count of last passes in the split-K kernels (GPU parity).

The split-K matvec kernels (the fused product, its pre-quantized and 4-row
matrix-core forms, the stacked gate|up form and the split-K kernel of the
4-bit exported formats) run whole ring turns of D passes while every load of
the turn falls among a wavefront's passes; the remaining R passes (1 .. 2 D
- 2) run as code specialised on R.  Rows are spread over one workgroup per
compute unit in whole 4-row passes, so rows = 4 p x (compute units) gives
every wavefront p passes, and p = 1 .. 7 and 10 reach every R for D = 4
(R = p up to 6, then 3 and 6) and for D = 3; rows 3 short of that leave the last
workgroup a shorter count.  The whole-row form (K / 32 <= 32) takes every
4th pass of 2-row passes, so there rows = 8 p x (compute units).  Each case
is compared with the oracle on every output."""
import numpy as np
import pytest
import torch

from block_quantized_decode_amd import qmv, synth
from gpu_util import announce, check_gemm_all, check_q4k_all, check_zp_all, dev, host
from oracle import oracle as orc
from test_gpu_neighbours import _swiglu_case, _swiglu_check

pytestmark = pytest.mark.gpu

PASSES = [1, 2, 3, 4, 5, 6, 7, 10]


def _cus() -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count


def _rows(p, per_pass=4, short=0):
    return per_pass * p * _cus() - short


def _x(rng, k):
    x = synth.normal(rng, (k,))
    x[rng.choice(k, size=max(1, k // 100), replace=False)] *= np.float32(20.0)
    return x


# Q4_0 with 257 .. 384 blocks per row runs 2 blocks per lane on K / 1024
# wavefronts where at most 5% of the block slots stay empty (K = 9216,
# 10240, 11008 and 12288 on 9, 10, 11 and 12), else 3 blocks on 8 (K = 8448)
FX_Q4_NAME = {4096: "fx_q4_t16_n1_d4_w8", 8448: "fx_q4_t16_n3_d3_w8", 9216: "fx_q4_t16_n2_d3_w9",
              10240: "fx_q4_t16_n2_d3_w10", 11008: "fx_q4_t16_n2_d3_w11", 12288: "fx_q4_t16_n2_d3_w12"}


@pytest.mark.parametrize("qtype,k", [(q, k) for q in (4, 8) for k in (4096, 11008)] +
                         [(4, k) for k in (8448, 9216, 10240, 12288)])
@pytest.mark.parametrize("p", PASSES)
def test_fused_every_tail(qtype, k, p):
    rows = _rows(p, short=3 if p in (2, 5) else 0)
    announce(f"tail fx q{qtype} {rows}x{k} p={p}")
    rng = np.random.default_rng(7000 + 31 * p + k + qtype)
    wq, wd = synth.raw_q4(rng, rows, k) if qtype == 4 else synth.raw_q8(rng, rows, k)
    x = _x(rng, k)
    xq, xd = orc.quantize_q8(x)
    f = qmv.qmv_matvec_q4_fx if qtype == 4 else qmv.qmv_matvec_q8_fx
    y = host(f(dev(wq), dev(wd), dev(x)))
    assert qmv.last_kernel().startswith("fx_"), qmv.last_kernel()
    if qtype == 4:
        assert qmv.last_kernel() == FX_Q4_NAME[k], qmv.last_kernel()
    check_gemm_all(qtype, y.reshape(1, -1), wq, wd, xq.reshape(1, -1), xd.reshape(1, -1),
                   what=f"fx q{qtype} {rows}x{k}")


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("p", PASSES)
def test_whole_rows_every_tail(qtype, p):
    k = 896
    rows = _rows(p, per_pass=8, short=3 if p in (2, 5) else 0)
    announce(f"tail fx whole rows q{qtype} {rows}x{k} p={p}")
    rng = np.random.default_rng(7100 + p + qtype)
    wq, wd = synth.raw_q4(rng, rows, k) if qtype == 4 else synth.raw_q8(rng, rows, k)
    x = _x(rng, k)
    xq, xd = orc.quantize_q8(x)
    f = qmv.qmv_matvec_q4_fx if qtype == 4 else qmv.qmv_matvec_q8_fx
    y = host(f(dev(wq), dev(wd), dev(x)))
    assert qmv.last_kernel().startswith("fx_"), qmv.last_kernel()
    check_gemm_all(qtype, y.reshape(1, -1), wq, wd, xq.reshape(1, -1), xd.reshape(1, -1),
                   what=f"fx whole rows q{qtype} {rows}x{k}")


# (qtype, M, K): Q8_0 and Q4_0 with 2 and 3 pre-quantized rows (the fused
# kernel's pre-quantized form, 3 blocks per lane and a ring of 3), Q4_0
# with 4 rows (the 4 x 4 matrix-core form)
PREQ = [(8, 2, 11008), (8, 3, 11008), (4, 2, 11008), (4, 3, 11008), (4, 4, 4096), (4, 4, 11008)]


@pytest.mark.parametrize("qtype,m,k", PREQ)
@pytest.mark.parametrize("p", PASSES)
def test_prequantized_every_tail(qtype, m, k, p):
    rows = _rows(p, short=3 if p in (2, 5) else 0)
    announce(f"tail gemm q{qtype} m={m} {rows}x{k} p={p}")
    rng = np.random.default_rng(7200 + 31 * p + k + m)
    wq, wd = synth.raw_q4(rng, rows, k) if qtype == 4 else synth.raw_q8(rng, rows, k)
    xq, xd = orc.quantize_q8(np.stack([_x(rng, k) for _ in range(m)]))
    f = qmv.qmv_gemm_q4 if qtype == 4 else qmv.qmv_gemm_q8
    Y = host(f(dev(wq), dev(wd), dev(xq), dev(xd)))
    kname = qmv.last_kernel()
    assert kname.startswith("mq_" if m == 4 else "px_"), kname
    check_gemm_all(qtype, Y, wq, wd, xq, xd, what=f"gemm q{qtype} m={m} {rows}x{k}")


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("p,short", [(1, 0), (2, 0), (3, 0), (1, 3), (2, 3), (3, 3)])
def test_swiglu_every_tail(qtype, p, short):
    """Stacked gate|up pairs: a wavefront's passes are its gate passes then
    as many up passes (2 p in all)."""
    F, k = _rows(p, short=short), 4096
    announce(f"tail swiglu q{qtype} F={F} K={k}")
    wq, wd, x, wn = _swiglu_case(qtype, F, k, 7300 + 7 * p + short, True)
    _swiglu_check(qtype, wq, wd, x, wn, expect_fused=True)


@pytest.mark.parametrize("k", [4096, 11008])
@pytest.mark.parametrize("p", PASSES)
def test_zero_point_every_tail(k, p):
    rows = _rows(p, short=3 if p in (2, 5) else 0)
    announce(f"tail zp4 {rows}x{k} p={p}")
    rng = np.random.default_rng(7400 + 31 * p + k)
    wq, wd, wzp = synth.raw_zp(rng, 4, rows, k, True)
    x = _x(rng, k)
    xq, xd = orc.quantize_q8_b128(x)
    y = host(qmv.qmv_matvec_zp_fx(dev(wq), dev(wd), dev(wzp), 4, dev(x)))
    check_zp_all(4, y, wq, wd, wzp, xq, xd, what=f"zp4 {rows}x{k} ({qmv.last_kernel()})")


@pytest.mark.parametrize("k", [2048, 4096, 11008])
@pytest.mark.parametrize("p", PASSES)
def test_k_quant_every_tail(k, p):
    rows = _rows(p, short=3 if p in (2, 5) else 0)
    announce(f"tail q4k {rows}x{k} p={p}")
    rng = np.random.default_rng(7500 + 31 * p + k)
    w = synth.raw_q4k(rng, rows, k)
    x = _x(rng, k)
    xq, xd = orc.quantize_q8_b256(x)
    y = host(qmv.qmv_matvec_q4k_fx(*[dev(a) for a in w], dev(x)))
    check_q4k_all(y, w, xq, xd, what=f"q4k {rows}x{k} ({qmv.last_kernel()})")
