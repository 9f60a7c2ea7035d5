"""Quantization kernels against the oracle, bit for bit (GPU)."""
import numpy as np
import pytest
import torch

import pins
from block_quantized_decode_amd import qmv, synth
from gpu_util import announce, dev, host
from oracle import oracle as orc

pytestmark = pytest.mark.gpu


def _q8_gpu(x):
    q, d = qmv.qmv_quantize_q8(dev(x))
    return host(q), host(d)


@pytest.mark.parametrize("shape,scale", [((32,), 1.0), ((64 * 1024,), 1.0), ((7, 4096), 3.0),
                                         ((3, 11008), 1e-3), ((1, 896), 1e4)])
def test_quantize_q8_bitexact(shape, scale):
    announce(f"quantize_q8 {shape} x{scale}")
    rng = np.random.default_rng(100)
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    x.reshape(-1)[::37] *= np.float32(20.0)
    q, d = _q8_gpu(x)
    qr, dr = orc.quantize_q8(x)
    assert np.array_equal(q, qr)
    assert np.array_equal(d.view(np.uint32), dr.view(np.uint32))


def test_quantize_q8_closed_forms_and_detectors():
    announce("quantize_q8 detectors")
    blocks = []
    for case in pins.golden("q8_rounding_detectors.json")["cases"]:
        b = np.zeros(32, np.float32)
        b[0] = pins.f32_from_bits(case["amax_bits"])
        b[5] = pins.f32_from_bits(case["x_bits"])
        b[9] = -b[5]
        blocks.append((b, case["q"]))
    zero = np.zeros(32, np.float32)
    equal = np.full(32, np.float32(0.37))
    ties = np.zeros(32, np.float32)
    ties[0] = 127.0
    ties[1:7] = [2.5, -2.5, 0.5, -0.5, 1.5, 126.5]
    x = np.concatenate([b for b, _ in blocks] + [zero, equal, -equal, ties])
    q, d = _q8_gpu(x)
    qr, dr = orc.quantize_q8(x)
    assert np.array_equal(q, qr) and np.array_equal(d.view(np.uint32), dr.view(np.uint32))
    for i, (_, want) in enumerate(blocks):
        assert q[32 * i + 5] == want and q[32 * i + 9] == -want
    n = len(blocks)
    assert np.all(q[32 * n:32 * (n + 1)] == 0) and d[n] == 0.0
    assert np.all(q[32 * (n + 1):32 * (n + 2)] == 127) and np.all(q[32 * (n + 2):32 * (n + 3)] == -127)
    assert list(q[32 * (n + 3) + 1:32 * (n + 3) + 7]) == [3, -3, 1, -1, 2, 127]


@pytest.mark.parametrize("qtype", [4, 8])
@pytest.mark.parametrize("rows,cols", [(1, 32), (5, 96), (256, 512), (37, 4096)])
def test_quantize_weights_bitexact(qtype, rows, cols):
    announce(f"quantize_weights q{qtype} {rows}x{cols}")
    rng = np.random.default_rng(101)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    if rows * cols >= 64:
        w.reshape(-1, 32)[::3] = 0.0
    q, d = qmv.qmv_quantize_weights(dev(w), qtype)
    q, d = host(q), host(d)
    if qtype == 4:
        qr, dr = orc.quantize_q4(w)
        assert np.array_equal(q.view(np.uint8), qr)
    else:
        qr, dr = orc.quantize_q8(w)
        assert np.array_equal(q, qr)
    assert np.array_equal(d.view(np.uint32), dr.view(np.uint32))


def test_quantize_determinism():
    announce("quantize determinism")
    wl = synth.WORKLOADS["llama7b_ffn_stack_q4"]
    x = synth.activation(wl, "x_down.0", 4)
    a = _q8_gpu(x)
    b = _q8_gpu(x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_quantize_empty():
    announce("quantize empty")
    x = torch.empty(0, dtype=torch.float32, device="cuda:0")
    q, d = qmv.qmv_quantize_q8(x)
    torch.cuda.synchronize()
    assert q.numel() == 0 and d.numel() == 0
