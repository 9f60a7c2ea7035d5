"""The two measurement kernels the bench divides by (GPU): the streaming
read must touch every word of its buffer (the XOR of the per-workgroup
results equals the XOR of all 32-bit words), and the int8 matrix-core loop
must run every instruction (each result element ends at iters * kdepth *
a * b, so the per-wavefront sums have a closed form)."""
import numpy as np
import pytest
import torch

from block_quantized_decode_amd import qmv
from gpu_util import announce, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,wgs,depth", [(16, 1, 4), (1 << 20, 7, 4), ((1 << 22) + 48, 256, 8), (4096, 300, 8)])
def test_stream_read_xor(nbytes, wgs, depth):
    announce(f"ceiling stream read {nbytes} B, {wgs} workgroups, depth {depth}")
    rng = np.random.default_rng(nbytes + wgs)
    words = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to("cuda:0")
    sink = torch.zeros(wgs, dtype=torch.int32, device="cuda:0")
    qmv.qmv_ceiling_stream_read(buf, sink, wgs, depth)
    got = np.bitwise_xor.reduce(host(sink).view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


@pytest.mark.parametrize("shape,kdepth,elems", [(0, 32, 256), (1, 64, 256), (2, 32, 1024)])
@pytest.mark.parametrize("a,b", [(1, 1), (-3, 5), (127, -127)])
def test_mfma_loop_closed_form(shape, kdepth, elems, a, b):
    announce(f"ceiling mfma shape {shape} a={a} b={b}")
    iters, wgs = 37, 5
    sink = torch.zeros(4 * wgs, dtype=torch.int32, device="cuda:0")
    qmv.qmv_ceiling_mfma_i8(sink, shape, iters, wgs, a, b)
    want = (4 * elems * iters * kdepth * a * b) % (1 << 32)
    assert np.all(host(sink).view(np.uint32) == np.uint32(want))
