"""The five workloads at their full sizes, in the launch configuration the
bench times, against the oracle (GPU).

Weights: the GPU quantizes the seeded float32 draw with
qmv_quantize_weights, the oracle quantizes the same draw on the CPU, and
the two must agree bit for bit.  Each side then multiplies with its own
quantized weights.  Activations go through the fused kernels (M = 1) or
qmv_quantize_q8 (M > 1); the quantized activation must match the oracle's
bit for bit and every output within the tolerance, at every size (the
oracle's rows split over the host's threads)."""
import numpy as np
import pytest
import torch

from block_quantized_decode_amd import qmv, synth
from gpu_util import announce, check_close, check_gemm_all, dev, host
from oracle import oracle as orc

pytestmark = pytest.mark.gpu


def _quantize_both(qtype, w):
    wq_g, wd_g = qmv.qmv_quantize_weights(dev(w), qtype)
    if qtype == 4:
        wq, wd = orc.quantize_q4(w)
        assert np.array_equal(host(wq_g).view(np.uint8), wq), "Q4_0 weight quants differ"
    else:
        wq, wd = orc.quantize_q8(w)
        assert np.array_equal(host(wq_g), wq), "Q8_0 weight quants differ"
    assert np.array_equal(host(wd_g).view(np.uint32), wd.view(np.uint32)), "weight scales differ"
    return wq_g, wd_g, wq, wd


def _cases(names, ms=(1,)):
    out = []
    for wname in names:
        wl = synth.WORKLOADS[wname]
        for mt in wl.matrices:
            for m in ms if ms else wl.ms:
                if m in wl.ms:
                    for qt in wl.qtypes:
                        out.append((wname, mt.name, m, qt))
    return out


M1_CASES = _cases(["q8_256x512", "tinyllama_layer_q4", "llama7b_ffn_stack_q4", "qwen05b_ffn_lmhead_q8"])


@pytest.mark.parametrize("wname,mname,m,qtype", M1_CASES, ids=[f"{a}-{b}" for a, b, _, _ in M1_CASES])
def test_workload_m1_fused(wname, mname, m, qtype):
    announce(f"workload {wname} {mname} m={m} q{qtype}")
    wl = synth.WORKLOADS[wname]
    mt = wl.matrix(mname)
    w = synth.weight(wl, mname)
    wq_g, wd_g, wq, wd = _quantize_both(qtype, w)
    del w
    x = synth.activation(wl, mt.act, 1).reshape(-1)
    xq, xd = orc.quantize_q8(x)
    yref = orc.matvec(qtype, wq, wd, xq, xd)
    qo = torch.zeros(mt.cols, dtype=torch.int8, device="cuda:0")
    do = torch.zeros(mt.cols // 32, dtype=torch.float32, device="cuda:0")
    f = qmv.qmv_matvec_q4_fx if qtype == 4 else qmv.qmv_matvec_q8_fx
    y = host(f(wq_g, wd_g, dev(x), xq_out=(qo, do)))
    assert np.array_equal(host(qo), xq) and np.array_equal(host(do).view(np.uint32), xd.view(np.uint32))
    worst = check_close(qtype, y, yref, wq, wd, xq, xd, what=f"{wname}/{mname}")
    print(f"  max |err| / tol = {worst:.4f}")
    # the pre-quantized entry point on the same data
    g = qmv.qmv_matvec_q4 if qtype == 4 else qmv.qmv_matvec_q8
    y2 = host(g(wq_g, wd_g, qo, do))
    check_close(qtype, y2, yref, wq, wd, xq, xd, what=f"{wname}/{mname} pre-quantized")


# every matrix of the 8-layer stack at M = 4 (the bench's small-batch step)
GEMM_CASES = [("llama7b_ffn_stack_q4", f"{w}.{i}", 4, 4) for i in range(8) for w in ("W_up", "W_down")]
for _mn in ("W_up", "W_down"):
    for _m in (16, 64):
        for _qt in (4, 8):
            GEMM_CASES.append(("batched_ffn_q4q8", _mn, _m, _qt))


@pytest.mark.parametrize("wname,mname,m,qtype", GEMM_CASES, ids=[f"{a}-{b}-m{c}-q{d}" for a, b, c, d in GEMM_CASES])
def test_workload_gemm(wname, mname, m, qtype):
    announce(f"workload {wname} {mname} m={m} q{qtype}")
    wl = synth.WORKLOADS[wname]
    mt = wl.matrix(mname)
    w = synth.weight(wl, mname)
    wq_g, wd_g, wq, wd = _quantize_both(qtype, w)
    del w
    X = synth.activation(wl, mt.act, m)
    xq_g, xd_g = qmv.qmv_quantize_q8(dev(X))
    xq, xd = orc.quantize_q8(X)
    assert np.array_equal(host(xq_g), xq) and np.array_equal(host(xd_g).view(np.uint32), xd.view(np.uint32))
    f = qmv.qmv_gemm_q4 if qtype == 4 else qmv.qmv_gemm_q8
    Y = host(f(wq_g, wd_g, xq_g, xd_g))
    kernel = qmv.last_kernel()
    worst = check_gemm_all(qtype, Y, wq, wd, xq, xd, what=f"{wname}/{mname} m={m}")
    print(f"  {kernel}: all {m} x {mt.rows} outputs, max |err| / tol = {worst:.4f}")
