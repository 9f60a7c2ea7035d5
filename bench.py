#!/usr/bin/env python3
"""Bench of the block-quantized decode product on one MI355X.

Default workload: the Llama-7B-shaped FFN stack, Q4_0, M = 1 -- 8 layers of
(W_up 11008 x 4096, W_down 4096 x 11008), 450,887,680 weight bytes per step,
more than the 256 MB last-level cache, so every step streams its weights
from HBM.  One step = the whole path once: for each of the 16 matrices, the
fused kernel quantizes that matrix's float32 activation to Q8_0 on chip and
streams the matrix (qmv_matvec_q4_fx).

The step's 16 launches are prepared once and captured in a HIP graph; the
timed region is K graph replays.  Printed: one JSON line with the metric
(weight GB/s = quant + scale bytes per step / step time), the roofline of
the dominant kernel (every launch in the timed region is the fused
matvec: its average launch duration is the timed region's HIP-event time
per launch) and the CPU oracle timed on the same workload on the host
cores.  The same stack at M = 4 (small-batch decode, qmv_gemm_q4 on
pre-quantized activation rows) is reported under "small_batch".  The
second half of the metric, the M >= 16 product on the int8 matrix cores
(GOP/s and % of the int8 peak on the batched workload: both FFN matrices,
Q4_0 and Q8_0, M = 16 and 64), is measured the same way and reported under
"batched".  The other configurations (256 x 512 Q8_0, a TinyLlama-1.1B
layer with and without concatenated projections, the Qwen2.5-0.5B FFN and
lm_head) are timed per call and per layer under "other_workloads", and the
decode-step neighbours (rmsnorm ahead of the quantization, the FFN gate
silu(g) * u) unfused, fused into the product's launch and as the stacked
gate|up form, under "fusion".  "env" holds the per-launch floor of the smallest libqmv kernel
replayed the same way and the shader clock rocm-smi reports; the CPU
baseline also gives the oracle's single-thread rate, the host CPU model
and the oracle's compiler flags.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_I8_PEAK_TOPS = 5000.0     # MI355X dense int8 matrix peak, vendor figure
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama7b_ffn_stack_q4")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-batched", action="store_true", help="skip the M >= 16 matrix-core measurement")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the per-call timings of the other configurations (keeps kernel traces to the step)")
    ap.add_argument("--q4k-only", action="store_true",
                    help="only the K-quant super-block measurement (for profiling)")
    ap.add_argument("--q4k-shapes", default="",
                    help="with --q4k-only: comma-separated shape groups (tinyllama_layer, llama7b_ffn); default all")
    ap.add_argument("--zp-only", action="store_true",
                    help="only the 128-block zero-point format measurement (for profiling)")
    ap.add_argument("--others-only", action="store_true",
                    help="only the per-call timings of the other configurations (for profiling)")
    ap.add_argument("--batched-only", action="store_true",
                    help="only the M >= 16 matrix-core measurement (one JSON object; for profiling that path)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 256 MiB (10 times), the reference for scaling the "
                         "HBM byte counters that rocprofv3 reports for the matvec kernel")
    return ap.parse_args()


def copy_calibration():
    """A plain device-to-device copy of a known size, profiled next to the
    matvec so its FETCH_SIZE / WRITE_SIZE readings calibrate the counters."""
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 10}), flush=True)


# The sources the timed kernel (the split-K fused matvec) is compiled from:
# the kernel file and every header it includes.
TIMED_KERNEL_SOURCES = ("count.h", "device_common.h", "launch.h", "kernels_fx.hip")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_quantized_decode_amd", "csrc")
    for f in TIMED_KERNEL_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, sha: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if
    they were taken on the kernel sources as they are now; else None."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get(kernel)
    if not ent or ent.get("source_sha") != sha:
        return None
    return ent.get("bytes_per_launch")


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.zp_only or args.q4k_only or args.others_only:
        import torch
        from block_quantized_decode_amd import qmv
        torch.cuda.set_device(0)
        qmv.qmv_device_check()
        stream = torch.cuda.Stream()
        if args.others_only:
            res = other_workloads_bench(stream)
        elif args.zp_only:
            res = zp_bench(stream)
        else:
            res = q4k_bench(stream, args.q4k_shapes.split(",") if args.q4k_shapes else None)
        print(json.dumps(res), flush=True)
        return
    if args.batched_only:
        import torch
        from block_quantized_decode_amd import qmv
        torch.cuda.set_device(0)
        qmv.qmv_device_check()
        stream = torch.cuda.Stream()
        ceil = ceilings_bench(stream, per_launch_bytes=28_240_896, step_bytes=16 * 28_240_896)
        print(json.dumps(batched_bench(torch.device("cuda:0"), ceil=ceil, sclk_mhz=gpu_clock_mhz())), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by weight rows across GPUs, but nothing here launches a second GPU)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_quantized_decode_amd import qmv, synth

    wl = synth.WORKLOADS[args.workload]
    assert wl.ms[0] == 1 and len(wl.qtypes) == 1, "the bench times the M = 1 fused path"
    qtype = wl.qtypes[0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    qmv.qmv_device_check()

    # ---- inputs, resident in HBM before timing starts
    t_setup = time.time()
    mats = []
    acts = {}
    for mt in wl.matrices:
        w = torch.from_numpy(synth.weight(wl, mt.name)).to(dev)
        q, d = qmv.qmv_quantize_weights(w, qtype)
        del w
        if mt.act not in acts:
            acts[mt.act] = torch.from_numpy(synth.activation(wl, mt.act, 1).reshape(-1)).to(dev)
        y = torch.zeros(mt.rows, dtype=torch.float32, device=dev)
        mats.append((mt, q, d, acts[mt.act], y))
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    setup_s = time.time() - t_setup
    fx = qmv.qmv_matvec_q4_fx if qtype == 4 else qmv.qmv_matvec_q8_fx

    weight_bytes = wl.weight_bytes(qtype)                      # q + d per step
    algo_bytes = [q.numel() + d.numel() * 4 + 4 * mt.cols + 4 * mt.rows for mt, q, d, _, _ in mats]

    # One step = every matrix of the workload once, as prepared libqmv calls
    # (arguments marshalled once), captured in a HIP graph so that the host
    # does not pace the GPU; decode serving replays such a graph per token.
    stream = torch.cuda.Stream()
    calls = [qmv.prepare_matvec_fx(qtype, q, d, x, y, stream=stream.cuda_stream) for mt, q, d, x, y in mats]
    with torch.cuda.stream(stream):
        for _ in range(max(1, args.warmup)):
            for c in calls:
                c()
    torch.cuda.synchronize()
    # the kernel variant each matrix shape runs (one per distinct shape)
    kernels = {}
    for (mt, *_r), c in zip(mats, calls):
        with torch.cuda.stream(stream):
            c()
        kernels.setdefault(qmv.last_kernel(), mt.name.split(".")[0])
    torch.cuda.synchronize()
    kernel = " + ".join(f"{k} ({v})" for k, v in kernels.items())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for c in calls:
            c()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()

    # ---- timed region: K graph replays, bracketed by synchronisation
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps

    # ---- the dominant kernel: every launch in the timed region is the fused
    # row-streaming matvec, so its average launch duration is the timed
    # region's HIP-event time over the number of launches (graph-node gaps
    # included, so it is an upper bound on the kernel-only time rocprofv3
    # reports).  Per-matrix figures: HIP events around each launch in a
    # second, eager pass (these include the event packets' own overhead).
    avg_launch_us = total_ms * 1e3 / (args.steps * len(calls))
    avg_algo_bytes = float(np.mean(algo_bytes))
    achieved_gbs = avg_algo_bytes / (avg_launch_us * 1e-6) / 1e9
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in mats]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for s_ in range(args.steps):
            for i, c in enumerate(calls):
                ev[s_][i][0].record(stream)
                c()
                ev[s_][i][1].record(stream)
    torch.cuda.synchronize()
    launch_ms = np.array([[a.elapsed_time(b) for a, b in row] for row in ev])   # [steps, matrices]
    per_matrix_us = {}
    for i, (mt, *_rest) in enumerate(mats):
        key = mt.name.split(".")[0]
        per_matrix_us.setdefault(key, []).append(float(launch_ms[:, i].mean()) * 1e3)

    value = weight_bytes / (ms_per_step * 1e-3) / 1e9
    sha = kernel_source_sha()
    traffic = load_traffic(kernel, sha)
    ceil = ceilings_bench(stream, per_launch_bytes=int(avg_algo_bytes), step_bytes=int(sum(algo_bytes)))

    # ---- the same stack at M = 4 (small-batch decode): 4 activation rows per
    # matrix, quantized once with qmv_quantize_q8, one qmv_gemm per matrix
    small = None
    if wl.name.startswith("llama7b") and 4 in wl.ms:
        small = small_batch_bench(wl, qtype, mats, stream, args.steps, args.warmup)

    floor_us = launch_floor(stream)
    sclk = gpu_clock_mhz()

    # ---- the other configurations: per call and per layer, cold
    others = None
    fusion = None
    zp = None
    q4k = None
    if not args.no_others:
        others = other_workloads_bench(stream)
        fusion = fusion_bench(stream)
        zp = zp_bench(stream)
        q4k = q4k_bench(stream)

    # ---- the M >= 16 path (second half of the metric), timed the same way
    batched = None
    if not args.no_batched:
        batched = batched_bench(dev, ceil=ceil, sclk_mhz=sclk)

    # ---- CPU oracle baseline on a bounded sample (and a parity spot-check)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, qtype, mats, args.cpu_seconds)

    line = {
        "metric": "M=1 matvec weight GB/s (% HBM peak)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4_0 x q8_0 -> i32 block sums, f32 accumulate" if qtype == 4 else "q8_0 x q8_0 -> i32 block sums, f32 accumulate",
        "data": "synthetic (seeded numpy draws, shapes of the named model; no trained weights)",
        "config": {
            "workload": wl.name,
            "shapes": "8 x (W_up 11008x4096, W_down 4096x11008)" if wl.name.startswith("llama7b") else
                      ", ".join(f"{mt.name} {mt.rows}x{mt.cols}" for mt in wl.matrices),
            "m": 1,
            "weight_bytes_per_step": weight_bytes,
            "launches_per_step": len(mats),
            "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
            "kernel": kernel,
            "event_timed_launch_us": {k: round(float(np.mean(v)), 3) for k, v in per_matrix_us.items()},
            "setup_s": round(setup_s, 1),
        },
        "env": {"launch_floor_us": floor_us, "gpu_sclk_mhz": sclk, "ceilings": ceil},
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "frac_of_measured_stream_ceiling": round(achieved_gbs / ceil["stream_read"]["per_launch"]["gb_s"], 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": round(avg_algo_bytes),
            "avg_launch_us": round(avg_launch_us, 3),
            "launches_timed": args.steps * len(calls),
            "kernel_source_sha": sha,
        },
        "cpu_baseline": cpu,
        "small_batch": small,
        "other_workloads": others,
        "fusion": fusion,
        "zp_b128": zp,
        "q4k_superblock": q4k,
        "batched": batched,
    }
    print(json.dumps(line), flush=True)
    if cpu is not None and not cpu.get("parity_ok", True):
        sys.exit(1)


def ceilings_bench(stream, per_launch_bytes, step_bytes):
    """What plain kernels reach on this chip, measured like the step:
      * stream_read.per_launch: 16 buffers of per_launch_bytes read in turn
        by one launch each (a graph of 16 launches, replayed), the best of
        a few grid shapes and load depths -- the ceiling of a single
        launch of that size, ramp and drain included;
      * stream_read.one_launch: step_bytes read by one launch (the plateau
        without per-launch ramp and drain);
      * mfma_i8: int8 matrix-core instructions with operands in registers,
        4 independent chains per wavefront, the best grid, per instruction
        shape (TOP/s; the vendor's dense int8 peak is 5000)."""
    import torch

    from block_quantized_decode_amd import qmv

    dev = torch.device("cuda:0")
    n16 = (per_launch_bytes + 15) // 16 * 16
    bufs = [torch.ones(n16 // 4, dtype=torch.int32, device=dev) for _ in range(16)]
    big = torch.ones((step_bytes + 15) // 16 * 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    sid = stream.cuda_stream
    per = None
    for wgs in (128, 256, 512):
        for depth in (4, 8):
            calls = [qmv.Prepared("qmv_ceiling_stream_read", [sink.data_ptr(), b.data_ptr(), n16, wgs, depth], [b])
                     for b in bufs]
            us = _graph_us(calls, stream, reps=20) / len(calls)
            if per is None or us < per["us"]:
                per = {"us": round(us, 3), "gb_s": round(n16 / (us * 1e-6) / 1e9, 1), "workgroups": wgs,
                       "depth": depth, "bytes": n16}
    one = None
    nb = big.numel() * 4
    for wgs in (512, 1024, 2048, 4096):
        calls = [qmv.Prepared("qmv_ceiling_stream_read", [sink.data_ptr(), big.data_ptr(), nb, wgs, 8], [big])]
        us = _graph_us(calls * 4, stream, reps=5) / 4
        if one is None or us < one["us"]:
            one = {"us": round(us, 2), "gb_s": round(nb / (us * 1e-6) / 1e9, 1), "workgroups": wgs, "bytes": nb}
    del bufs, big
    mfma = {}
    for shape, (nm, e, kd) in enumerate((("16x16x32", 256, 32), ("16x16x64", 256, 64), ("32x32x32", 1024, 32))):
        best = None
        for wgs in (512, 1024, 2048):
            iters = 2000 if e == 256 else 500
            calls = [qmv.Prepared("qmv_ceiling_mfma_i8", [sink.data_ptr(), shape, iters, wgs, 1, 1], [])]
            us = _graph_us(calls * 4, stream, reps=3) / 4
            tops = wgs * 16 * iters * 2 * e * kd / (us * 1e-6) / 1e12
            if best is None or tops > best["top_s"]:
                best = {"top_s": round(tops, 1), "us": round(us, 2), "workgroups": wgs}
        mfma[nm] = best
    torch.cuda.empty_cache()
    return {"stream_read": {"per_launch": per, "one_launch": one,
                            "pct_hbm_peak_per_launch": round(100.0 * per["gb_s"] / HBM_PEAK_GBS, 2),
                            "pct_hbm_peak_one_launch": round(100.0 * one["gb_s"] / HBM_PEAK_GBS, 2)},
            "mfma_i8": mfma, "mfma_i8_best_top_s": max(v["top_s"] for v in mfma.values())}


def launch_floor(stream, n=16, reps=50):
    """Per-launch time of the smallest libqmv kernel (Q8_0 quantization of
    one 32-element block), n launches per HIP graph: the floor under any
    one launch of the step, replayed the same way."""
    import torch

    from block_quantized_decode_amd import qmv

    x = torch.ones(32, dtype=torch.float32, device="cuda:0")
    q = torch.empty(32, dtype=torch.int8, device="cuda:0")
    d = torch.empty(1, dtype=torch.float32, device="cuda:0")
    with torch.cuda.stream(stream):
        qmv.qmv_quantize_q8(x, q, d)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(n):
            qmv.qmv_quantize_q8(x, q, d)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(reps):
            g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return round(t0.elapsed_time(t1) * 1e3 / (reps * n), 3)


def gpu_clock_mhz():
    """Current shader clock of cuda:0 from its sysfs DPM table (the level
    marked '*' in pp_dpm_sclk), or None where that file is not readable.
    A plain file read: no subprocess is started from this GPU process."""
    import glob
    import re

    import torch

    try:
        p = torch.cuda.get_device_properties(0)
        bus = "%04x:%02x:%02x" % (p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
    except (AttributeError, AssertionError, RuntimeError):
        return None
    for dev_dir in glob.glob("/sys/class/drm/card*/device"):
        try:
            if not os.path.realpath(dev_dir).rsplit("/", 1)[-1].startswith(bus):
                continue
            with open(os.path.join(dev_dir, "pp_dpm_sclk")) as f:
                for ln in f:
                    if "*" in ln:
                        m = re.search(r"(\d+)\s*Mhz", ln, re.I)
                        return int(m.group(1)) if m else None
        except OSError:
            return None
    return None


def _graph_us(calls, stream, reps=20):
    """Microseconds per replay of a HIP graph of `calls` (after warm-up)."""
    import torch

    with torch.cuda.stream(stream):
        for c in calls:
            c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in calls:
            c()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(reps):
            g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / reps


def other_workloads_bench(stream):
    """The other configurations, per call and per layer, through the fused
    entry point (M = 1, float32 activation), timed like the step: graphs of
    prepared calls.  Weights are random normal draws quantized on the GPU.
    Every timed graph cycles through copies of its matrices totalling more
    than 600 MB (at least 4), more than the 256 MB last-level cache, so each
    call streams from HBM: per matrix, the copies of that matrix alone; per
    layer, whole copies of the layer.  The 256 x 512 parity matrix (147 KB)
    is timed warm.  The TinyLlama layer is also timed with the projections
    concatenated as the forward pass writes them (W_q|W_k|W_v 2560 x 2048,
    W_gate|W_up 11264 x 2048): 4 launches per layer instead of 7."""
    import torch

    from block_quantized_decode_amd import qmv, synth

    dev = torch.device("cuda:0")
    torch.manual_seed(5)
    out = {}
    cold = 600 << 20

    def quantized(rows, cols, qtype):
        w = torch.randn(rows, cols, device=dev) * 0.02
        q, d = qmv.qmv_quantize_weights(w, qtype)
        del w
        return q, d

    def nbytes(rows, cols, qtype):
        return rows * cols // 32 * ((16 if qtype == 4 else 32) + 4)

    def copies_for(total):
        return max(4, -(-cold // total))

    def calls_for(mats, qtype, copies):
        """Per copy: [(name, prepared call, weight bytes)] in matrix order."""
        xs = {}
        res = []
        for c in range(copies):
            row = []
            for name, rows, cols, act in mats:
                q, d = quantized(rows, cols, qtype)
                if act not in xs:
                    xs[act] = torch.randn(cols, device=dev)
                y = torch.zeros(rows, device=dev)
                row.append((name, qmv.prepare_matvec_fx(qtype, q, d, xs[act], y, stream=stream.cuda_stream),
                            q.numel() + d.numel() * 4))
            res.append(row)
        return res

    def per_matrix(mats, qtype):
        """us per call and weight GB/s of each matrix, over its own cold copies."""
        us, gbs = {}, {}
        for m in mats:
            n = copies_for(nbytes(m[1], m[2], qtype))
            cs = calls_for([m], qtype, n)
            t = _graph_us([row[0][1] for row in cs], stream) / n
            us[m[0]] = round(t, 3)
            gbs[m[0]] = round(cs[0][0][2] / (t * 1e-6) / 1e9, 1)
            del cs
            torch.cuda.empty_cache()
        return us, gbs

    # 256 x 512 Q8_0, warm
    wl = synth.WORKLOADS["q8_256x512"]
    cs = calls_for([(m.name, m.rows, m.cols, m.act) for m in wl.matrices], 8, 1)
    us = _graph_us([cs[0][0][1]] * 16, stream) / 16
    out[wl.name] = {"us_per_call": round(us, 3), "weight_gb_s": round(cs[0][0][2] / (us * 1e-6) / 1e9, 1),
                    "note": "warm (147 KB stays in cache)", "kernel": qmv.last_kernel()}

    # TinyLlama layer, Q4_0: per matrix, per layer, and concatenated
    wl = synth.WORKLOADS["tinyllama_layer_q4"]
    mats = [(m.name, m.rows, m.cols, m.act) for m in wl.matrices]
    per, _ = per_matrix(mats, 4)
    lbytes = sum(nbytes(r, c, 4) for _, r, c, _ in mats)
    copies = copies_for(lbytes)
    cs = calls_for(mats, 4, copies)
    layer_us = _graph_us([call for row in cs for _, call, _ in row], stream) / copies
    del cs
    torch.cuda.empty_cache()
    cat = [("W_qkv", 2560, 2048, "x_attn"), ("W_o", 2048, 2048, "x_o"), ("W_gate_up", 11264, 2048, "x_ffn"),
           ("W_down", 2048, 5632, "x_down")]
    cs = calls_for(cat, 4, copies)
    cat_us = _graph_us([call for row in cs for _, call, _ in row], stream) / copies
    del cs
    torch.cuda.empty_cache()
    out[wl.name] = {"per_matrix_us": per, "layer_us": round(layer_us, 3), "layer_launches": len(mats),
                    "layer_weight_gb_s": round(lbytes / (layer_us * 1e-6) / 1e9, 1),
                    "layer_concat_us": round(cat_us, 3), "layer_concat_launches": len(cat),
                    "layer_concat_weight_gb_s": round(lbytes / (cat_us * 1e-6) / 1e9, 1),
                    "layer_copies": copies}

    # Qwen2.5-0.5B FFN + lm_head, Q8_0
    wl = synth.WORKLOADS["qwen05b_ffn_lmhead_q8"]
    mats = [(m.name, m.rows, m.cols, m.act) for m in wl.matrices]
    per, gbs = per_matrix(mats, 8)
    ffn = mats[:3]
    fbytes = sum(nbytes(r, c, 8) for _, r, c, _ in ffn)
    copies = copies_for(fbytes)
    cs = calls_for(ffn, 8, copies)
    ffn_us = _graph_us([call for row in cs for _, call, _ in row], stream) / copies
    del cs
    torch.cuda.empty_cache()
    out[wl.name] = {"per_matrix_us": per, "per_matrix_weight_gb_s": gbs, "ffn_us": round(ffn_us, 3),
                    "lm_head_pct_hbm_peak": round(100.0 * gbs["lm_head"] / HBM_PEAK_GBS, 2), "ffn_copies": copies}
    return out

def zp_bench(stream):
    """The exported-model format (128-element blocks with a zero point,
    qmv_matvec_zp_fx, the activation quantized in the launch), 8 and 4 bits,
    on the Qwen2.5-0.5B FFN and lm_head shapes of the ONNX page's real
    export and on the Llama-7B FFN matrices.  Codes, scales and zero points
    are uniform random draws on the GPU (seeded); each matrix is rotated
    over copies totalling more than 600 MB, so every launch streams from
    HBM, and timed as a graph of prepared calls.  Weight bytes = codes +
    scales + zero points."""
    import torch

    from block_quantized_decode_amd import qmv

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    shapes = {
        "qwen05b_ffn_lmhead": [("W_gate", 4864, 896), ("W_up", 4864, 896), ("W_down", 896, 4864),
                               ("lm_head", 151936, 896)],
        "llama7b_ffn": [("W_up", 11008, 4096), ("W_down", 4096, 11008)],
    }
    out = {}
    for bits in (8, 4):
        for wname, mats in shapes.items():
            per = {}
            for name, rows, cols in mats:
                nb = cols // 128
                rb = cols if bits == 8 else cols // 2
                wbytes = rows * rb + rows * nb * 5
                copies = max(2, (600 << 20) // wbytes + 1)
                x = torch.randn(cols, device=dev, generator=gen)
                calls = []
                for _ in range(copies):
                    q = torch.randint(0, 256, (rows, rb), dtype=torch.uint8, device=dev, generator=gen)
                    d = torch.rand(rows, nb, device=dev, generator=gen) * 0.01 + 0.001
                    zp = torch.randint(0, 1 << bits, (rows, nb), dtype=torch.uint8, device=dev, generator=gen)
                    y = torch.zeros(rows, device=dev)
                    calls.append(qmv.prepare_matvec_zp_fx(q, d, zp, bits, x, y, stream=stream.cuda_stream))
                us = _graph_us(calls, stream) / len(calls)
                gbs = wbytes / (us * 1e-6) / 1e9
                per[name] = {"shape": f"{rows}x{cols}", "us": round(us, 3), "weight_gb_s": round(gbs, 1),
                             "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2), "kernel": qmv.last_kernel(),
                             "copies": copies}
                del calls
                torch.cuda.empty_cache()
            out[f"{wname}_int{bits}_b128"] = per
    return out


def q4k_bench(stream, groups=None):
    """The K-quant super-block format (qmv_matvec_q4k_fx, the activation
    quantized in the launch) on the shapes of the SKaiNET page's model
    (TinyLlama-1.1B, every matrix of a layer) and on the Llama-7B FFN
    matrices.  Nibbles, sub-block scales and minima (0..63) and super-block
    scales are seeded random draws on the GPU; each matrix is rotated over
    copies totalling more than 600 MB, so every launch streams from HBM.
    Weight bytes = nibbles + scales + minima + d + dmin (0.59375 B per
    element)."""
    import torch

    from block_quantized_decode_amd import qmv

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    shapes = {
        "tinyllama_layer": [("W_q", 2048, 2048), ("W_k", 256, 2048), ("W_v", 256, 2048), ("W_o", 2048, 2048),
                            ("W_gate", 5632, 2048), ("W_up", 5632, 2048), ("W_down", 2048, 5632)],
        "llama7b_ffn": [("W_up", 11008, 4096), ("W_down", 4096, 11008)],
    }
    if groups:
        shapes = {k: v for k, v in shapes.items() if k in groups}
    out = {}
    for wname, mats in shapes.items():
        per = {}
        for name, rows, cols in mats:
            wbytes = rows * (cols // 2 + 2 * (cols // 32) + 8 * (cols // 256))
            copies = max(2, (600 << 20) // wbytes + 1)
            x = torch.randn(cols, device=dev, generator=gen)
            calls = []
            for _ in range(copies):
                q = torch.randint(0, 256, (rows, cols // 2), dtype=torch.uint8, device=dev, generator=gen)
                sc = torch.randint(0, 64, (rows, cols // 32), dtype=torch.uint8, device=dev, generator=gen)
                mn = torch.randint(0, 64, (rows, cols // 32), dtype=torch.uint8, device=dev, generator=gen)
                d = torch.rand(rows, cols // 256, device=dev, generator=gen) * 1e-3
                dmin = torch.rand(rows, cols // 256, device=dev, generator=gen) * 1e-3
                y = torch.zeros(rows, device=dev)
                calls.append(qmv.prepare_matvec_q4k_fx(q, sc, mn, d, dmin, x, y, stream=stream.cuda_stream))
            us = _graph_us(calls, stream) / len(calls)
            gbs = wbytes / (us * 1e-6) / 1e9
            per[name] = {"shape": f"{rows}x{cols}", "us": round(us, 3), "weight_gb_s": round(gbs, 1),
                         "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2), "kernel": qmv.last_kernel(),
                         "copies": copies}
            del calls
            torch.cuda.empty_cache()
        out[wname] = per
    return out


def fusion_bench(stream):
    """The decode-step neighbours (rmsnorm ahead of a quantization, the FFN
    gate silu(g) * u) with the product, timed like the step (graphs of
    prepared calls, weights rotated over copies beyond the 256 MB cache),
    in three forms:
      * unfused: each neighbour a launch of its own (qmv_rmsnorm,
        qmv_silu_mul) ahead of the plain fused product;
      * fused: the neighbour inside the product's launch (_fx_rmsnorm,
        _fx_silu_mul);
      * swiglu: rmsnorm + stacked gate|up + gate in one launch
        (_fx_swiglu), the down projection a plain fused product of the
        gate's output;
    against "plain": the same products with no neighbour at all (the
    layer_concat figure of other_workloads).  For a TinyLlama-1.1B layer's
    matrix path (Q|K|V 2560 x 2048, W_o, gate|up 11264 x 2048, down 2048 x
    5632) and single Llama-7B FFN launches (W_up 11008 x 4096 with rmsnorm,
    W_down 4096 x 11008 with the gate, stacked gate|up 22016 x 4096)."""
    import torch

    from block_quantized_decode_amd import qmv

    dev = torch.device("cuda:0")
    torch.manual_seed(6)

    def quantized(rows, cols, qtype=4):
        w = torch.randn(rows, cols, device=dev) * 0.02
        q, d = qmv.qmv_quantize_weights(w, qtype)
        del w
        return q, d

    out = {}
    sid = stream.cuda_stream
    # TinyLlama layer
    copies = 20
    H, F = 2048, 5632
    x_attn = torch.randn(H, device=dev)
    x_o = torch.randn(H, device=dev)
    x_ffn = torch.randn(H, device=dev)
    n_attn = 1.0 + 0.1 * torch.randn(H, device=dev)
    n_ffn = 1.0 + 0.1 * torch.randn(H, device=dev)
    h_attn = torch.zeros(H, device=dev)
    h_ffn = torch.zeros(H, device=dev)
    a_ffn = torch.zeros(F, device=dev)
    forms = {"plain": [], "unfused": [], "fused": [], "swiglu": []}
    keep = []
    for _ in range(copies):
        qkv, wo, gu, dn = quantized(2560, H), quantized(H, H), quantized(2 * F, H), quantized(H, F)
        y_qkv = torch.zeros(2560, device=dev)
        y_o = torch.zeros(H, device=dev)
        y_gu = torch.randn(2 * F, device=dev)
        y_dn = torch.zeros(H, device=dev)
        forms["plain"] += [qmv.prepare_matvec_fx(4, *qkv, x_attn, y_qkv, stream=sid),
                           qmv.prepare_matvec_fx(4, *wo, x_o, y_o, stream=sid),
                           qmv.prepare_matvec_fx(4, *gu, x_ffn, y_gu, stream=sid),
                           qmv.prepare_matvec_fx(4, *dn, y_gu[:F], y_dn, stream=sid)]
        forms["unfused"] += [qmv.prepare_rmsnorm(x_attn, n_attn, 1e-5, h_attn, stream=sid),
                             qmv.prepare_matvec_fx(4, *qkv, h_attn, y_qkv, stream=sid),
                             qmv.prepare_matvec_fx(4, *wo, x_o, y_o, stream=sid),
                             qmv.prepare_rmsnorm(x_ffn, n_ffn, 1e-5, h_ffn, stream=sid),
                             qmv.prepare_matvec_fx(4, *gu, h_ffn, y_gu, stream=sid),
                             qmv.prepare_silu_mul(y_gu[:F], y_gu[F:], a_ffn, stream=sid),
                             qmv.prepare_matvec_fx(4, *dn, a_ffn, y_dn, stream=sid)]
        forms["fused"] += [qmv.prepare_matvec_fx_rmsnorm(4, *qkv, x_attn, n_attn, 1e-5, y_qkv, stream=sid),
                           qmv.prepare_matvec_fx(4, *wo, x_o, y_o, stream=sid),
                           qmv.prepare_matvec_fx_rmsnorm(4, *gu, x_ffn, n_ffn, 1e-5, y_gu, stream=sid),
                           qmv.prepare_matvec_fx_silu_mul(4, *dn, y_gu[:F], y_gu[F:], y_dn, stream=sid)]
        forms["swiglu"] += [qmv.prepare_matvec_fx_rmsnorm(4, *qkv, x_attn, n_attn, 1e-5, y_qkv, stream=sid),
                            qmv.prepare_matvec_fx(4, *wo, x_o, y_o, stream=sid),
                            qmv.prepare_matvec_fx_swiglu(4, *gu, x_ffn, a_ffn, y_gu, w_norm=n_ffn, eps=1e-5,
                                                         stream=sid),
                            qmv.prepare_matvec_fx(4, *dn, a_ffn, y_dn, stream=sid)]
        keep.append((qkv, wo, gu, dn, y_qkv, y_o, y_gu, y_dn))
    lay = {k: round(_graph_us(v, stream) / copies, 3) for k, v in forms.items()}
    lay["launches"] = {"plain": 4, "unfused": 7, "fused": 4, "swiglu": 4}
    lay["copies"] = copies
    out["tinyllama_layer_q4_us"] = lay
    del keep, forms
    torch.cuda.empty_cache()
    # Llama-7B FFN launches
    copies = 8
    res = {}
    for name, rows, cols, form in (("W_up+rmsnorm", 11008, 4096, "rms"), ("W_down+silu_mul", 4096, 11008, "silu"),
                                   ("W_gate|W_up+rmsnorm+gate", 22016, 4096, "swiglu")):
        x = torch.randn(cols, device=dev)
        x2 = 1.0 + 0.1 * torch.randn(cols, device=dev)
        hbuf = torch.zeros(cols, device=dev)
        abuf = torch.zeros(rows // 2, device=dev)
        calls = {"plain": [], "unfused": [], "fused": []}
        keep = []
        for _ in range(copies):
            q, d = quantized(rows, cols)
            y = torch.zeros(rows, device=dev)
            calls["plain"].append(qmv.prepare_matvec_fx(4, q, d, x, y, stream=sid))
            if form == "rms":
                calls["unfused"] += [qmv.prepare_rmsnorm(x, x2, 1e-5, hbuf, stream=sid),
                                     qmv.prepare_matvec_fx(4, q, d, hbuf, y, stream=sid)]
                calls["fused"].append(qmv.prepare_matvec_fx_rmsnorm(4, q, d, x, x2, 1e-5, y, stream=sid))
            elif form == "silu":
                calls["unfused"] += [qmv.prepare_silu_mul(x, x2, hbuf, stream=sid),
                                     qmv.prepare_matvec_fx(4, q, d, hbuf, y, stream=sid)]
                calls["fused"].append(qmv.prepare_matvec_fx_silu_mul(4, q, d, x, x2, y, stream=sid))
            else:
                F7 = rows // 2
                calls["unfused"] += [qmv.prepare_rmsnorm(x, x2, 1e-5, hbuf, stream=sid),
                                     qmv.prepare_matvec_fx(4, q, d, hbuf, y, stream=sid),
                                     qmv.prepare_silu_mul(y[:F7], y[F7:], abuf, stream=sid)]
                calls["fused"].append(qmv.prepare_matvec_fx_swiglu(4, q, d, x, abuf, y, w_norm=x2, eps=1e-5,
                                                                   stream=sid))
            keep.append((q, d, y))
        res[name] = {k: round(_graph_us(v, stream) / copies, 3) for k, v in calls.items()}
        del keep, calls
        torch.cuda.empty_cache()
    out["llama7b_ffn_q4_us"] = res
    out["launch_floor_us"] = launch_floor(stream)
    return out

def small_batch_bench(wl, qtype, mats, stream, steps, warmup):
    """The workload's stack at M = 4 activation rows: weight bytes per step
    over the step time of a graph of one qmv_gemm per matrix (the weights of
    the M = 1 step, already resident)."""
    import torch

    from block_quantized_decode_amd import qmv, synth

    m = 4
    calls, keep = [], []
    xs = {}
    for mt, q, d, _x, _y in mats:
        if mt.act not in xs:
            x = torch.from_numpy(synth.activation(wl, mt.act, m)).to(q.device)
            xs[mt.act] = qmv.qmv_quantize_q8(x)
        xq, xd = xs[mt.act]
        Y = torch.zeros((m, mt.rows), dtype=torch.float32, device=q.device)
        calls.append(qmv.prepare_gemm(qtype, q, d, xq, xd, Y, stream=stream.cuda_stream))
        keep.append(Y)
    with torch.cuda.stream(stream):
        for c in calls:
            c()
    torch.cuda.synchronize()
    kernel = qmv.last_kernel()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for c in calls:
            c()
    for _ in range(max(1, warmup)):
        graph.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(steps):
            graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    wbytes = wl.weight_bytes(qtype)
    ops = sum(2 * m * mt.rows * mt.cols for mt, *_ in mats)
    return {"m": m, "ms_per_step": round(ms, 5), "weight_gb_s": round(wbytes / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100.0 * wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "gop_s": round(ops / (ms * 1e-3) / 1e9, 1), "launches_per_step": len(calls), "kernel": kernel}


def batched_bench(dev, name="batched_ffn_q4q8", replays=5, ceil=None, sclk_mhz=None):
    """The M >= 16 product (qmv_gemm_q4 / _q8, the int8 matrix-core kernel) on
    the batched workload: both matrices, both weight formats, M = 16 and 64.
    Weights are quantized on the GPU from the seeded float32 draw, then
    copied so that the launches of one graph cycle through more than twice
    the 256 MB last-level cache (every launch streams its weights from HBM);
    activations are quantized with qmv_quantize_q8.  Each case is a graph of
    2 x copies launches replayed `replays` times between HIP events on the
    launch stream.  GOP/s counts 2 M N K operations per launch.

    Each case is also timed warm: the same weight copy every launch (28 or
    51 MB, resident in the 256 MB last-level cache after the first), which
    takes HBM out of the way and shows the matrix-core and VALU side.  The
    rooflines next to each figure:
      * cold: min(int8 peak, 2 M ops per weight byte x HBM bandwidth), with
        the vendor figures (hbm_cap_*) and with the measured ceilings
        (measured_cold_cap_*: the best int8 matrix-core loop and the
        per-launch streaming read of env.ceilings);
      * warm: min(measured int8 loop, the fp32 epilogue) -- the kernel
        spends E non-packed VALU operations per output and block against
        the block's 64 int8 operations, and the VALU does 64 lanes x 256
        compute units per clock, so the epilogue caps the rate at
        64 / E x 64 x 256 x clock.  E = 3 (convert, scale product, fused
        multiply-add) for 17 .. 64 rows; E = 2 for up to 16 rows, where the
        scale products come from the matrix core."""
    import torch

    from block_quantized_decode_amd import qmv, synth

    wl = synth.WORKLOADS[name]
    stream = torch.cuda.Stream()
    cases = []
    for mt in wl.matrices:
        w = torch.from_numpy(synth.weight(wl, mt.name)).to(dev)
        for qtype in wl.qtypes:
            q0, d0 = qmv.qmv_quantize_weights(w, qtype)
            wbytes = q0.numel() + 4 * d0.numel()
            ncopy = max(2, (600 << 20) // wbytes + 1)
            copies = [(q0, d0)] + [(q0.clone(), d0.clone()) for _ in range(ncopy - 1)]
            # the same copies in the pack-once layout (qmv_pack_weights, once, untimed)
            packed = [qmv.qmv_pack_weights(q, d, qtype) for q, d in copies]
            torch.cuda.synchronize()
            for m in wl.ms:
                x = torch.from_numpy(synth.activation(wl, mt.act, m)).to(dev)
                xq, xd = qmv.qmv_quantize_q8(x)
                y = torch.zeros((m, mt.rows), dtype=torch.float32, device=dev)
                with torch.cuda.stream(stream):
                    calls = [qmv.prepare_gemm(qtype, q, d, xq, xd, y, stream=stream.cuda_stream) for q, d in copies]
                    for c in calls:
                        c()
                torch.cuda.synchronize()
                kernel = qmv.last_kernel()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=stream):
                    for _ in range(2):
                        for c in calls:
                            c()
                with torch.cuda.stream(stream):
                    graph.replay()
                torch.cuda.synchronize()
                t0 = torch.cuda.Event(enable_timing=True)
                t1 = torch.cuda.Event(enable_timing=True)
                with torch.cuda.stream(stream):
                    t0.record(stream)
                    for _ in range(replays):
                        graph.replay()
                    t1.record(stream)
                torch.cuda.synchronize()
                us = t0.elapsed_time(t1) * 1e3 / (replays * 2 * len(calls))
                gops = 2.0 * m * mt.rows * mt.cols / (us * 1e-6) / 1e9
                # ceiling from HBM alone: 2 m operations per weight against its
                # bytes (0.625 B for Q4_0, 1.125 B for Q8_0), at the vendor 8 TB/s
                hbm_cap = min(MFMA_I8_PEAK_TOPS * 1e3, 2.0 * m * (mt.rows * mt.cols) / wbytes * HBM_PEAK_GBS)
                case = {"qtype": f"q{qtype}_0", "matrix": mt.name, "shape": f"{mt.rows}x{mt.cols}", "m": m,
                        "us_per_launch": round(us, 2), "gop_s": round(gops, 1),
                        "pct_int8_peak": round(100.0 * gops / (MFMA_I8_PEAK_TOPS * 1e3), 2),
                        "hbm_cap_pct_int8_peak": round(100.0 * hbm_cap / (MFMA_I8_PEAK_TOPS * 1e3), 1),
                        "weight_gb_s": round(wbytes / (us * 1e-6) / 1e9, 1), "kernel": kernel}
                # warm: one weight copy, resident in the last-level cache
                wus = _graph_us([calls[0]] * (2 * len(calls)), stream, reps=replays) / (2 * len(calls))
                wgops = 2.0 * m * mt.rows * mt.cols / (wus * 1e-6) / 1e9
                case.update({"warm_us_per_launch": round(wus, 2), "warm_gop_s": round(wgops, 1),
                             "warm_pct_int8_peak": round(100.0 * wgops / (MFMA_I8_PEAK_TOPS * 1e3), 2)})
                clock = (sclk_mhz or 2400) * 1e6
                epi_valu = 2.0 if m <= 16 else 3.0
                epi_cap = 64.0 / epi_valu * 64 * 256 * clock / 1e9   # GOP/s
                case["epilogue_cap_gop_s"] = round(epi_cap, 1)
                if ceil is not None:
                    mfma = ceil["mfma_i8_best_top_s"] * 1e3
                    bw = ceil["stream_read"]["per_launch"]["gb_s"]
                    cold_cap = min(mfma, 2.0 * m * (mt.rows * mt.cols) / wbytes * bw)
                    warm_cap = min(mfma, epi_cap)
                    case.update({"measured_cold_cap_gop_s": round(cold_cap, 1),
                                 "pct_of_measured_cold_cap": round(100.0 * gops / cold_cap, 1),
                                 "measured_warm_cap_gop_s": round(warm_cap, 1),
                                 "warm_pct_of_measured_warm_cap": round(100.0 * wgops / warm_cap, 1)})
                cases.append(case)
                del graph, calls
                pcalls = [qmv.prepare_gemm_packed(P, xq, xd, y, stream=stream.cuda_stream) for P in packed]
                pus = _graph_us(pcalls + pcalls, stream, reps=replays) / (2 * len(pcalls))
                pgops = 2.0 * m * mt.rows * mt.cols / (pus * 1e-6) / 1e9
                cases[-1].update({"packed_us_per_launch": round(pus, 2), "packed_gop_s": round(pgops, 1),
                                  "packed_pct_int8_peak": round(100.0 * pgops / (MFMA_I8_PEAK_TOPS * 1e3), 2),
                                  "packed_kernel": qmv.last_kernel()})
                del pcalls
            del copies, packed, q0, d0
            torch.cuda.empty_cache()
        del w
    best = max(cases, key=lambda c: c["gop_s"])
    best_p = max(cases, key=lambda c: c["packed_gop_s"])
    return {
        "metric": "M>=16 int8 GOP/s (% MFMA peak)",
        "workload": name,
        "best_gop_s": best["gop_s"],
        "best_pct_int8_peak": best["pct_int8_peak"],
        "best_case": f"{best['qtype']} {best['matrix']} {best['shape']} M={best['m']}",
        "best_packed_gop_s": best_p["packed_gop_s"],
        "best_packed_case": f"{best_p['qtype']} {best_p['matrix']} {best_p['shape']} M={best_p['m']}",
        "packed_note": "packed_*: the same product on weights re-laid once by qmv_pack_weights (qmv_gemm_*_packed)",
        "bound_note": "cold: HBM-bound for M <= 64: 2M ops per weight element against 0.625 B (Q4_0) or 1.125 B "
                      "(Q8_0) stays below the chip's 625 op/B ridge (hbm_cap_pct_int8_peak per case; "
                      "measured_cold_cap_gop_s with the measured stream and matrix-core ceilings); warm: the fp32 "
                      "per-block epilogue (3 VALU per output per block against 64 int8 ops, 2 for up to 16 rows, "
                      "epilogue_cap_gop_s) caps every case at ~17% (~25% for up to 16 rows) of the int8 peak",
        "best_warm_gop_s": max(c["warm_gop_s"] for c in cases),
        "best_warm_pct_int8_peak": max(c["warm_pct_int8_peak"] for c in cases),
        "cases": cases,
    }


def cpu_baseline(wl, qtype, mats, target_s):
    """Time the CPU oracle (plain C, as committed) on the same workload: the
    oracle quantizes each matrix's activation and multiplies all matrices of
    the step, rows split over the host cores by the oracle's own row-range
    contract (ctypes drops the GIL inside each call).  Whole steps are
    repeated until about target_s seconds have passed.  The GPU outputs of
    the last timed GPU step are checked against the oracle's within the
    tolerance on every row."""
    import concurrent.futures as cf

    import numpy as np

    from block_quantized_decode_amd import synth
    from oracle import oracle as orc

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))
    prepared = []
    xs = {}
    for mt, q, d, x, y in mats:
        w = synth.weight(wl, mt.name)
        wq, wd = (orc.quantize_q4(w) if qtype == 4 else orc.quantize_q8(w))
        del w
        if mt.act not in xs:
            xs[mt.act] = synth.activation(wl, mt.act, 1).reshape(-1)
        prepared.append((mt, wq, wd, xs[mt.act], y.cpu().numpy(), np.zeros(mt.rows, np.float32)))

    pool = cf.ThreadPoolExecutor(cores)

    def oracle_step():
        for mt, wq, wd, xh, _, out in prepared:
            xq, xd = orc.quantize_q8(xh)
            bounds = np.linspace(0, mt.rows, cores + 1).astype(int)
            list(pool.map(lambda i: orc.matvec(qtype, wq, wd, xq, xd, int(bounds[i]), int(bounds[i + 1]), y=out),
                          range(cores)))

    passes = 0
    t = time.perf_counter()
    while True:
        oracle_step()
        passes += 1
        el = time.perf_counter() - t
        if el >= target_s:
            break
    pool.shutdown()
    # the same step on one thread (rows [0, rows) per call)
    t1 = time.perf_counter()
    for mt, wq, wd, xh, _, out in prepared:
        xq, xd = orc.quantize_q8(xh)
        orc.matvec(qtype, wq, wd, xq, xd, 0, mt.rows, y=out)
    el1 = time.perf_counter() - t1
    parity_ok = True
    worst = 0.0
    for mt, wq, wd, xh, ygpu, out in prepared:
        xq, xd = orc.quantize_q8(xh)
        tol = orc.tolerance(qtype, wq, wd, xq, xd)
        err = np.abs(ygpu.astype(np.float64) - out.astype(np.float64))
        worst = max(worst, float((err / tol).max()))
        parity_ok &= bool(np.all(err <= tol))
    wbytes = wl.weight_bytes(qtype)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": round(wbytes * passes / el / 1e9, 3),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "single_thread_gb_s": round(wbytes / el1 / 1e9, 3),
        "cpu_model": cpu_model,
        "oracle_cflags": " ".join(["gcc", *orc.CFLAGS]),
        "sample": f"the full step ({len(prepared)} matrices, {wbytes} weight bytes, activation quantization "
                  f"included) repeated {passes} times in {el:.1f} s, rows split over {cores} threads; "
                  f"once more on one thread in {el1:.1f} s",
        "parity_ok": parity_ok,
        "parity_max_err_over_tol": round(worst, 4),
    }


if __name__ == "__main__":
    main()
