"""Seeded synthetic inputs for the block-quantized decode product.

This module only draws random numbers and arranges them in the shapes of
the workloads; it performs none of the method's arithmetic (no
quantization, no dot products).  Both the HIP path and the CPU oracle take
their inputs from here.

Recipe (each tensor, and each 4 Mi-element chunk of it, has its own
generator, so any one tensor can be drawn without drawing the others and
the chunks can be filled on several threads with the same result):
  * generator of chunk c = numpy PCG64 seeded by SeedSequence(entropy =
    workload seed, spawn_key = (kind, index, m, c)), kind 0 for weights, 1
    for activations, index = the tensor's position in the workload's list,
    m = activation rows (0 for weights);
  * values = standard_normal(float32) * sigma (sigma 0.02 for weights, 1.0
    for activations), chunk c covering flat elements [c * 2^22, (c+1) * 2^22);
  * activation outliers (Llama-7B FFN stack): exactly round(0.01 * m * K)
    distinct elements, drawn without replacement by the generator of chunk
    id 2^31 - 1, are multiplied by 20;
  * all-zero weight blocks (Qwen2.5-0.5B shapes): exactly
    round(0.01 * rows * K / 32) distinct 32-element blocks, drawn without
    replacement by the generator of chunk id 2^31 - 1, are set to 0 before
    quantization.

The shapes follow the model dimensions the pages quote for decode: a
TinyLlama-1.1B layer, a Llama-7B FFN stack (1 x 4096 x 11008 products), a
Qwen2.5-0.5B FFN plus lm_head.  Trained weights are not used anywhere: the
models are stand-ins by shape only.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

QK = 32


@dataclass(frozen=True)
class Matrix:
    name: str
    rows: int          # N (output features)
    cols: int          # K (input features), multiple of 32
    act: str           # activation tensor that multiplies it


@dataclass
class Workload:
    name: str
    seed: int
    qtypes: tuple      # (8,), (4,) or (4, 8)
    matrices: list
    ms: tuple          # activation row counts the workload is run at
    outlier_frac: float = 0.0
    outlier_mult: float = 20.0
    zero_block_frac: float = 0.0
    acts: list = field(default_factory=list)

    def __post_init__(self):
        if not self.acts:
            seen = []
            for mt in self.matrices:
                if mt.act not in [a for a, _ in seen]:
                    seen.append((mt.act, mt.cols))
            self.acts = seen

    def matrix(self, name) -> Matrix:
        for mt in self.matrices:
            if mt.name == name:
                return mt
        raise KeyError(name)

    def act_cols(self, act) -> int:
        for a, k in self.acts:
            if a == act:
                return k
        raise KeyError(act)

    def weight_bytes(self, qtype) -> int:
        """Storage bytes (quants + fp32 scales) of all matrices in `qtype`:
        20 B per 32-element block for Q4_0, 36 B for Q8_0."""
        per_block = (16 if qtype == 4 else 32) + 4
        return sum(mt.rows * mt.cols // QK for mt in self.matrices) * per_block


def _llama_stack(layers=8):
    mats = []
    for l in range(layers):
        mats.append(Matrix(f"W_up.{l}", 11008, 4096, f"x_up.{l}"))
        mats.append(Matrix(f"W_down.{l}", 4096, 11008, f"x_down.{l}"))
    return mats


WORKLOADS = {
    # Q8_0 256 x 512, the small parity case.
    "q8_256x512": Workload(
        "q8_256x512", 0, (8,), [Matrix("W", 256, 512, "x")], (1,)),
    # One TinyLlama-1.1B-shaped decoder layer (hidden 2048, 32 q / 4 kv
    # heads of 64, FFN 5632), Q4_0, M = 1.
    "tinyllama_layer_q4": Workload(
        "tinyllama_layer_q4", 1, (4,),
        [Matrix("W_q", 2048, 2048, "x_attn"), Matrix("W_k", 256, 2048, "x_attn"),
         Matrix("W_v", 256, 2048, "x_attn"), Matrix("W_o", 2048, 2048, "x_o"),
         Matrix("W_gate", 5632, 2048, "x_ffn"), Matrix("W_up", 5632, 2048, "x_ffn"),
         Matrix("W_down", 2048, 5632, "x_down")], (1,)),
    # Llama-7B-shaped FFN stack: 8 x (W_up 11008x4096, W_down 4096x11008),
    # Q4_0, activations with 1% outliers x20, run at M = 1 and M = 4.
    "llama7b_ffn_stack_q4": Workload(
        "llama7b_ffn_stack_q4", 2, (4,), _llama_stack(8), (1, 4),
        outlier_frac=0.01, outlier_mult=20.0),
    # Qwen2.5-0.5B-shaped FFN (hidden 896, FFN 4864) plus lm_head, Q8_0,
    # 1% of weight blocks all-zero.
    "qwen05b_ffn_lmhead_q8": Workload(
        "qwen05b_ffn_lmhead_q8", 3, (8,),
        [Matrix("W_gate", 4864, 896, "x_ffn"), Matrix("W_up", 4864, 896, "x_ffn"),
         Matrix("W_down", 896, 4864, "x_down"), Matrix("lm_head", 151936, 896, "x_final")],
        (1,), zero_block_frac=0.01),
    # Batched path: M in {16, 64} against the Llama-7B FFN pair, each weight
    # quantized both to Q4_0 and to Q8_0.
    "batched_ffn_q4q8": Workload(
        "batched_ffn_q4q8", 4, (4, 8),
        [Matrix("W_up", 11008, 4096, "x_up"), Matrix("W_down", 4096, 11008, "x_down")],
        (16, 64)),
}


CHUNK = 1 << 22
SELECT = (1 << 31) - 1   # chunk id of the generator that picks outliers / zero blocks


def _rng(seed: int, kind: int, index: int, m: int, chunk: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=(kind, index, m, chunk)))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_fill(out: np.ndarray, seed: int, kind: int, index: int, m: int, sigma: float):
    flat = out.reshape(-1)
    nch = (flat.size + CHUNK - 1) // CHUNK

    def fill(c):
        seg = flat[c * CHUNK:(c + 1) * CHUNK]
        _rng(seed, kind, index, m, c).standard_normal(out=seg, dtype=np.float32)
        if sigma != 1.0:
            seg *= np.float32(sigma)

    if nch <= 1:
        for c in range(nch):
            fill(c)
    else:
        with ThreadPoolExecutor(min(_threads(), nch)) as ex:
            list(ex.map(fill, range(nch)))


def weight(wl: Workload, name: str) -> np.ndarray:
    """float32 [rows, cols] weight draw for matrix `name` of workload `wl`."""
    idx = [mt.name for mt in wl.matrices].index(name)
    mt = wl.matrices[idx]
    w = np.empty((mt.rows, mt.cols), np.float32)
    _normal_fill(w, wl.seed, 0, idx, 0, 0.02)
    if wl.zero_block_frac > 0.0:
        nblk = mt.rows * mt.cols // QK
        cnt = int(round(wl.zero_block_frac * nblk))
        blk = _rng(wl.seed, 0, idx, 0, SELECT).choice(nblk, size=cnt, replace=False)
        w.reshape(nblk, QK)[blk] = 0.0
    return w


def activation(wl: Workload, act: str, m: int = 1) -> np.ndarray:
    """float32 [m, K] activation draw `act` of workload `wl` at m rows."""
    idx = [a for a, _ in wl.acts].index(act)
    k = wl.acts[idx][1]
    x = np.empty((m, k), np.float32)
    _normal_fill(x, wl.seed, 1, idx, m, 1.0)
    if wl.outlier_frac > 0.0:
        cnt = int(round(wl.outlier_frac * m * k))
        sel = _rng(wl.seed, 1, idx, m, SELECT).choice(m * k, size=cnt, replace=False)
        x.reshape(-1)[sel] *= np.float32(wl.outlier_mult)
    return x


# ---------------------------------------------------------------------------
# Raw fixtures: random storage bytes and scales, bypassing any quantizer, so
# that every representable byte value reaches the product.
# ---------------------------------------------------------------------------

def raw_q4(rng: np.random.Generator, rows: int, cols: int):
    """Uniform random Q4_0 storage (every byte value 0..255, so every nibble
    0..15 including nibble 0 = -8) and scales 2^U(-8,0) * U(0.5, 2)."""
    q = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    d = raw_scales(rng, (rows, cols // QK))
    return q, d


def raw_q8(rng: np.random.Generator, rows: int, cols: int, lo: int = -127, hi: int = 127):
    """Uniform random Q8_0 storage in [lo, hi] and scales as raw_q4."""
    q = rng.integers(lo, hi + 1, size=(rows, cols), dtype=np.int16).astype(np.int8)
    d = raw_scales(rng, (rows, cols // QK))
    return q, d


def raw_zp(rng: np.random.Generator, bits: int, rows: int, cols: int, with_zp: bool = True, block: int = 128):
    """Uniform random storage of the 128-block zero-point format: codes over
    every value (bytes 0..255, or both nibbles 0..15), zero points uniform
    over the code range (or None), scales as raw_q4."""
    q = rng.integers(0, 256, size=(rows, cols if bits == 8 else cols // 2), dtype=np.uint8)
    zp = rng.integers(0, 1 << bits, size=(rows, cols // block), dtype=np.uint8) if with_zp else None
    d = raw_scales(rng, (rows, cols // block))
    return q, d, zp


def raw_q4k(rng: np.random.Generator, rows: int, cols: int):
    """Uniform random K-quant storage: every nibble value, scales and minima
    over 0..63, super-block scales 2^U(-10,-4)."""
    q = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    sc = rng.integers(0, 64, size=(rows, cols // QK), dtype=np.uint8)
    mn = rng.integers(0, 64, size=(rows, cols // QK), dtype=np.uint8)
    d = np.exp2(rng.uniform(-10, -4, size=(rows, cols // 256))).astype(np.float32)
    dmin = np.exp2(rng.uniform(-10, -4, size=(rows, cols // 256))).astype(np.float32)
    return q, sc, mn, d, dmin


def raw_scales(rng: np.random.Generator, shape):
    e = rng.uniform(-8.0, 0.0, size=shape)
    u = rng.uniform(0.5, 2.0, size=shape)
    return (np.exp2(e) * u).astype(np.float32)


def normal(rng: np.random.Generator, shape, sigma=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x
