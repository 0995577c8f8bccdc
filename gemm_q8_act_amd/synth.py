"""Seeded synthetic inputs for the NVFP4 / Q4_1 / Q4_K / IQ4_XS x Q8_0 product.

This module only draws random numbers; it holds none of the product's arithmetic
(no decode, no quantization, no dot products).  Both the GPU path's tests/benchmark
and the oracle's tests take their inputs from here, so the two sides always see the
same bytes.

Workload recipes (the shapes and value distributions of the decode/prefill
workloads this library targets):

* NVFP4 weights: every 4-bit code uniform over all 16 codes; one UE4M3 scale per
  16 weights with its unbiased exponent uniform in [-4, 4] and its 3-bit mantissa
  uniform, i.e. byte = ((e + 7) << 3) | m; a float32 per-tensor scale (1.0, or
  uniform in [0.5, 2] for the layer-set workloads).
* Activations: float32 N(0, 1); the prefill workload also multiplies
  round(0.001 * M * K) distinct, seeded positions by 50 (sign kept).
* Q4_1 weights: codes uniform 0..15, per 32 weights d ~ U[1e-3, 2e-2] and
  m ~ U[-0.1, 0], drawn in float32 and stored as binary16 (numpy's
  round-to-nearest-even conversion).
* Q4_K weights (the pages give the block size only; this recipe mirrors the Q4_1 one
  at the sub-block level): codes uniform 0..15, per 32 weights a 6-bit scale and a
  6-bit min uniform 0..63, per 256 weights d ~ U[2e-5, 3e-4] and dmin ~ U[0, 1.6e-3]
  (so d * sc lies in [0, 0.019] and dmin * mn in [0, 0.1]), drawn in float32 and
  stored as binary16; N = K = 4096 like the Q4_1 workload.
* IQ4_XS weights (the pages give the block size only): codes uniform 0..15; a value
  table of 16 distinct int8 values drawn uniformly from -127..127 and sorted (the
  non-linear table the format indexes; the pages do not print one); per 32 weights a
  6-bit scale uniform 0..63 (used as ls - 32); per 256 weights d ~ U[5e-5, 2e-4]
  (weights of magnitude up to ~0.8, most below 0.1); N = K = 4096.
* Expert routing (the mixture-of-experts decode step): 256 experts of shape
  N = K = 2048 (the pages give K = 2048, 256 experts, 6 active; N is taken equal to
  K), NVFP4 weights as above with a per-expert scale uniform in [0.5, 2]; each
  token's 6 experts are distinct and uniform over the 256 (a top-6 router over
  random logits).
"""
from __future__ import annotations

import numpy as np

# Decode GEMV set of one transformer layer at hidden 5120, ffn 17408 (N, K).
LAYER = (("qkv", 7168, 5120), ("o", 5120, 5120), ("gate_up", 34816, 5120), ("down", 5120, 17408))

WORKLOADS = {
    "gemv_small": dict(M=1, N=4864, K=896),
    "layer": dict(M=1, mats=LAYER),
    "prefill": dict(Ms=(256, 2048), N=17408, K=5120),
    "q4_1": dict(Ms=(1, 512), N=4096, K=4096),
    "q4_k": dict(Ms=(1, 512), N=4096, K=4096),
    "iq4_xs": dict(Ms=(1, 512), N=4096, K=4096),
    "q5_k": dict(Ms=(1, 512), N=4096, K=4096),
    "q6_k": dict(Ms=(1, 512), N=4096, K=4096),
    "stack": dict(Ms=(1, 8), layers=64, mats=LAYER),
    "moe": dict(M=1, experts=256, active=6, N=2048, K=2048),
}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def nvfp4_weights(N: int, K: int, seed: int, w_scale: str | float = 1.0):
    """Returns (codes uint8 [N, K] in 0..15, scales uint8 [N, K/16], w_scale float32)."""
    assert K % 16 == 0
    r = rng(seed)
    codes = r.integers(0, 16, size=(N, K), dtype=np.uint8)
    e = r.integers(-4, 5, size=(N, K // 16), dtype=np.int16)
    m = r.integers(0, 8, size=(N, K // 16), dtype=np.int16)
    scales = (((e + 7) << 3) | m).astype(np.uint8)
    if w_scale == "uniform":
        ws = np.float32(r.uniform(0.5, 2.0))
    else:
        ws = np.float32(w_scale)
    return codes, scales, ws


def activations(M: int, K: int, seed: int, outliers: bool = False) -> np.ndarray:
    """float32 [M, K], N(0,1); with ``outliers`` 0.1 % of positions scaled by 50."""
    r = rng(seed)
    x = r.standard_normal(size=(M, K), dtype=np.float32)
    if outliers:
        n = int(round(0.001 * M * K))
        if n:
            idx = r.choice(M * K, size=n, replace=False)
            x.reshape(-1)[idx] *= np.float32(50.0)
    return x


def q4_1_weights(N: int, K: int, seed: int):
    """Returns (qw uint8 [N, K] in 0..15, dw uint16 [N, K/32], mw uint16 [N, K/32])."""
    assert K % 32 == 0
    r = rng(seed)
    qw = r.integers(0, 16, size=(N, K), dtype=np.uint8)
    d = r.uniform(1e-3, 2e-2, size=(N, K // 32)).astype(np.float32)
    m = r.uniform(-0.1, 0.0, size=(N, K // 32)).astype(np.float32)
    return qw, d.astype(np.float16).view(np.uint16), m.astype(np.float16).view(np.uint16)


def q4_k_weights(N: int, K: int, seed: int):
    """Returns (qw uint8 [N, K] in 0..15, sc uint8 [N, K/32] in 0..63, mn uint8 [N, K/32]
    in 0..63, d uint16 [N, K/256], dmin uint16 [N, K/256])."""
    assert K % 256 == 0
    r = rng(seed)
    qw = r.integers(0, 16, size=(N, K), dtype=np.uint8)
    sc = r.integers(0, 64, size=(N, K // 32), dtype=np.uint8)
    mn = r.integers(0, 64, size=(N, K // 32), dtype=np.uint8)
    d = r.uniform(2e-5, 3e-4, size=(N, K // 256)).astype(np.float32)
    dmin = r.uniform(0.0, 1.6e-3, size=(N, K // 256)).astype(np.float32)
    return qw, sc, mn, d.astype(np.float16).view(np.uint16), dmin.astype(np.float16).view(np.uint16)


def q5_k_weights(N: int, K: int, seed: int):
    """Returns (qw uint8 [N, K] in 0..31, sc uint8 [N, K/32] in 0..63, mn uint8 [N, K/32]
    in 0..63, d uint16 [N, K/256], dmin uint16 [N, K/256])."""
    assert K % 256 == 0
    r = rng(seed)
    qw = r.integers(0, 32, size=(N, K), dtype=np.uint8)
    sc = r.integers(0, 64, size=(N, K // 32), dtype=np.uint8)
    mn = r.integers(0, 64, size=(N, K // 32), dtype=np.uint8)
    d = r.uniform(1e-5, 1.5e-4, size=(N, K // 256)).astype(np.float32)
    dmin = r.uniform(0.0, 1.6e-3, size=(N, K // 256)).astype(np.float32)
    return qw, sc, mn, d.astype(np.float16).view(np.uint16), dmin.astype(np.float16).view(np.uint16)


def q6_k_weights(N: int, K: int, seed: int):
    """Returns (qw uint8 [N, K] in 0..63 (used as qw - 32), sc int8 [N, K/16] in
    -128..127, d uint16 [N, K/256])."""
    assert K % 256 == 0
    r = rng(seed)
    qw = r.integers(0, 64, size=(N, K), dtype=np.uint8)
    sc = r.integers(-128, 128, size=(N, K // 16), dtype=np.int16).astype(np.int8)
    d = r.uniform(2e-6, 3e-5, size=(N, K // 256)).astype(np.float32)
    return qw, sc, d.astype(np.float16).view(np.uint16)


def iq4_xs_weights(N: int, K: int, seed: int):
    """Returns (qw uint8 [N, K] in 0..15, ls uint8 [N, K/32] in 0..63, d uint16 [N, K/256],
    table int8 [16])."""
    assert K % 256 == 0
    r = rng(seed)
    qw = r.integers(0, 16, size=(N, K), dtype=np.uint8)
    ls = r.integers(0, 64, size=(N, K // 32), dtype=np.uint8)
    d = r.uniform(5e-5, 2e-4, size=(N, K // 256)).astype(np.float32)
    table = np.sort(r.choice(np.arange(-127, 128), size=16, replace=False)).astype(np.int8)
    return qw, ls, d.astype(np.float16).view(np.uint16), table


def expert_ids(M: int, A: int, E: int, seed: int) -> np.ndarray:
    """int32 [M, A]: for each token A distinct experts, uniform over E."""
    r = rng(seed)
    return np.stack([r.choice(E, size=A, replace=False) for _ in range(M)]).astype(np.int32)


def seed_for(workload: str, tensor: str, index: int = 0) -> int:
    """Fixed, documented seed per (workload, tensor, index)."""
    base = {"gemv_small": 100, "layer": 200, "prefill": 300, "q4_1": 400, "stack": 500,
            "moe": 600, "q4_k": 700, "iq4_xs": 800, "test": 900, "q5_k": 1000, "q6_k": 1100}[workload]
    tag = sum((i + 1) * ord(ch) for i, ch in enumerate(tensor)) % 997
    return base * 1_000_003 + tag * 1009 + index
