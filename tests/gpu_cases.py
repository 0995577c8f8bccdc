"""Shared helpers of the GPU parity tests: build seeded cases, run the library
through its C ABI binding, compute the oracle on the same bytes, compare."""
from __future__ import annotations

import sys

import numpy as np

import gemm_q8_act_amd as nvq
from gemm_q8_act_amd import synth

TOL_REL = 1e-5
TOL_ABS = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch

    assert torch.cuda.is_available(), "GPU test needs a visible gfx950 device"
    return torch


def to_dev(a: np.ndarray):
    torch = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def quantize_gpu(x: np.ndarray):
    torch = torch_dev()
    M, K = x.shape
    xd = to_dev(x)
    q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    d = torch.empty((M, K // 32), dtype=torch.int16, device="cuda")
    b = torch.empty((M, K // 16), dtype=torch.int16, device="cuda")
    nvq.nvq_quantize_act_q8_0(xd, q, d, b)
    return q, d, b


def host(t) -> np.ndarray:
    return t.cpu().numpy()


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, awa: np.ndarray, what: str):
    """|y_gpu - y_oracle| <= 1e-5 * sum|w*a| + 1e-6 element by element; also rejects
    an all-zero result (a silent no-op would otherwise pass on zero inputs)."""
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.isfinite(y_gpu).all(), f"{what}: non-finite output"
    err = np.abs(y_gpu.astype(np.float64) - y_ref.astype(np.float64))
    bound = TOL_REL * awa + TOL_ABS
    worst = float((err / bound).max()) if err.size else 0.0
    bad = int((err > bound).sum())
    assert bad == 0, f"{what}: {bad} of {err.size} outputs outside the bound (worst err/bound {worst:.3g})"
    if np.abs(y_ref).max() > 0:
        assert np.abs(y_gpu).max() > 0, f"{what}: output all zero"
    return worst


class NvCase:
    """Seeded NVFP4 case: logical weights (oracle side), packed weights on the GPU."""

    def __init__(self, M, N, K, seed, w_scale=1.0, outliers=False):
        self.M, self.N, self.K = M, N, K
        self.codes, self.scales, self.ws = synth.nvfp4_weights(N, K, seed, w_scale)
        self.x = synth.activations(M, K, seed + 1, outliers=outliers)
        self.w = to_dev(nvq.nvq_pack_nvfp4(self.codes, self.scales))
        self.q, self.d, self.b = quantize_gpu(self.x)
        self.qh, self.dh = host(self.q), host(self.d).view(np.uint16)

    def oracle_y(self, o, cols=None):
        return o.matmul_nvfp4(self.codes, self.scales, self.ws, self.qh, self.dh, cols=cols)


class Q41Case:
    """Seeded Q4_1 case; ``weights`` = (qw, dw, mw) and ``x`` replace the seeded ones."""

    def __init__(self, M, N, K, seed, weights=None, x=None):
        self.M, self.N, self.K = M, N, K
        self.qw, self.dw, self.mw = weights if weights is not None else synth.q4_1_weights(N, K, seed)
        self.x = x if x is not None else synth.activations(M, K, seed + 1)
        self.w = to_dev(nvq.nvq_pack_q4_1(self.qw, self.dw, self.mw))
        self.q, self.d, self.b = quantize_gpu(self.x)
        self.qh, self.dh = host(self.q), host(self.d).view(np.uint16)

    def oracle_y(self, o, cols=None):
        return o.matmul_q4_1(self.qw, self.dw, self.mw, self.qh, self.dh, cols=cols)


class Q4KCase:
    """Seeded Q4_K case; ``weights`` = (qw, sc, mn, d, dmin) and ``x`` replace the seeded ones."""

    def __init__(self, M, N, K, seed, weights=None, x=None):
        self.M, self.N, self.K = M, N, K
        self.qw, self.sc, self.mn, self.dd, self.dm = weights if weights is not None else synth.q4_k_weights(N, K, seed)
        self.x = x if x is not None else synth.activations(M, K, seed + 1)
        self.w = to_dev(nvq.nvq_pack_q4_k(self.qw, self.sc, self.mn, self.dd, self.dm))
        self.q, self.d, self.b = quantize_gpu(self.x)
        self.qh, self.dh = host(self.q), host(self.d).view(np.uint16)

    def oracle_y(self, o, cols=None):
        return o.matmul_q4_k(self.qw, self.sc, self.mn, self.dd, self.dm, self.qh, self.dh, cols=cols)


class Q5KCase:
    """Seeded Q5_K case; ``weights`` = (qw, sc, mn, d, dmin) and ``x`` replace the seeded ones."""

    def __init__(self, M, N, K, seed, weights=None, x=None):
        self.M, self.N, self.K = M, N, K
        self.qw, self.sc, self.mn, self.dd, self.dm = weights if weights is not None else synth.q5_k_weights(N, K, seed)
        self.x = x if x is not None else synth.activations(M, K, seed + 1)
        self.w = to_dev(nvq.nvq_pack_q5_k(self.qw, self.sc, self.mn, self.dd, self.dm))
        self.q, self.d, self.b = quantize_gpu(self.x)
        self.qh, self.dh = host(self.q), host(self.d).view(np.uint16)

    def oracle_y(self, o, cols=None):
        return o.matmul_q5_k(self.qw, self.sc, self.mn, self.dd, self.dm, self.qh, self.dh, cols=cols)


class Q6KCase:
    """Seeded Q6_K case; ``weights`` = (qw, sc, d) and ``x`` replace the seeded ones."""

    def __init__(self, M, N, K, seed, weights=None, x=None):
        self.M, self.N, self.K = M, N, K
        self.qw, self.sc, self.dd = weights if weights is not None else synth.q6_k_weights(N, K, seed)
        self.x = x if x is not None else synth.activations(M, K, seed + 1)
        self.w = to_dev(nvq.nvq_pack_q6_k(self.qw, self.sc, self.dd))
        self.q, self.d, self.b = quantize_gpu(self.x)
        self.qh, self.dh = host(self.q), host(self.d).view(np.uint16)

    def oracle_y(self, o, cols=None):
        return o.matmul_q6_k(self.qw, self.sc, self.dd, self.qh, self.dh, cols=cols)


class IQ4Case:
    """Seeded IQ4_XS case; ``weights`` = (qw, ls, d, table) and ``x`` replace the seeded ones."""

    def __init__(self, M, N, K, seed, weights=None, x=None):
        self.M, self.N, self.K = M, N, K
        self.qw, self.ls, self.dd, self.table = weights if weights is not None else synth.iq4_xs_weights(N, K, seed)
        self.x = x if x is not None else synth.activations(M, K, seed + 1)
        self.w = to_dev(nvq.nvq_pack_iq4_xs(self.qw, self.ls, self.dd))
        self.q, self.d, self.b = quantize_gpu(self.x)
        self.qh, self.dh = host(self.q), host(self.d).view(np.uint16)

    def oracle_y(self, o, cols=None):
        return o.matmul_iq4_xs(self.qw, self.ls, self.dd, self.table, self.qh, self.dh, cols=cols)


def spike_activations(M: int, K: int, seed: int) -> np.ndarray:
    """One large value (|x| in 500..2000) per 32-block at a position k % 4 == 0, over
    N(0, 0.1) that quantizes to 0: every block's Q8_0 codes are one +-127 and zeros."""
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, 0.1, (M, K)).astype(np.float32)
    nb = K // 32
    pos = 32 * np.arange(nb)[None, :] + 4 * rng.integers(0, 8, (M, nb))
    x[np.arange(M)[:, None], pos] = (rng.choice([-1.0, 1.0], (M, nb)) * rng.uniform(500.0, 2000.0, (M, nb)))
    return x


def sample_cols(N: int, count: int, seed: int, tile: int = 128) -> np.ndarray:
    """First/last columns, both sides of tile boundaries, plus seeded random ones."""
    base = {0, 1, N - 1, N - 2}
    for t in (tile, 2 * tile, (N // tile) * tile):
        base |= {t - 1, t}
    r = np.random.Generator(np.random.PCG64(seed))
    base |= set(int(v) for v in r.integers(0, N, count))
    return np.array(sorted(c for c in base if 0 <= c < N), np.int64)
