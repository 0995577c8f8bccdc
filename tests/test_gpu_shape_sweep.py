"""Seeded random shapes through every product entry, against the oracle.

The other parity tests pick their shapes by hand (tile boundaries, K-split plans,
ragged tails).  Here a fixed-seed generator draws further (M, N, K) per entry point:
N anywhere in 1..3000, K any multiple of the format's block granularity, and M across
the whole range of the entry, so the kernel choice, tile counts and K-split plans land
on combinations no hand-picked case names.  Outputs are compared on sampled columns
(both ends, tile boundaries, random ones) within |dy| <= 1e-5 sum|w a| + 1e-6.
"""
import numpy as np
import pytest

import gemm_q8_act_amd as nvq
from gpu_cases import (IQ4Case, NvCase, Q41Case, Q4KCase, Q5KCase, Q6KCase, check_y, host, sample_cols, say,
                       to_dev, torch_dev)

pytestmark = pytest.mark.gpu

# (entry, M range, K granularity, K max); GEMV entries take 1 <= M <= 15, GEMM entries
# M >= 16 (at M = 16 they run the batched or GEMV kernels)
_ENTRIES = [
    ("nvfp4_gemv", (1, 15), 64, 8192),
    ("nvfp4_dot4", (1, 15), 64, 8192),
    ("nvfp4_fused", (1, 1), 64, 8192),
    ("nvfp4_gemm", (16, 1100), 64, 4096),
    ("q4_1_gemv", (1, 15), 32, 8192),
    ("q4_1_gemm", (16, 1100), 32, 4096),
    ("q4_k_gemv", (1, 15), 256, 8192),
    ("q4_k_gemm", (16, 1100), 256, 4096),
    ("q5_k_gemv", (1, 15), 256, 8192),
    ("q5_k_gemm", (16, 1100), 256, 4096),
    ("q6_k_gemv", (1, 15), 256, 8192),
    ("q6_k_gemm", (16, 1100), 256, 4096),
    ("iq4_xs_gemv", (1, 15), 256, 8192),
    ("iq4_xs_gemm", (16, 1100), 256, 4096),
]
_PER_ENTRY = 16


def _cases():
    rng = np.random.Generator(np.random.PCG64(20261204))
    out = []
    for name, (m0, m1), kg, kmax in _ENTRIES:
        for i in range(_PER_ENTRY):
            M = int(rng.integers(m0, m1 + 1))
            N = int(rng.integers(1, 3001))
            K = kg * int(rng.integers(1, kmax // kg + 1))
            out.append(pytest.param(name, M, N, K, 7000 + 97 * len(out), id=f"{name}-M{M}-N{N}-K{K}"))
    return out


@pytest.mark.parametrize("entry,M,N,K,seed", _cases())
def test_random_shape(oracle, entry, M, N, K, seed):
    say(f"shape sweep {entry} M={M} N={N} K={K} seed={seed}")
    torch = torch_dev()
    fmt = "nvfp4" if entry.startswith("nvfp4") else entry.split("_gem")[0]
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    if fmt == "nvfp4":
        c = NvCase(M, N, K, seed, w_scale=0.75, outliers=entry == "nvfp4_gemm")
        if entry == "nvfp4_gemv":
            nvq.nvq_gemv_nvfp4(c.w, c.ws, c.q, c.d, y)
        elif entry == "nvfp4_dot4":
            nvq.nvq_gemv_nvfp4_dot4(c.w, c.ws, c.q, c.d, y)
        elif entry == "nvfp4_fused":
            nvq.nvq_gemv_nvfp4_fused(c.w, c.ws, to_dev(c.x), y)
        else:
            nvq.nvq_gemm_nvfp4(c.w, c.ws, c.q, c.d, y)
    else:
        case = {"q4_1": Q41Case, "q4_k": Q4KCase, "q5_k": Q5KCase, "q6_k": Q6KCase, "iq4_xs": IQ4Case}[fmt]
        c = case(M, N, K, seed)
        gemv = entry.endswith("gemv")
        if fmt == "iq4_xs":
            t = np.ascontiguousarray(c.table, dtype=np.int8)
            (nvq.nvq_gemv_iq4_xs if gemv else nvq.nvq_gemm_iq4_xs)(c.w, t, c.q, c.d, y)
        elif fmt == "q6_k":
            (nvq.nvq_gemv_q6_k if gemv else nvq.nvq_gemm_q6_k)(c.w, c.q, c.d, y)
        else:
            f = getattr(nvq, f"nvq_{'gemv' if gemv else 'gemm'}_{fmt}")
            f(c.w, c.q, c.d, c.b, y)
    cols = sample_cols(N, 24, seed)
    yo, awa = c.oracle_y(oracle, cols=cols)
    check_y(host(y)[:, cols], yo, awa, f"{entry} M={M} N={N} K={K}")
