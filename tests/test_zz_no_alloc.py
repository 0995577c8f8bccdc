"""The no-allocation prefill GEMM (nvq_gemm_nvfp4_noalloc, K-split partials in the
library's static per-GPU scratch) against nvq_gemm_nvfp4 with a caller workspace, on
calls in a row with shrinking inputs: the largest K-split plan (the scratch's full
64 MiB at the prefill shape), a smaller one, and shapes with no split at all."""
import numpy as np
import pytest

import gemm_q8_act_amd as nvq
from gemm_q8_act_amd import synth
from gpu_cases import NvCase, check_y, host, sample_cols, say, torch_dev

pytestmark = pytest.mark.gpu


def test_noalloc_gemm_matches_workspace_gemm(oracle):
    torch = torch_dev()
    # (M, N, K): 256 x 16384 x 4096 and 2048 x 17408 x 5120 need all 64 MiB (64 tiles in
    # 4 parts, 32 tiles in 8 parts), 256 x 17408 x 5120 51 MiB (68 tiles in 3 parts), 300 x
    # 2560 x 1280 12 parts per split tile, 100 x 520 x 1024 16 parts (256 x 128 tiles), 40 x
    # 70 x 64 a single stage (no split, no scratch)
    shapes = [(256, 16384, 4096), (2048, 17408, 5120), (256, 17408, 5120), (300, 2560, 1280), (100, 520, 1024),
              (40, 70, 64)]
    assert nvq.nvq_gemm_workspace_bytes(nvq.NVQ_FMT_NVFP4, 2048, 17408, 5120) == 64 << 20
    assert nvq.nvq_gemm_workspace_bytes(nvq.NVQ_FMT_NVFP4, 256, 16384, 4096) == 64 << 20
    for M, N, K in shapes:
        say(f"noalloc gemm M={M} N={N} K={K}")
        c = NvCase(M, N, K, synth.seed_for("test", "noalloc", M), w_scale=1.25, outliers=True)
        y_ws = torch.empty((M, N), dtype=torch.float32, device="cuda")
        nvq.nvq_gemm_nvfp4(c.w, c.ws, c.q, c.d, y_ws)
        y_na = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        nvq.nvq_gemm_nvfp4_noalloc(c.w, c.ws, c.q, c.d, y_na)
        torch.cuda.synchronize()
        a, b = host(y_na), host(y_ws)
        # same kernels and K-split plan: the same bits; and within the oracle's bound
        assert (a.view(np.uint32) == b.view(np.uint32)).all(), f"M={M} N={N} K={K}"
        cols = sample_cols(N, 16, M + N)
        yo, awa = c.oracle_y(oracle, cols=cols)
        check_y(a[:, cols], yo, awa, f"noalloc M={M} N={N} K={K}")


def test_noalloc_gemm_rejects_bad_arguments():
    torch = torch_dev()
    y = torch.full((8, 64), 7.0, dtype=torch.float32, device="cuda")
    w = torch.zeros(nvq.nvq_nvfp4_weight_bytes(64, 128), dtype=torch.uint8, device="cuda")
    q = torch.zeros((8, 128), dtype=torch.int8, device="cuda")
    d = torch.zeros((8, 4), dtype=torch.int16, device="cuda")
    st = nvq.lib().nvq_gemm_nvfp4_noalloc(w.data_ptr(), 1.0, q.data_ptr(), d.data_ptr(), 8, 64, 128,
                                          y.data_ptr(), None)
    assert st == -2  # M < 16
    torch.cuda.synchronize()
    assert (host(y) == 7.0).all()
