"""GPU parity of the Q5_K x Q8_0 entries (nvq_gemv_q5_k, nvq_gemm_q5_k and the Q5_K
debug sums) against the oracle, through the C ABI binding.  Q5_K follows the GGML
format's rule stated in include/nvq.h (the pages only name the format); the oracle
computes the same rule as its plain definition."""
import numpy as np
import pytest

import gemm_q8_act_amd as nvq
from gemm_q8_act_amd import synth
from gpu_cases import Q5KCase, check_y, host, sample_cols, say, spike_activations, torch_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (1, 33, 256), (4, 70, 512), (8, 300, 4096), (15, 129, 768),
                                   (3, 33, 20480), (2, 50, 20736)])
def test_q5_k_gemv(oracle, M, N, K):
    """GEMV entry: the integer-dot GEMV kernel (rows up to 20480 weights), and past it
    the integer-MFMA kernel with one work item per tile (K = 20736)."""
    say(f"q5_k gemv M={M} N={N} K={K}")
    torch = torch_dev()
    c = Q5KCase(M, N, K, 11001 + M * N)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemv_q5_k(c.w, c.q, c.d, c.b, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"q5_k gemv M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(16, 64, 256), (17, 300, 768), (40, 77, 512), (64, 520, 1024),
                                   (100, 130, 1024), (128, 40, 4096), (257, 77, 256), (16, 70, 20736)])
def test_q5_k_gemm(oracle, M, N, K):
    """GEMM entry: M = 16 on the GEMV kernel (or, past 20480 weights per row, the
    integer-MFMA kernel), M > 16 the integer-MFMA kernel's three tile heights with K-split
    parts on small grids, ragged N and M tiles."""
    say(f"q5_k gemm M={M} N={N} K={K}")
    torch = torch_dev()
    c = Q5KCase(M, N, K, 11103 + M + N)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemm_q5_k(c.w, c.q, c.d, c.b, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"q5_k gemm M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [512, 1])
def test_q5_k_full_size(oracle, M):
    """The benchmarked shape N = K = 4096 (GEMM at M = 512 on sampled columns, GEMV at
    M = 1 in full)."""
    say(f"q5_k M={M} N=K=4096")
    torch = torch_dev()
    c = Q5KCase(M, 4096, 4096, synth.seed_for("q5_k", "w"))
    y = torch.empty((M, 4096), dtype=torch.float32, device="cuda")
    (nvq.nvq_gemm_q5_k if M > nvq.NVQ_GEMV_MAX_M else nvq.nvq_gemv_q5_k)(c.w, c.q, c.d, c.b, y)
    cols = sample_cols(4096, 48, 13) if M > 1 else None
    yo, awa = c.oracle_y(oracle, cols=cols)
    check_y(host(y) if cols is None else host(y)[:, cols], yo, awa, f"q5_k M={M}")


def _q5k_extreme_rows(N, K, seed):
    """Q5_K rows across the binary16 range: largest d and dmin with 63 scales and mins and
    code 31, subnormal d and dmin, an all-zero row, a min-only row, very different
    super-blocks in one row, codes that all carry the fifth bit."""
    qw, sc, mn, dd, dm = synth.q5_k_weights(N, K, seed)
    d = dd.view(np.float16).astype(np.float32)
    m = dm.view(np.float16).astype(np.float32)
    d[0], m[0], sc[0], mn[0], qw[0, ::3] = 65504.0, 65504.0, 63, 63, 31
    d[1], m[1] = 6e-8, 3e-7
    sc[2], mn[2] = 0, 0
    sc[3] = 0
    d[4, ::2], m[4, ::2] = 2000.0, 0.0
    qw[5] |= 16
    return qw, sc, mn, d.astype(np.float16).view(np.uint16), m.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("M", [200, 80, 40, 8])
def test_q5_k_extreme_weight_rows(oracle, M):
    """Per-row weight magnitudes from ~1e-8 to 1e8 through the three integer-MFMA tile
    shapes (M = 200, 80, 40) and the GEMV kernel (M = 8)."""
    say(f"q5_k extreme weight rows M={M}")
    torch = torch_dev()
    N, K = 70, 768
    c = Q5KCase(M, N, K, 0, weights=_q5k_extreme_rows(N, K, 1121), x=synth.activations(M, K, 1122))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    (nvq.nvq_gemm_q5_k if M > nvq.NVQ_GEMV_MAX_M else nvq.nvq_gemv_q5_k)(c.w, c.q, c.d, c.b, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"q5_k extreme rows M={M}")
    assert (host(y)[:, 2] == 0.0).all()


def _cancelling_rows(N, K, seed):
    """Q5_K super-blocks whose weights d sc c - dmin mn cross zero at a code z0:
    mn = sc and dmin = fp16(d z0), and every fourth code is z0, so those weights are
    sc times the binary16 rounding of d z0 (often 0) against parts of sc d z0."""
    qw, sc, mn, d, dmin = synth.q5_k_weights(N, K, seed)
    rng = np.random.default_rng(seed + 1)
    z0 = rng.integers(1, 32, (N, K // 256))
    df = d.view(np.float16).astype(np.float32)
    dmin = (df * z0).astype(np.float16).view(np.uint16)
    sc = np.maximum(sc, 1).astype(np.uint8)
    qw = qw.copy()
    qw.reshape(N, K // 256, 256)[:, :, ::4] = z0[:, :, None]
    return qw, sc, sc.copy(), d, dmin


@pytest.mark.parametrize("M", [200, 100, 40])
def test_q5_k_gemm_cancelling_weights(oracle, M):
    """Weights far smaller than their scale and offset parts, met by activation blocks
    with one nonzero code on those weights (every tile height): within the bound
    relative to sum |w * a|."""
    say(f"q5_k gemm (M={M}) cancelling weights")
    torch = torch_dev()
    N, K = 300, 768
    c = Q5KCase(M, N, K, 0, weights=_cancelling_rows(N, K, 5252), x=spike_activations(M, K, 5253))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemm_q5_k(c.w, c.q, c.d, c.b, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"q5_k cancelling weights M={M}")


@pytest.mark.parametrize("M", [200, 24])
def test_q5_k_gemm_activation_range(oracle, M):
    """Activation blocks with d >= 512 through the integer-MFMA kernel (d applied in float32)."""
    say(f"q5_k gemm (M={M}) large activations")
    torch = torch_dev()
    N, K = 300, 768
    x = synth.activations(M, K, 1131)
    x[5, 3] = 1.0e6
    x[2, :] *= 1.0e5
    x[M // 2, K - 32:] = 8.0e6
    c = Q5KCase(M, N, K, 1130, x=x)
    assert ((c.dh[2] & 0x7FFF) >= 0x6000).all()
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemm_q5_k(c.w, c.q, c.d, c.b, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"q5_k large activations M={M}")


@pytest.mark.parametrize("path,M,N,K", [(0, 1, 37, 256), (0, 3, 70, 512), (0, 15, 33, 768), (0, 2, 20, 20736),
                                        (1, 16, 64, 256), (1, 17, 300, 768), (1, 100, 130, 1024),
                                        (1, 512, 256, 4096), (1, 16, 40, 20736)])
def test_q5_k_isums_bit_exact(oracle, path, M, N, K):
    """Integer per-16 sums (5-bit codes times activation codes) of the kernel each Q5_K
    entry dispatches, bit for bit."""
    say(f"q5_k isums path={path} M={M} N={N} K={K}")
    torch = torch_dev()
    c = Q5KCase(M, N, K, 11207 + M + N)
    isums = torch.full((M, N, K // 16), -7, dtype=torch.int32, device="cuda")
    nvq.nvq_debug_isums(nvq.NVQ_FMT_Q5_K, path, c.w, c.q, N, isums)
    ref = oracle.isums_q5_k(c.qw, c.qh)
    assert (host(isums) == ref).all()
    assert np.abs(ref).max() > 0


def test_q5_k_gemm_split_determinism_and_guard_bands(oracle):
    """Junk workspace on entry, bitwise-identical repeats, nothing written outside y."""
    say("q5_k gemm K-split determinism + guard bands")
    torch = torch_dev()
    M, N, K = 100, 260, 1024
    c = Q5KCase(M, N, K, 11333)
    need = nvq.nvq_gemm_workspace_bytes(nvq.NVQ_FMT_Q5_K, M, N, K)
    assert need > 0
    guard = 4096
    outs = []
    for rep in range(2):
        buf = torch.full((M * N + 2 * guard,), 12345.0, dtype=torch.float32, device="cuda")
        y = buf[guard:guard + M * N].view(M, N)
        ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
        nvq.nvq_gemm_q5_k(c.w, c.q, c.d, c.b, y, workspace=ws)
        torch.cuda.synchronize()
        b = host(buf)
        assert (b[:guard] == 12345.0).all() and (b[guard + M * N:] == 12345.0).all()
        outs.append(b[guard:guard + M * N].copy())
    assert (outs[0].view(np.uint32) == outs[1].view(np.uint32)).all()
    yo, awa = c.oracle_y(oracle, cols=np.arange(0, N, 5))
    check_y(outs[0].reshape(M, N)[:, ::5], yo, awa, "q5_k split determinism case")
