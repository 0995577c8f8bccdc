"""GPU parity of the IQ4_XS x Q8_0 entries (nvq_gemv_iq4_xs, nvq_gemm_iq4_xs and
nvq_debug_isums_iq4_xs) against the oracle, through the C ABI binding.  The 16-entry
value table the codes index is an argument (the pages print none): seeded tables, the
extremes -128 / 127, and an affine one."""
import numpy as np
import pytest

import gemm_q8_act_amd as nvq
from gemm_q8_act_amd import synth
from gpu_cases import IQ4Case, check_y, host, sample_cols, say, torch_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (1, 33, 256), (4, 70, 512), (8, 300, 4096), (15, 129, 768),
                                   (3, 33, 20480), (2, 50, 20736)])
def test_iq4_xs_gemv(oracle, M, N, K):
    """GEMV entry: the integer-dot GEMV kernel with the table lookups, and past 20480
    weights per row the integer-MFMA kernel with one work item per tile."""
    say(f"iq4_xs gemv M={M} N={N} K={K}")
    torch = torch_dev()
    c = IQ4Case(M, N, K, 8001 + M * N)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemv_iq4_xs(c.w, c.table, c.q, c.d, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"iq4_xs gemv M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(16, 64, 256), (17, 300, 768), (40, 77, 512), (100, 130, 1024),
                                   (128, 40, 4096), (257, 77, 256), (16, 70, 20736)])
def test_iq4_xs_gemm(oracle, M, N, K):
    """GEMM entry: M = 16 on the GEMV kernel (or the integer-MFMA kernel past 20480
    weights per row), M > 16 the integer-MFMA kernel's three tile heights with K-split
    parts."""
    say(f"iq4_xs gemm M={M} N={N} K={K}")
    torch = torch_dev()
    c = IQ4Case(M, N, K, 8103 + M + N)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemm_iq4_xs(c.w, c.table, c.q, c.d, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"iq4_xs gemm M={M} N={N} K={K}")


def test_iq4_xs_gemm_full_size(oracle):
    say("iq4_xs gemm M=512 N=K=4096")
    torch = torch_dev()
    c = IQ4Case(512, 4096, 4096, synth.seed_for("iq4_xs", "w"))
    y = torch.empty((512, 4096), dtype=torch.float32, device="cuda")
    nvq.nvq_gemm_iq4_xs(c.w, c.table, c.q, c.d, y)
    cols = sample_cols(4096, 48, 13)
    yo, awa = c.oracle_y(oracle, cols=cols)
    check_y(host(y)[:, cols], yo, awa, "iq4_xs M=512")


def _iq4_special(N, K, seed, table):
    """Rows with the largest d and scales (ls = 0 and 63: factors -32 and 31), a
    subnormal d, a zero-scale row (ls = 32), and every code of the table in one row."""
    qw, ls, dd, _ = synth.iq4_xs_weights(N, K, seed)
    d = dd.view(np.float16).astype(np.float32)
    d[0], ls[0] = 65504.0, 0
    d[1], ls[1] = 65504.0, 63
    d[2] = 6e-8
    ls[3] = 32
    qw[4] = np.arange(K) % 16
    return qw, ls, d.astype(np.float16).view(np.uint16), table


@pytest.mark.parametrize("M", [200, 40, 8, 1])
@pytest.mark.parametrize("kind", ["extremes", "affine"])
def test_iq4_xs_special_rows_and_tables(oracle, M, kind):
    """Tables holding -128 and 127 (the int8 extremes) or the affine c - 8; rows up to
    65504 * 32 * 128 in magnitude, a zero row; through the integer-MFMA tile heights
    (M = 200, 40) and the GEMV kernel (M = 8, 1)."""
    say(f"iq4_xs special rows M={M} table={kind}")
    torch = torch_dev()
    N, K = 70, 768
    table = (np.array([-128, -100, -64, -33, -17, -9, -2, -1, 0, 1, 3, 11, 30, 64, 99, 127], np.int8)
             if kind == "extremes" else (np.arange(16) - 8).astype(np.int8))
    c = IQ4Case(M, N, K, 0, weights=_iq4_special(N, K, 941, table), x=synth.activations(M, K, 942))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    (nvq.nvq_gemm_iq4_xs if M > nvq.NVQ_GEMV_MAX_M else nvq.nvq_gemv_iq4_xs)(c.w, c.table, c.q, c.d, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"iq4_xs special M={M} {kind}")
    assert (host(y)[:, 3] == 0.0).all()


@pytest.mark.parametrize("path,M,N,K", [(0, 1, 37, 256), (0, 3, 70, 512), (0, 15, 33, 768), (0, 2, 20, 20736),
                                        (1, 16, 64, 256), (1, 17, 300, 768), (1, 100, 130, 1024),
                                        (1, 512, 256, 4096), (1, 16, 40, 20736)])
def test_iq4_xs_isums_bit_exact(oracle, path, M, N, K):
    """Per-16 sums of table values times activation codes from the kernel each entry
    dispatches, bit for bit, with a table that holds both int8 extremes."""
    say(f"iq4_xs isums path={path} M={M} N={N} K={K}")
    torch = torch_dev()
    qw, ls, dd, _ = synth.iq4_xs_weights(N, K, 8207 + M + N)
    table = np.array([-128, -90, -60, -41, -25, -12, -5, -1, 2, 7, 15, 29, 48, 70, 101, 127], np.int8)
    c = IQ4Case(M, N, K, 0, weights=(qw, ls, dd, table), x=synth.activations(M, K, 8208 + M))
    isums = torch.full((M, N, K // 16), -7, dtype=torch.int32, device="cuda")
    nvq.nvq_debug_isums_iq4_xs(c.table, path, c.w, c.q, N, isums)
    ref = oracle.isums_iq4_xs(c.qw, c.table, c.qh)
    assert (host(isums) == ref).all()
    assert np.abs(ref).max() > 0
