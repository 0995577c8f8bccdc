"""GPU parity: every entry point of libnvq against the oracle, through the C ABI.

Integer outputs (Q8_0 codes, binary16 scales, per-16 code sums, integer per-16
dot sums) must be bit-exact; float32 outputs must satisfy
|y - y_oracle| <= 1e-5 * sum_k |W*A| + 1e-6 for every element.  Small cases are
checked in full (several tiles plus ragged tails); the full workload sizes are
checked on sampled output columns the oracle computes one by one."""
import numpy as np
import pytest

import gemm_q8_act_amd as nvq
from gemm_q8_act_amd import synth
from gpu_cases import (NvCase, Q41Case, check_y, host, quantize_gpu, sample_cols, say, spike_activations, to_dev,
                       torch_dev)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# Q8_0 activation quantization: bit-exact
# ---------------------------------------------------------------------------

def _edge_rows(K):
    rows = []
    z = np.zeros(K, np.float32)
    rows.append(z)                                             # all-zero blocks
    t = np.zeros(K, np.float32)
    t[:10] = [127.0, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 126.5, -3.5, 4.5]   # exact ties
    rows.append(t)
    r = np.random.Generator(np.random.PCG64(77))
    rows.append((r.standard_normal(K) * 1e-5).astype(np.float32))       # binary16-subnormal d
    rows.append((r.standard_normal(K) * 1e-9).astype(np.float32))       # d rounds to 0 in binary16
    rows.append((r.standard_normal(K) * 3e4).astype(np.float32))        # large values
    one = np.zeros(K, np.float32)
    one[K // 2] = -1.0                                         # single non-zero per row
    rows.append(one)
    sub = (r.integers(-60, 61, K) * np.float32(2.0 ** -149)).astype(np.float32)
    sub[32:64] *= 2                                            # float32 subnormals: d32 rounds to 0 where
    sub[32] = 127 * np.float32(2.0 ** -149)                    # amax < 63.5 * 2^-149, else d32 = 2^-149
    rows.append(sub)
    return np.stack(rows)


@pytest.mark.parametrize("M,K,outliers", [(1, 32, False), (1, 896, False), (3, 5120, False),
                                          (5, 17408, False), (37, 4096, True), (256, 5120, True)])
def test_act_quant_bit_exact(oracle, M, K, outliers):
    say(f"act_quant M={M} K={K}")
    x = synth.activations(M, K, synth.seed_for("test", "act", M * K), outliers=outliers)
    q, d, b = quantize_gpu(x)
    qo, do, bo = oracle.quantize_q8_0(x)
    assert (host(q) == qo).all()
    assert (host(d).view(np.uint16) == do).all()
    assert (host(b) == bo).all()


@pytest.mark.parametrize("K", [64, 5120])
def test_act_quant_edge_blocks(oracle, K):
    say(f"act_quant edge K={K}")
    x = _edge_rows(K)
    q, d, b = quantize_gpu(x)
    qo, do, bo = oracle.quantize_q8_0(x)
    assert (host(q) == qo).all()
    assert (host(d).view(np.uint16) == do).all()
    assert (host(b) == bo).all()
    assert do[2].max() < 0x0400 and do[2].max() > 0      # the subnormal-scale row is exercised
    assert not qo[6, :32].any() and qo[6, 32] == 127 and qo[6, 33:64].any()  # d32 = 0 and d32 = 2^-149 blocks


def _near_tie_rows(rows, K, seed):
    """Blocks whose quotients x / d32 sit on or within a few ulps of half-integers: the
    block's first value is amax (it fixes d32 = float32(amax / 127)), the others are
    float32((k + 0.5) * d32) moved by -3 .. +3 ulps, for random amax and k."""
    r = np.random.Generator(np.random.PCG64(seed))
    x = np.zeros((rows, K), np.float32)
    for i in range(rows):
        for b in range(K // 32):
            amax = np.float32(r.choice([1.0, 127.0, 3.0e4, 1e-3]) * r.uniform(0.5, 2.0))
            d32 = np.float32(amax / np.float32(127.0))
            k = r.integers(-127, 127, 31).astype(np.float32)
            base = ((k + np.float32(0.5)) * d32).astype(np.float32)
            steps = r.integers(-3, 4, 31)
            v = base.copy()
            for j in range(31):
                for _ in range(abs(int(steps[j]))):
                    v[j] = np.nextafter(v[j], np.float32(np.inf) if steps[j] > 0 else np.float32(-np.inf))
            v = np.clip(v, -amax, amax)
            x[i, 32 * b] = amax if r.integers(0, 2) else -amax
            x[i, 32 * b + 1: 32 * b + 32] = v
    return x


def test_act_quant_near_ties(oracle):
    """Quotients on and next to rounding ties decide the same codes as the oracle's
    correctly rounded division."""
    say("act_quant near-tie blocks")
    x = _near_tie_rows(48, 1024, 4711)
    q, d, b = quantize_gpu(x)
    qo, do, bo = oracle.quantize_q8_0(x)
    assert (host(q) == qo).all()
    assert (host(d).view(np.uint16) == do).all()
    assert (host(b) == bo).all()


def test_act_quant_large(oracle):
    """The prefill input shape (two blocks per thread), outliers included."""
    say("act_quant M=512 K=5120")
    x = synth.activations(512, 5120, synth.seed_for("test", "act_large"), outliers=True)
    q, d, b = quantize_gpu(x)
    qo, do, bo = oracle.quantize_q8_0(x)
    assert (host(q) == qo).all()
    assert (host(d).view(np.uint16) == do).all()
    assert (host(b) == bo).all()


def test_act_quant_without_bsum(oracle):
    torch = torch_dev()
    x = synth.activations(4, 256, 5)
    xd = to_dev(x)
    q = torch.empty((4, 256), dtype=torch.int8, device="cuda")
    d = torch.empty((4, 8), dtype=torch.int16, device="cuda")
    nvq.nvq_quantize_act_q8_0(xd, q, d, None)
    qo, do, _ = oracle.quantize_q8_0(x)
    assert (host(q) == qo).all() and (host(d).view(np.uint16) == do).all()


# ---------------------------------------------------------------------------
# NVFP4 decode GEMV, M = 1 (integer-dot kernel)
# ---------------------------------------------------------------------------

GEMV_SHAPES = [(4864, 896), (1, 64), (37, 128), (129, 640), (33, 320), (1000, 4096),
               (300, 5120), (130, 17408), (20, 20544)]


@pytest.mark.parametrize("N,K", GEMV_SHAPES)
@pytest.mark.parametrize("kernel", ["mfma", "dot4"])
def test_gemv_nvfp4_m1(oracle, N, K, kernel):
    say(f"gemv_nvfp4 ({kernel}) M=1 N={N} K={K}")
    torch = torch_dev()
    c = NvCase(1, N, K, synth.seed_for("test", "gemv", N * 7 + K), w_scale="uniform")
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    fn = nvq.nvq_gemv_nvfp4 if kernel == "mfma" else nvq.nvq_gemv_nvfp4_dot4
    fn(c.w, c.ws, c.q, c.d, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"gemv {kernel} N={N} K={K}")


# ---------------------------------------------------------------------------
# Fused Q8_0 quantization + decode GEMV (one token)
# ---------------------------------------------------------------------------

def _fused_run(w, ws, x, N):
    """One fused launch on the float32 row x; returns y, q_out, d_out on the host."""
    torch = torch_dev()
    K = x.shape[-1]
    y = torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda")
    qo = torch.full((1, K), 99, dtype=torch.int8, device="cuda")
    do = torch.full((1, K // 32), 0x7E00, dtype=torch.int16, device="cuda")
    nvq.nvq_gemv_nvfp4_fused(w, ws, to_dev(x.reshape(1, K)), y, qo, do)
    return host(y), host(qo), host(do).view(np.uint16)


# (N, K): several tiles with a ragged last one; K % 128 == 64; one to nine float4
# groups per thread and the in-block loop past nine (K = 20544 and 65536); the
# 8-wavefront launch (down projection: K = 17408, few tiles)
FUSED_SHAPES = [(4864, 896), (1, 64), (37, 128), (129, 640), (33, 320), (1000, 4096), (300, 5120),
                (130, 17408), (20, 20544), (40, 65536), (70, 9216), (17, 2304)]


@pytest.mark.parametrize("N,K", FUSED_SHAPES)
def test_gemv_fused(oracle, N, K):
    """y against the oracle's product on the oracle's own Q8_0 of x; the codes and
    scales the kernel used (q_out, d_out) bit-exact with the oracle's."""
    say(f"gemv fused N={N} K={K}")
    codes, scales, ws = synth.nvfp4_weights(N, K, synth.seed_for("test", "fused", N * 3 + K), "uniform")
    w = to_dev(nvq.nvq_pack_nvfp4(codes, scales))
    x = synth.activations(1, K, synth.seed_for("test", "fused_x", K), outliers=True)
    y, qk, dk = _fused_run(w, ws, x, N)
    qo, do, _ = oracle.quantize_q8_0(x)
    assert (qk == qo).all() and (dk == do).all()
    yo, awa = oracle.matmul_nvfp4(codes, scales, ws, qo, do)
    check_y(y, yo, awa, f"fused N={N} K={K}")


def test_gemv_fused_edge_and_tie_rows(oracle):
    """Rows whose Q8_0 decisions are delicate, one fused launch each: all-zero blocks,
    exact ties, binary16-subnormal and zero d, float32-subnormal blocks (d32 = 0 and
    d32 = 2^-149), large values, a single non-zero, and 48 rows of quotients on or
    within a few ulps of rounding ties."""
    say("gemv fused edge and near-tie rows")
    N, K = 40, 1024
    codes, scales, ws = synth.nvfp4_weights(N, K, 4040, "uniform")
    w = to_dev(nvq.nvq_pack_nvfp4(codes, scales))
    rows = np.concatenate([_edge_rows(K), _near_tie_rows(48, K, 4041)])
    for i, x in enumerate(rows):
        y, qk, dk = _fused_run(w, ws, x[None, :], N)
        qo, do, _ = oracle.quantize_q8_0(x[None, :])
        assert (qk == qo).all() and (dk == do).all(), f"row {i}"
        yo, awa = oracle.matmul_nvfp4(codes, scales, ws, qo, do)
        if np.abs(yo).max() > 0:
            check_y(y, yo, awa, f"fused edge row {i}")
        else:
            assert (y == 0).all(), f"row {i}"


@pytest.mark.parametrize("M", [1, 3])
@pytest.mark.parametrize("path", [nvq.NVQ_PATH_GEMV, nvq.NVQ_PATH_GEMV_DOT4])
def test_gemv_isums_bit_exact(oracle, M, path):
    """GEMV dispatch: M = 1 the decode kernel (matrix-core or v_dot4 inner loop),
    M = 3 the batched kernel (GEMV path) or one v_dot4 launch per token."""
    say(f"debug isums GEMV path={path} M={M}")
    torch = torch_dev()
    for N, K in [(37, 128), (33, 320), (70, 5120), (9, 20544)]:
        c = NvCase(M, N, K, 1234 + N)
        isums = torch.full((M, N, K // 16), -7, dtype=torch.int32, device="cuda")
        nvq.nvq_debug_isums(nvq.NVQ_FMT_NVFP4, path, c.w, c.q, N, isums)
        ref = oracle.isums_nvfp4(c.codes, c.qh)
        assert (host(isums) == ref).all(), (N, K)
        assert np.abs(ref).max() > 0


# Batched decode kernel, every token-group count and both launch shapes (fewer than
# 1024 tiles: 2 tiles x 8 wavefronts; from 1024 tiles up: T tiles x 4 wavefronts).
@pytest.mark.parametrize("M,N,K", [(2, 300, 640), (8, 129, 1024), (12, 77, 320), (15, 64, 5120),
                                   (8, 16379, 128), (12, 17627, 192), (5, 40, 64)])
def test_batched_isums_bit_exact(oracle, M, N, K):
    say(f"debug isums batched GEMV M={M} N={N} K={K}")
    torch = torch_dev()
    c = NvCase(M, N, K, 4400 + M + N)
    isums = torch.full((M, N, K // 16), -7, dtype=torch.int32, device="cuda")
    nvq.nvq_debug_isums(nvq.NVQ_FMT_NVFP4, nvq.NVQ_PATH_GEMV, c.w, c.q, N, isums)
    assert (host(isums) == oracle.isums_nvfp4(c.codes, c.qh)).all()


# ---------------------------------------------------------------------------
# NVFP4 tiled MFMA path: GEMV with 2 <= M <= 15 and GEMM with M >= 16
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(2, 300, 512), (8, 129, 1024), (15, 64, 64), (8, 77, 5120), (3, 50, 320)])
@pytest.mark.parametrize("kernel", ["mfma", "dot4"])
def test_gemv_nvfp4_small_batch(oracle, M, N, K, kernel):
    say(f"gemv_nvfp4 ({kernel}) M={M} N={N} K={K}")
    torch = torch_dev()
    c = NvCase(M, N, K, 4321 + M * N, w_scale="uniform")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    fn = nvq.nvq_gemv_nvfp4 if kernel == "mfma" else nvq.nvq_gemv_nvfp4_dot4
    fn(c.w, c.ws, c.q, c.d, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"gemv M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(2, 100, 640), (8, 100, 320), (5, 40, 128)])
def test_gemv_batched_large_activations(oracle, M, N, K):
    """Blocks whose binary16 scale d is >= 512 (|d * q| can pass the binary16 range)
    take the batched kernel's second pass; blocks just below stay in the main loop."""
    say(f"batched gemv large activations M={M} N={N} K={K}")
    torch = torch_dev()
    c = NvCase(M, N, K, 900 + M, w_scale="uniform")
    x = c.x.copy()
    x[1, 40:44] = [3.0e5, -2.0e5, 1.0e5, 7.0]      # d ~ 2362: second pass
    x[M - 1, 0:32] *= 6.0e4 / np.abs(x[M - 1, 0:32]).max()   # d ~ 472: main loop, |hi| near 60000
    x[0, :] *= 1.0e5                                # every block of token 0: d >= 512
    c.x = x
    c.q, c.d, c.b = quantize_gpu(x)
    c.qh, c.dh = host(c.q), host(c.d).view(np.uint16)
    assert (c.dh[1] & 0x7FFF).max() >= 0x6000 and (c.dh[M - 1, 0] & 0x7FFF) < 0x6000
    assert ((c.dh[0] & 0x7FFF) >= 0x6000).all()
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemv_nvfp4(c.w, c.ws, c.q, c.d, y)
    yo, awa = c.oracle_y(oracle)
    assert np.isfinite(host(y)).all()
    check_y(host(y), yo, awa, f"large activations M={M} N={N} K={K}")


# Batched decode from 1024 tiles up: T tiles per block with T chosen by tile count.
# (M, N): tiles -> T, blocks, tiles in the last block; every N leaves a ragged last tile.
@pytest.mark.parametrize("M,N", [
    (3, 16379),   # 1024 tiles -> T 4, 256 blocks, last full
    (3, 17627),   # 1102 -> T 5, 221 blocks, last 2
    (3, 22395),   # 1400 -> T 6, 234, last 2
    (3, 25595),   # 1600 -> T 7, 229, last 4
    (3, 28843),   # 1803 -> T 8, 226, last 3
    (3, 33595),   # 2100 -> T 9, 234, last 3
    (12, 17627),  # two token groups: 1102 -> T 5
    (12, 22395),  # 1400 -> T 6
    (12, 25595),  # 1600 -> T 7
    (12, 28843),  # 1803 -> T 8
    (12, 34811),  # 2176 -> T 9, 242 blocks, last 7
])
def test_gemv_batched_ragged_tile_groups(oracle, M, N):
    """Every tiles-per-block choice of the batched decode kernel, each with a last block
    that is only partly filled (or exactly full) and a ragged last tile."""
    say(f"batched gemv M={M} N={N} K=128")
    torch = torch_dev()
    K = 128
    c = NvCase(M, N, K, 4242 + M)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemv_nvfp4(c.w, c.ws, c.q, c.d, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"M={M} N={N} K=128")


# M = 16: batched decode kernel (two token groups); 16 < M <= 64 and M > 64: the
# split-activation kernel in 256 x 64 and 256 x 256 tiles, whose small shapes always
# take the K-split + ordered-reduction route (fewer tiles than compute units), except
# K = 64 (one stage: no split)
@pytest.mark.parametrize("M,N,K", [(16, 64, 64), (17, 77, 192), (100, 300, 640), (64, 128, 2048),
                                   (129, 257, 1024), (40, 70, 320), (300, 600, 384), (65, 33, 64),
                                   (257, 1000, 448), (520, 129, 128), (16, 300, 5120), (33, 520, 64),
                                   (64, 2000, 1024)])
def test_gemm_nvfp4(oracle, M, N, K):
    say(f"gemm_nvfp4 M={M} N={N} K={K}")
    torch = torch_dev()
    c = NvCase(M, N, K, 999 + M + N, w_scale=1.5, outliers=True)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemm_nvfp4(c.w, c.ws, c.q, c.d, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"gemm M={M} N={N} K={K}")


# GEMM dispatch: M = 1 the tiled kernel; 2 <= M <= 16 the batched kernel; the
# two-term kernel's three token-tile heights above (64: M <= 64, 128: M <= 128,
# 256), small grids split along K (up to 16 parts per tile), ragged N and M tiles.
@pytest.mark.parametrize("M,N,K", [(1, 70, 128), (2, 33, 192), (8, 64, 1024), (12, 20, 320), (15, 77, 640),
                                   (16, 100, 5120), (17, 33, 192), (40, 300, 1024), (64, 257, 640),
                                   (65, 70, 448), (100, 300, 1024), (128, 64, 2048), (129, 33, 320),
                                   (300, 300, 1024), (257, 520, 64)])
def test_gemm_isums_bit_exact(oracle, M, N, K):
    say(f"debug isums GEMM path M={M} N={N} K={K}")
    torch = torch_dev()
    c = NvCase(M, N, K, 55 + M)
    isums = torch.full((M, N, K // 16), -7, dtype=torch.int32, device="cuda")
    nvq.nvq_debug_isums(nvq.NVQ_FMT_NVFP4, nvq.NVQ_PATH_GEMM, c.w, c.q, N, isums)
    ref = oracle.isums_nvfp4(c.codes, c.qh)
    assert (host(isums) == ref).all()
    assert np.abs(ref).max() > 0


def test_gemm_isums_prefill_depth(oracle):
    """The two-term kernel's sums over the full prefill depth K = 5120 (80 stages, 256 x
    256 tiles, every tile split along K on this small grid), 256 tokens."""
    say("debug isums GEMM path M=256 N=512 K=5120")
    torch = torch_dev()
    M, N, K = 256, 512, 5120
    c = NvCase(M, N, K, 5151, outliers=True)
    isums = torch.empty((M, N, K // 16), dtype=torch.int32, device="cuda")
    nvq.nvq_debug_isums(nvq.NVQ_FMT_NVFP4, nvq.NVQ_PATH_GEMM, c.w, c.q, N, isums)
    assert (host(isums) == oracle.isums_nvfp4(c.codes, c.qh)).all()


# ---------------------------------------------------------------------------
# Full workload sizes (sampled columns)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,N,K", list(synth.LAYER))
@pytest.mark.parametrize("kernel", ["mfma", "dot4"])
def test_layer_gemv_full_size(oracle, name, N, K, kernel):
    say(f"layer gemv ({kernel}) {name} N={N} K={K}")
    torch = torch_dev()
    c = NvCase(1, N, K, synth.seed_for("layer", name), w_scale="uniform")
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    fn = nvq.nvq_gemv_nvfp4 if kernel == "mfma" else nvq.nvq_gemv_nvfp4_dot4
    fn(c.w, c.ws, c.q, c.d, y)
    cols = sample_cols(N, 64, N)
    yo, awa = c.oracle_y(oracle, cols=cols)
    check_y(host(y)[:, cols], yo, awa, f"layer {name}")


@pytest.mark.parametrize("name,N,K", list(synth.LAYER))
def test_layer_gemv_fused_full_size(oracle, name, N, K):
    """The layer set through the fused quantization + GEMV, sampled columns."""
    say(f"layer gemv fused {name} N={N} K={K}")
    codes, scales, ws = synth.nvfp4_weights(N, K, synth.seed_for("layer", name), "uniform")
    w = to_dev(nvq.nvq_pack_nvfp4(codes, scales))
    x = synth.activations(1, K, synth.seed_for("layer", "x_" + name))
    y, qk, dk = _fused_run(w, ws, x, N)
    qo, do, _ = oracle.quantize_q8_0(x)
    assert (qk == qo).all() and (dk == do).all()
    cols = sample_cols(N, 64, N + 1)
    yo, awa = oracle.matmul_nvfp4(codes, scales, ws, qo, do, cols=cols)
    check_y(y[:, cols], yo, awa, f"fused layer {name}")


@pytest.mark.parametrize("M", [256, 2048])
def test_prefill_gemm_full_size(oracle, M):
    say(f"prefill gemm M={M} N=17408 K=5120")
    torch = torch_dev()
    N, K = 17408, 5120
    c = NvCase(M, N, K, synth.seed_for("prefill", "w") + M, outliers=True)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemm_nvfp4(c.w, c.ws, c.q, c.d, y)
    cols = sample_cols(N, 24, M)
    yo, awa = c.oracle_y(oracle, cols=cols)
    check_y(host(y)[:, cols], yo, awa, f"prefill M={M}")


@pytest.mark.parametrize("name,N,K", list(synth.LAYER))
def test_batched_decode_m8_full_size(oracle, name, N, K):
    """The layer set at M = 8 (batched decode of the 64-layer stack): gate+up takes the
    many-tile launch (T tiles per block), QKV, O and down the fewer-than-1024-tile one;
    down runs 136 chunks per row."""
    say(f"batched decode M=8 {name} N={N} K={K}")
    torch = torch_dev()
    c = NvCase(8, N, K, synth.seed_for("stack", name), w_scale="uniform")
    y = torch.empty((8, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemv_nvfp4(c.w, c.ws, c.q, c.d, y)
    cols = sample_cols(N, 48, 8)
    yo, awa = c.oracle_y(oracle, cols=cols)
    check_y(host(y)[:, cols], yo, awa, f"M=8 {name}")


def test_batched_decode_m12_down(oracle):
    """Two token groups at the down projection's shape (N = 5120, K = 17408)."""
    say("batched decode M=12 down N=5120 K=17408")
    torch = torch_dev()
    N, K = 5120, 17408
    c = NvCase(12, N, K, synth.seed_for("stack", "down12"), w_scale="uniform")
    y = torch.empty((12, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemv_nvfp4(c.w, c.ws, c.q, c.d, y)
    cols = sample_cols(N, 48, 12)
    yo, awa = c.oracle_y(oracle, cols=cols)
    check_y(host(y)[:, cols], yo, awa, "M=12 down")


@pytest.mark.parametrize("M", [12, 16])
def test_batched_decode_two_groups_full_size(oracle, M):
    """Two token groups over many tiles and chunks: N = 17408 (1088 tiles, 5 per block),
    K = 5120 (40 chunks); M = 16 through the GEMM entry (which sends it here)."""
    say(f"batched decode M={M} N=17408 K=5120")
    torch = torch_dev()
    N, K = 17408, 5120
    c = NvCase(M, N, K, 4100 + M, w_scale="uniform")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    (nvq.nvq_gemv_nvfp4 if M <= nvq.NVQ_GEMV_MAX_M else nvq.nvq_gemm_nvfp4)(c.w, c.ws, c.q, c.d, y)
    cols = sample_cols(N, 48, 9)
    yo, awa = c.oracle_y(oracle, cols=cols)
    check_y(host(y)[:, cols], yo, awa, f"M={M} N=17408")


# ---------------------------------------------------------------------------
# Q4_1
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (1, 33, 96), (4, 70, 160), (16, 64, 32),
                                   (33, 100, 320), (8, 300, 4096), (15, 129, 640), (3, 33, 20480),
                                   (2, 50, 24576), (1, 40, 24576)])
def test_q4_1_small(oracle, M, N, K):
    say(f"q4_1 M={M} N={N} K={K}")
    torch = torch_dev()
    c = Q41Case(M, N, K, 31 + M * N)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    if M <= nvq.NVQ_GEMV_MAX_M:
        nvq.nvq_gemv_q4_1(c.w, c.q, c.d, c.b, y)
    else:
        nvq.nvq_gemm_q4_1(c.w, c.q, c.d, c.b, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"q4_1 M={M} N={N} K={K}")


def test_q4_1_gemm_full_size(oracle):
    say("q4_1 gemm M=512 N=K=4096")
    torch = torch_dev()
    c = Q41Case(512, 4096, 4096, synth.seed_for("q4_1", "w"))
    y = torch.empty((512, 4096), dtype=torch.float32, device="cuda")
    nvq.nvq_gemm_q4_1(c.w, c.q, c.d, c.b, y)
    cols = sample_cols(4096, 48, 3)
    yo, awa = c.oracle_y(oracle, cols=cols)
    check_y(host(y)[:, cols], yo, awa, "q4_1 M=512")


@pytest.mark.parametrize("M,N,K", [(65, 128, 64), (100, 300, 640), (257, 77, 192), (300, 130, 1024),
                                   (96, 64, 96), (128, 40, 4096), (17, 300, 640), (40, 77, 192),
                                   (64, 520, 1024), (50, 64, 96)])
def test_q4_1_gemm_large_m(oracle, M, N, K):
    """M > 16: the integer-MFMA kernel (256 x 64 tiles up to M = 64, 128 x 128 up to
    M = 512, 128 x 256 above; K % 64 == 0; K-split parts on small grids, ragged N and M
    tiles, N % 4 != 0) and the tiled kernel (K = 96)."""
    say(f"q4_1 gemm M={M} N={N} K={K}")
    torch = torch_dev()
    c = Q41Case(M, N, K, 53 + M + N)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemm_q4_1(c.w, c.q, c.d, c.b, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"q4_1 M={M} N={N} K={K}")


def test_q4_1_gemm_full_and_split_tiles(oracle):
    """300 tiles of 128 x 128: 256 whole-K work items plus 44 tiles split along K."""
    say("q4_1 gemm M=300 N=12800 K=256")
    torch = torch_dev()
    M, N, K = 300, 12800, 256
    c = Q41Case(M, N, K, 8181)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemm_q4_1(c.w, c.q, c.d, c.b, y)
    cols = sample_cols(N, 64, 5)
    yo, awa = c.oracle_y(oracle, cols=cols)
    check_y(host(y)[:, cols], yo, awa, "q4_1 M=300 N=12800")


def _q41_extreme_rows(N, K, seed):
    """Q4_1 weights whose rows span the binary16 range: tiny (subnormal d, m), huge
    (|d * 15 + m| near 1e6), all-zero, mixed-sign offsets, and ordinary rows."""
    qw, dw, mw = synth.q4_1_weights(N, K, seed)
    d = dw.view(np.float16).astype(np.float32)
    m = mw.view(np.float16).astype(np.float32)
    d[0], m[0] = 3e-7, -2e-6          # binary16 subnormals
    d[1], m[1] = 65504.0, -65504.0    # largest finite d and m
    d[2], m[2] = 0.0, 0.0             # zero row
    d[3], m[3] = 1e-3, 7.0            # offset far above the code range
    d[4, ::2], m[4, ::2] = 4000.0, 1e-4  # blocks of very different size in one row
    d[5], m[5] = 6e-8, 0.0            # least binary16 magnitude
    return qw, d.astype(np.float16).view(np.uint16), m.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("M,N,K", [(200, 70, 640), (80, 70, 640), (40, 70, 640), (8, 70, 640)])
def test_q4_1_extreme_weight_rows(oracle, M, N, K):
    """Per-row weight magnitudes from 6e-8 to 1e6 in one matrix, through the three
    integer-MFMA GEMM tile shapes (M = 200, 80, 40) and the GEMV (M = 8)."""
    say(f"q4_1 extreme weight rows M={M}")
    torch = torch_dev()
    c = Q41Case(M, N, K, 0, weights=_q41_extreme_rows(N, K, 919), x=synth.activations(M, K, 920))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    (nvq.nvq_gemm_q4_1 if M > nvq.NVQ_GEMV_MAX_M else nvq.nvq_gemv_q4_1)(c.w, c.q, c.d, c.b, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"q4_1 extreme rows M={M}")
    assert (host(y)[:, 2] == 0.0).all()


@pytest.mark.parametrize("M", [300, 100, 48])
def test_q4_1_gemm_split_determinism_and_guard_bands(oracle, M):
    """Two-term Q4_1 kernels with K-split parts: junk workspace on entry,
    bitwise-identical repeats, nothing written outside y."""
    say(f"q4_1 gemm (M={M}, K-split) determinism + guard bands")
    torch = torch_dev()
    N, K = 260, 1024
    c = Q41Case(M, N, K, 4343)
    need = nvq.nvq_gemm_workspace_bytes(nvq.NVQ_FMT_Q4_1, M, N, K)
    assert need > 0
    guard = 4096
    outs = []
    for rep in range(2):
        buf = torch.full((M * N + 2 * guard,), 12345.0, dtype=torch.float32, device="cuda")
        y = buf[guard:guard + M * N].view(M, N)
        ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
        nvq.nvq_gemm_q4_1(c.w, c.q, c.d, c.b, y, workspace=ws)
        torch.cuda.synchronize()
        b = host(buf)
        assert (b[:guard] == 12345.0).all() and (b[guard + M * N:] == 12345.0).all()
        outs.append(b[guard:guard + M * N].copy())
    assert (outs[0].view(np.uint32) == outs[1].view(np.uint32)).all()
    yo, awa = c.oracle_y(oracle, cols=np.arange(0, N, 5))
    check_y(outs[0].reshape(M, N)[:, ::5], yo, awa, "q4_1 split determinism case")


def _large_activations(M, K, seed):
    """Activations that reach past the binary16 range once scaled: blocks with d >= 512
    (the NVFP4 two-term kernel's second pass; the Q4_1 integer-MFMA kernel applies d in
    float32), one token with every block that large, one
    block just below the threshold (|d * q| near 60000, main pass), the rest N(0, 1)."""
    x = synth.activations(M, K, seed)
    x[5, 3] = 1.0e6                                        # d ~ 7874
    x[1, 40:44] = [3.0e5, -2.0e5, 1.0e5, 7.0]              # d ~ 2362
    x[M - 1, 0:32] *= 6.0e4 / np.abs(x[M - 1, 0:32]).max()  # d ~ 472
    x[2, :] *= 1.0e5                                       # every block of token 2
    x[M // 2, K - 32:] = 8.0e6                             # d ~ 63000, the last block of a row
    return x


@pytest.mark.parametrize("M", [200, 96, 24])
def test_q4_1_gemm_activation_range(oracle, M):
    """Q4_1 GEMM (M > 16, the integer-MFMA kernel): activations whose scaled values pass
    the binary16 range (blocks with d >= 512), every tile height and K-split parts
    included."""
    say(f"q4_1 gemm (M={M}) large activations")
    torch = torch_dev()
    N, K = 300, 640
    c = Q41Case(M, N, K, 79, x=_large_activations(M, K, 80))
    assert ((c.dh[2] & 0x7FFF) >= 0x6000).all() and (c.dh[M - 1, 0] & 0x7FFF) < 0x6000
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemm_q4_1(c.w, c.q, c.d, c.b, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"q4_1 large activations M={M}")


def _q41_cancelling_rows(N, K, seed):
    """Q4_1 blocks whose line d * c + m crosses zero at a code z0: m is -d * z0 moved one
    binary16 ulp toward zero, and every fourth code is z0, so those weights are a few
    ulps of d * z0 -- thousands of times smaller than either part."""
    qw, dw, _ = synth.q4_1_weights(N, K, seed)
    rng = np.random.default_rng(seed + 1)
    z0 = rng.integers(0, 16, (N, K // 32))
    d = dw.view(np.float16).astype(np.float32)
    mb = (-(d * z0)).astype(np.float16).view(np.uint16)
    mb = np.where((z0 > 0) & ((mb & 0x7FFF) > 0), mb - 1, mb).astype(np.uint16)
    qw = qw.copy()
    qw.reshape(N, K // 32, 32)[:, :, ::4] = z0[:, :, None]
    return qw, dw, mb


@pytest.mark.parametrize("M", [200, 100, 40])
def test_q4_1_gemm_cancelling_weights(oracle, M):
    """Weights far smaller than their scale and offset parts, met by activation blocks
    with a single nonzero code on exactly those weights: the GEMM (every tile height)
    stays within the bound relative to sum |w * a| (the integer-MFMA kernel stages each
    block's codes shifted to the line's root; a plain scale-and-offset split of these
    blocks misses the bound on about half of the outputs)."""
    say(f"q4_1 gemm (M={M}) cancelling weights")
    torch = torch_dev()
    N, K = 300, 640
    c = Q41Case(M, N, K, 0, weights=_q41_cancelling_rows(N, K, 4242), x=spike_activations(M, K, 4243))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemm_q4_1(c.w, c.q, c.d, c.b, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"q4_1 cancelling weights M={M}")


@pytest.mark.parametrize("fmt,M,N", [("nvfp4", 300, 2560), ("nvfp4", 100, 5120), ("nvfp4", 40, 5120),
                                      ("q4_1", 300, 2560), ("q4_1", 100, 2560), ("q4_1", 40, 5120)])
def test_gemm_ksplit_many_parts(oracle, fmt, M, N):
    """Tiles of 20 stages in a last round far short of the compute units, each split
    into several K parts (up to 12) summed in order; repeat calls bitwise identical.
    One shape per token-tile height and format."""
    say(f"{fmt} gemm K-split parts M={M} N={N}")
    torch = torch_dev()
    K = 1280
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    cols = sample_cols(N, 96, M + N)
    if fmt == "nvfp4":
        c = NvCase(M, N, K, 7100 + M, w_scale=0.75)
        nvq.nvq_gemm_nvfp4(c.w, c.ws, c.q, c.d, y)
        first = host(y).copy()
        nvq.nvq_gemm_nvfp4(c.w, c.ws, c.q, c.d, y)
    else:
        c = Q41Case(M, N, K, 7200 + M)
        nvq.nvq_gemm_q4_1(c.w, c.q, c.d, c.b, y)
        first = host(y).copy()
        nvq.nvq_gemm_q4_1(c.w, c.q, c.d, c.b, y)
    assert (host(y).view(np.uint32) == first.view(np.uint32)).all()
    yo, awa = c.oracle_y(oracle, cols=cols)
    check_y(first[:, cols], yo, awa, f"{fmt} tail crossing M={M} N={N}")


@pytest.mark.parametrize("M", [3, 12, 16, 20, 100, 300])
def test_single_output_row(oracle, M):
    """N = 1 (one weight row, every tile ragged) through each NVFP4 and Q4_1 dispatch,
    at the shortest and a long K."""
    say(f"N = 1, M={M}")
    torch = torch_dev()
    for K in (64, 5120):
        c = NvCase(M, 1, K, 5000 + M + K)
        y = torch.empty((M, 1), dtype=torch.float32, device="cuda")
        (nvq.nvq_gemv_nvfp4 if M <= nvq.NVQ_GEMV_MAX_M else nvq.nvq_gemm_nvfp4)(c.w, c.ws, c.q, c.d, y)
        yo, awa = c.oracle_y(oracle)
        check_y(host(y), yo, awa, f"nvfp4 N=1 M={M} K={K}")
        c4 = Q41Case(M, 1, K, 6000 + M + K)
        y4 = torch.empty((M, 1), dtype=torch.float32, device="cuda")
        (nvq.nvq_gemv_q4_1 if M <= nvq.NVQ_GEMV_MAX_M else nvq.nvq_gemm_q4_1)(c4.w, c4.q, c4.d, c4.b, y4)
        yo4, awa4 = c4.oracle_y(oracle)
        check_y(host(y4), yo4, awa4, f"q4_1 N=1 M={M} K={K}")


@pytest.mark.parametrize("path", [nvq.NVQ_PATH_GEMV, nvq.NVQ_PATH_GEMM])
def test_q4_1_isums_bit_exact(oracle, path):
    say(f"q4_1 isums path={path}")
    torch = torch_dev()
    for M, N, K in [(1, 37, 96), (3, 70, 256)]:
        c = Q41Case(M, N, K, 71 + N)
        isums = torch.full((M, N, K // 16), -7, dtype=torch.int32, device="cuda")
        nvq.nvq_debug_isums(nvq.NVQ_FMT_Q4_1, path, c.w, c.q, N, isums)
        assert (host(isums) == oracle.isums_q4_1(c.qw, c.qh)).all(), (M, N, K)


# Q4_1 GEMM dispatch for M > 16: the integer-MFMA kernel (K % 64 == 0; its three tile
# shapes, K-split parts on small grids) or the tiled kernel (K = 96).
@pytest.mark.parametrize("M,N,K", [(17, 300, 640), (40, 77, 192), (64, 520, 1024), (100, 130, 1024),
                                   (128, 40, 4096), (200, 70, 640), (512, 256, 4096), (20, 33, 96)])
def test_q4_1_gemm_isums_bit_exact(oracle, M, N, K):
    say(f"q4_1 isums GEMM path M={M} N={N} K={K}")
    torch = torch_dev()
    c = Q41Case(M, N, K, 83 + M + N)
    isums = torch.full((M, N, K // 16), -7, dtype=torch.int32, device="cuda")
    nvq.nvq_debug_isums(nvq.NVQ_FMT_Q4_1, nvq.NVQ_PATH_GEMM, c.w, c.q, N, isums)
    ref = oracle.isums_q4_1(c.qw, c.qh)
    assert (host(isums) == ref).all()
    assert np.abs(ref).max() > 0


# ---------------------------------------------------------------------------
# Contract: determinism, guard bands, per-tensor scale, error codes on device
# ---------------------------------------------------------------------------

def test_determinism_and_guard_bands(oracle):
    say("determinism + guard bands")
    torch = torch_dev()
    M, N, K = 40, 200, 640
    c = NvCase(M, N, K, 2024, w_scale=0.75)
    guard = 1024
    outs = []
    for rep in range(2):
        buf = torch.full((M * N + 2 * guard,), 12345.0, dtype=torch.float32, device="cuda")
        y = buf[guard:guard + M * N].view(M, N)
        nvq.nvq_gemm_nvfp4(c.w, c.ws, c.q, c.d, y)
        torch.cuda.synchronize()
        b = host(buf)
        assert (b[:guard] == 12345.0).all() and (b[guard + M * N:] == 12345.0).all()
        outs.append(b[guard:guard + M * N].copy())
    assert (outs[0].view(np.uint32) == outs[1].view(np.uint32)).all()
    y1 = torch.empty((1, N), dtype=torch.float32, device="cuda")
    y2 = torch.empty((1, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemv_nvfp4(c.w, 1.0, c.q[:1], c.d[:1], y1)
    nvq.nvq_gemv_nvfp4(c.w, 4.0, c.q[:1], c.d[:1], y2)
    assert (host(y2) == 4.0 * host(y1)).all()


def test_side_stream_and_graph_replay():
    """Every compute entry on a non-default stream, then the same sequence captured in a
    HIP graph and replayed three times, with eager work on the inputs between replays:
    each replay equals the eager run bit for bit (no memset nodes are involved)."""
    say("side stream + graph replay")
    torch = torch_dev()
    N, K = 300, 640
    codes, scales, ws = synth.nvfp4_weights(N, K, 61, "uniform")
    w = to_dev(nvq.nvq_pack_nvfp4(codes, scales))
    experts = [synth.nvfp4_weights(N, K, 62 + e, "uniform") for e in range(3)]
    wr = to_dev(np.concatenate([nvq.nvq_pack_nvfp4(c, s) for c, s, _ in experts]))
    wsc = torch.from_numpy(np.array([v for _, _, v in experts], np.float32)).cuda()
    ids = torch.from_numpy(np.array([[2, 0]], np.int32)).cuda()
    qw, dw, mw = synth.q4_1_weights(N, K, 63)
    w41 = to_dev(nvq.nvq_pack_q4_1(qw, dw, mw))
    # every dispatch: decode, batched (one and two column groups), the three GEMM tile
    # heights with K-split parts; Q4_1 GEMV (one and several tokens) and GEMM
    Ms = (1, 8, 12, 40, 80, 200)
    xs = {M: to_dev(synth.activations(M, K, 70 + M, outliers=True)) for M in Ms}
    qd = {M: (torch.empty((M, K), dtype=torch.int8, device="cuda"),
              torch.empty((M, K // 32), dtype=torch.int16, device="cuda"),
              torch.empty((M, K // 16), dtype=torch.int16, device="cuda")) for M in xs}
    ys = {M: torch.empty((M, N), dtype=torch.float32, device="cuda") for M in xs}
    ys41 = {M: torch.empty((M, N), dtype=torch.float32, device="cuda") for M in xs}
    yr = torch.empty((1, 2, N), dtype=torch.float32, device="cuda")
    yf = torch.empty((1, N), dtype=torch.float32, device="cuda")
    Nk, Kk = 17408, 256
    ck, sk, wsk = synth.nvfp4_weights(Nk, Kk, 64, "uniform")
    wk = to_dev(nvq.nvq_pack_nvfp4(ck, sk))
    xk = to_dev(synth.activations(64, Kk, 65))
    qk = torch.empty((64, Kk), dtype=torch.int8, device="cuda")
    dk = torch.empty((64, Kk // 32), dtype=torch.int16, device="cuda")
    yk = torch.empty((64, Nk), dtype=torch.float32, device="cuda")
    # Q4_K (K % 256 == 0): GEMV at M = 1 and the integer-MFMA GEMM with K-split parts at M = 100
    K4 = 768
    w4k = to_dev(nvq.nvq_pack_q4_k(*synth.q4_k_weights(N, K4, 66)))
    x4k = {M: to_dev(synth.activations(M, K4, 67 + M)) for M in (1, 100)}
    qd4k = {M: (torch.empty((M, K4), dtype=torch.int8, device="cuda"),
                torch.empty((M, K4 // 32), dtype=torch.int16, device="cuda"),
                torch.empty((M, K4 // 16), dtype=torch.int16, device="cuda")) for M in x4k}
    y4k = {M: torch.empty((M, N), dtype=torch.float32, device="cuda") for M in x4k}
    qwx, lsx, ddx, tabx = synth.iq4_xs_weights(N, K4, 68)
    wx = to_dev(nvq.nvq_pack_iq4_xs(qwx, lsx, ddx))
    yx = {M: torch.empty((M, N), dtype=torch.float32, device="cuda") for M in x4k}
    w5k = to_dev(nvq.nvq_pack_q5_k(*synth.q5_k_weights(N, K4, 69)))
    w6k = to_dev(nvq.nvq_pack_q6_k(*synth.q6_k_weights(N, K4, 70)))
    y5k = {M: torch.empty((M, N), dtype=torch.float32, device="cuda") for M in x4k}
    y6k = {M: torch.empty((M, N), dtype=torch.float32, device="cuda") for M in x4k}
    need = max([nvq.nvq_gemm_workspace_bytes(f, M, N, K) for f in (nvq.NVQ_FMT_NVFP4, nvq.NVQ_FMT_Q4_1) for M in Ms]
               + [nvq.nvq_gemm_workspace_bytes(nvq.NVQ_FMT_NVFP4, 64, Nk, Kk),
                  nvq.nvq_gemm_workspace_bytes(nvq.NVQ_FMT_Q4_K, 100, N, K4)])
    wsp = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()

    def seq():
        for M, x in xs.items():
            q, d, b = qd[M]
            nvq.nvq_quantize_act_q8_0(x, q, d, b)
            if M < 16:
                nvq.nvq_gemv_nvfp4(w, ws, q, d, ys[M])
                nvq.nvq_gemv_q4_1(w41, q, d, b, ys41[M])
            else:
                nvq.nvq_gemm_nvfp4(w, ws, q, d, ys[M], workspace=wsp)
                nvq.nvq_gemm_q4_1(w41, q, d, b, ys41[M], workspace=wsp)
        nvq.nvq_gemv_nvfp4_routed(wr, wsc, ids, qd[1][0], qd[1][1], yr)
        nvq.nvq_gemv_nvfp4_fused(w, ws, xs[1], yf)
        # 68 tiles of 256 x 64 in 3 K parts (a prefill-like grid on few stages)
        nvq.nvq_quantize_act_q8_0(xk, qk, dk)
        nvq.nvq_gemm_nvfp4(wk, ws, qk, dk, yk, workspace=wsp)
        for M, x in x4k.items():
            q, d, b = qd4k[M]
            nvq.nvq_quantize_act_q8_0(x, q, d, b)
            (nvq.nvq_gemv_q4_k if M == 1 else nvq.nvq_gemm_q4_k)(w4k, q, d, b, y4k[M], **({} if M == 1 else {"workspace": wsp}))
            (nvq.nvq_gemv_iq4_xs if M == 1 else nvq.nvq_gemm_iq4_xs)(wx, tabx, q, d, yx[M], **({} if M == 1 else {"workspace": wsp}))
            (nvq.nvq_gemv_q5_k if M == 1 else nvq.nvq_gemm_q5_k)(w5k, q, d, b, y5k[M], **({} if M == 1 else {"workspace": wsp}))
            (nvq.nvq_gemv_q6_k if M == 1 else nvq.nvq_gemm_q6_k)(w6k, q, d, y6k[M], **({} if M == 1 else {"workspace": wsp}))

    def snapshot():
        return ([host(ys[M]).copy() for M in xs] + [host(ys41[M]).copy() for M in xs] + [host(yr).copy()]
                + [host(yf).copy(), host(yk).copy()] + [host(y4k[M]).copy() for M in x4k]
                + [host(yx[M]).copy() for M in x4k] + [host(y5k[M]).copy() for M in x4k]
                + [host(y6k[M]).copy() for M in x4k])

    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        seq()
    s.synchronize()
    eager = snapshot()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            seq()
    s.synchronize()
    saved = {M: x.clone() for M, x in xs.items()}
    for rep in range(3):
        for M in xs:                      # eager work between replays, then inputs restored
            xs[M].mul_(-1.0)
        xk.mul_(-1.0)
        for x in x4k.values():
            x.mul_(-1.0)
        seq()
        torch.cuda.synchronize()
        for M in xs:
            xs[M].copy_(saved[M])
        xk.mul_(-1.0)
        for x in x4k.values():
            x.mul_(-1.0)
        for y in (list(ys.values()) + list(ys41.values()) + [yr, yf, yk] + list(y4k.values()) + list(yx.values())
                  + list(y5k.values()) + list(y6k.values())):
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(snapshot(), eager):
            assert (a.view(np.uint32) == b.view(np.uint32)).all(), f"replay {rep}"


@pytest.mark.parametrize("M", [300, 100, 40])
def test_gemm_split_kernel_determinism_and_guard_bands(oracle, M):
    """Two-term GEMM (all three token-tile heights) with K-split parts:
    bitwise-identical repeats, nothing written outside y."""
    say(f"gemm (M={M}, K-split) determinism + guard bands")
    torch = torch_dev()
    N, K = 520, 1024
    c = NvCase(M, N, K, 4242, w_scale=1.25, outliers=True)
    guard = 4096
    outs = []
    for rep in range(2):
        buf = torch.full((M * N + 2 * guard,), 12345.0, dtype=torch.float32, device="cuda")
        y = buf[guard:guard + M * N].view(M, N)
        ws = torch.full((nvq.nvq_gemm_workspace_bytes(nvq.NVQ_FMT_NVFP4, M, N, K),), 0x7F, dtype=torch.uint8,
                        device="cuda")  # junk on entry must not matter
        nvq.nvq_gemm_nvfp4(c.w, c.ws, c.q, c.d, y, workspace=ws)
        torch.cuda.synchronize()
        b = host(buf)
        assert (b[:guard] == 12345.0).all() and (b[guard + M * N:] == 12345.0).all()
        outs.append(b[guard:guard + M * N].copy())
    assert (outs[0].view(np.uint32) == outs[1].view(np.uint32)).all()
    yo, awa = c.oracle_y(oracle, cols=np.arange(0, N, 7))
    check_y(outs[0].reshape(M, N)[:, ::7], yo, awa, "gemm split determinism case")


@pytest.mark.parametrize("M,N", [(200, 300), (96, 300), (24, 300), (16, 300), (12, 300), (12, 17627),
                                 (16, 16379)])
def test_gemm_split_kernel_activation_range(oracle, M, N):
    """NVFP4 GEMM entry: activations whose scaled values pass the binary16 range
    (blocks with d >= 512) are exact through the second pass of the two-term kernel
    (M > 16: every tile height, K-split parts on this small grid) and of the batched
    kernel (M = 16 through the GEMM entry, M = 12 through the GEMV entry; both launch
    shapes: 2 tiles per block below 1024 tiles, 4 or 5 from 1024 up)."""
    say(f"gemm (M={M}) large activations N={N}")
    torch = torch_dev()
    K = 640
    c = NvCase(M, N, K, 77, w_scale=1.5)
    c.x = _large_activations(M, K, 78)
    c.q, c.d, c.b = quantize_gpu(c.x)
    c.qh, c.dh = host(c.q), host(c.d).view(np.uint16)
    assert ((c.dh[2] & 0x7FFF) >= 0x6000).all() and (c.dh[M - 1, 0] & 0x7FFF) < 0x6000
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    (nvq.nvq_gemv_nvfp4 if M <= nvq.NVQ_GEMV_MAX_M else nvq.nvq_gemm_nvfp4)(c.w, c.ws, c.q, c.d, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"large activations M={M}")


def test_gemm_large_activations_prefill_shape(oracle):
    """The prefill shape (M = 2048, N = 17408, K = 5120: whole tiles and split tiles) with
    a few large-activation tokens, sampled output columns."""
    say("prefill gemm M=2048 with large activations")
    torch = torch_dev()
    M, N, K = 2048, 17408, 5120
    c = NvCase(M, N, K, synth.seed_for("prefill", "big"), outliers=True)
    x = c.x
    x[7, 100] = 2.0e6                    # m-tile 0
    x[1500, :64] *= 3.0e4                # m-tile 5, two blocks
    x[2047, 5000:5090] = -9.0e5          # last token, blocks near the end of K
    c.q, c.d, c.b = quantize_gpu(x)
    c.qh, c.dh = host(c.q), host(c.d).view(np.uint16)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemm_nvfp4(c.w, c.ws, c.q, c.d, y)
    cols = sample_cols(N, 24, 77)
    yo, awa = c.oracle_y(oracle, cols=cols)
    check_y(host(y)[:, cols], yo, awa, "prefill with large activations")


def _experts(E, N, K, seed):
    """E seeded NVFP4 experts: logical codes/scales [E, N, K], per-expert scales, and
    the packed table on the GPU (expert e at e * nvq_nvfp4_weight_bytes(N, K))."""
    torch = torch_dev()
    ws = [synth.nvfp4_weights(N, K, seed + e, "uniform") for e in range(E)]
    codes = np.stack([c for c, _, _ in ws])
    scales = np.stack([s for _, s, _ in ws])
    wsc = np.array([v for _, _, v in ws], np.float32)
    w = to_dev(np.concatenate([nvq.nvq_pack_nvfp4(c, s) for c, s, _ in ws]))
    return codes, scales, wsc, w, torch.from_numpy(wsc).cuda()


@pytest.mark.parametrize("E,A,M,N,K", [(5, 2, 3, 100, 320), (3, 4, 2, 33, 640), (8, 6, 1, 300, 2048),
                                       (4, 3, 1, 40, 17408)])
def test_gemv_routed(oracle, E, A, M, N, K):
    """Expert-routed GEMV: every (token, slot) against the oracle's routed product,
    with repeated experts; an out-of-range id gives a NaN row and leaves the others."""
    say(f"routed gemv E={E} A={A} M={M} N={N} K={K}")
    torch = torch_dev()
    codes, scales, wsc, w, wsc_d = _experts(E, N, K, 700 + N)
    ids = synth.rng(701 + N).integers(0, E, (M, A)).astype(np.int32)
    ids[0, 0] = ids[0, A - 1] if A > 1 else ids[0, 0]       # one repeated expert
    if M > 1:
        ids[M - 1, A - 1] = E                                  # out of range
    x = synth.activations(M, K, 702 + N)
    q, d, _ = quantize_gpu(x)
    y = torch.full((M, A, N), 7.0, dtype=torch.float32, device="cuda")
    nvq.nvq_gemv_nvfp4_routed(w, wsc_d, torch.from_numpy(ids).cuda(), q, d, y)
    yo, awa = oracle.matmul_nvfp4_routed(codes, scales, wsc, ids, host(q), host(d).view(np.uint16))
    yh = host(y)
    bad = (ids < 0) | (ids >= E)
    assert np.isnan(yh[bad]).all() and np.isnan(yo[bad]).all()
    check_y(yh[~bad], yo[~bad], awa[~bad], f"routed E={E} A={A} M={M} N={N} K={K}")


def test_gemv_routed_expert_shape(oracle):
    """The routed step at the expert shape N = K = 2048, 6 active of 16 experts, two
    tokens, sampled output columns."""
    say("routed gemv at the expert shape")
    torch = torch_dev()
    E, A, M, N, K = 16, 6, 2, 2048, 2048
    codes, scales, wsc, w, wsc_d = _experts(E, N, K, synth.seed_for("moe", "w"))
    ids = synth.expert_ids(M, A, E, synth.seed_for("moe", "ids"))
    x = synth.activations(M, K, synth.seed_for("moe", "x"))
    q, d, _ = quantize_gpu(x)
    y = torch.empty((M, A, N), dtype=torch.float32, device="cuda")
    nvq.nvq_gemv_nvfp4_routed(w, wsc_d, torch.from_numpy(ids).cuda(), q, d, y)
    cols = sample_cols(N, 40, 3)
    yo, awa = oracle.matmul_nvfp4_routed(codes, scales, wsc, ids, host(q), host(d).view(np.uint16), cols=cols)
    check_y(host(y)[:, :, cols].reshape(M * A, -1), yo.reshape(M * A, -1), awa.reshape(M * A, -1),
            "routed expert shape")


@pytest.mark.parametrize("K", [65536, 98304])
def test_gemv_long_rows(oracle, K):
    """K = 65536 keeps the decode GEMV's activation table in LDS; K = 98304 does not
    and takes the tiled kernel instead (both must agree with the oracle)."""
    say(f"gemv long row N=40 K={K}")
    torch = torch_dev()
    c = NvCase(1, 40, K, 31 + K // 1024)
    y = torch.empty((1, 40), dtype=torch.float32, device="cuda")
    nvq.nvq_gemv_nvfp4(c.w, c.ws, c.q, c.d, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"gemv K={K}")


@pytest.mark.parametrize("M", [1, 8, 100])
def test_zero_weights_give_exact_zero(M):
    """Codes 0 and 8 (+0, -0) only: every output is exactly 0 on every path."""
    say(f"zero weights M={M}")
    torch = torch_dev()
    N, K = 70, 640
    codes, scales, ws = synth.nvfp4_weights(N, K, 5)
    codes = (codes & 8).astype(np.uint8)  # 0 or 8
    w = to_dev(nvq.nvq_pack_nvfp4(codes, scales))
    q, d, _ = quantize_gpu(synth.activations(M, K, 6, outliers=True))
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    (nvq.nvq_gemv_nvfp4 if M <= 15 else nvq.nvq_gemm_nvfp4)(w, float(ws), q, d, y)
    yh = host(y)
    assert (yh == 0.0).all()


@pytest.mark.parametrize("M", [1, 5, 90])
def test_subnormal_ue4m3_scales(oracle, M):
    """UE4M3 bytes 0x01..0x07 (M * 2^-9) mixed with normal scales."""
    say(f"subnormal UE4M3 scales M={M}")
    torch = torch_dev()
    N, K = 50, 384
    codes, scales, ws = synth.nvfp4_weights(N, K, 9)
    r = np.random.Generator(np.random.PCG64(10))
    sub = r.random(scales.shape) < 0.5
    scales = np.where(sub, r.integers(1, 8, scales.shape), scales).astype(np.uint8)
    c = NvCase(M, N, K, 11)
    c.codes, c.scales, c.ws = codes, scales, ws
    c.w = to_dev(nvq.nvq_pack_nvfp4(codes, scales))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    (nvq.nvq_gemv_nvfp4 if M <= 15 else nvq.nvq_gemm_nvfp4)(c.w, c.ws, c.q, c.d, y)
    yo, awa = c.oracle_y(oracle)
    check_y(host(y), yo, awa, f"subnormal scales M={M}")


@pytest.mark.parametrize("M", [1, 5, 12, 40, 300])
def test_every_ue4m3_byte(oracle, M):
    """Row n of the weights uses the single UE4M3 byte n (0x00 .. 0x7E, every valid byte,
    subnormals included) for all its scales, so a wrong decode of any byte in any path
    shows in that row alone."""
    say(f"every UE4M3 byte M={M}")
    torch = torch_dev()
    N, K = 127, 256
    codes, _, ws = synth.nvfp4_weights(N, K, 21)
    scales = np.repeat(np.arange(N, dtype=np.uint8)[:, None], K // 16, axis=1)
    c = NvCase(M, N, K, 22)
    c.codes, c.scales, c.ws = codes, scales, ws
    c.w = to_dev(nvq.nvq_pack_nvfp4(codes, scales))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    (nvq.nvq_gemv_nvfp4 if M <= 15 else nvq.nvq_gemm_nvfp4)(c.w, c.ws, c.q, c.d, y)
    yo, awa = c.oracle_y(oracle)
    yh = host(y)
    assert (yh[:, 0] == 0.0).all()  # byte 0x00: scale 0
    check_y(yh, yo, awa, f"every UE4M3 byte M={M}")


def test_validation_leaves_output_untouched():
    torch = torch_dev()
    y = torch.full((16, 64), 7.0, dtype=torch.float32, device="cuda")
    w = torch.zeros(nvq.nvq_nvfp4_weight_bytes(64, 128), dtype=torch.uint8, device="cuda")
    q = torch.zeros((16, 96), dtype=torch.int8, device="cuda")
    d = torch.zeros((16, 3), dtype=torch.int16, device="cuda")
    with pytest.raises(nvq.NvqError) as e:
        nvq.lib()  # binding-level shape checks pass; the C layer rejects K % 64
        st = nvq.lib().nvq_gemm_nvfp4(w.data_ptr(), 1.0, q.data_ptr(), d.data_ptr(), 16, 64, 96,
                                      y.data_ptr(), None, 0, None)
        raise nvq.NvqError(st, "gemm", nvq.last_error())
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert (host(y) == 7.0).all()
