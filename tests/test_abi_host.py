"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, the sizes and packers follow the documented layout, and every
argument error is reported before any HIP call (so these run on a CPU host)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import gemm_q8_act_amd as nvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvq.h")


def declared_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvq_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_binding_exports():
    assert declared_symbols() == sorted(nvq.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = nvq.lib()
    for name in declared_symbols():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", nvq.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (nvq_[a-z0-9_]+)\b", out))
    assert set(declared_symbols()) <= exported


def test_library_has_only_gfx950_code(tmp_path):
    fb = tmp_path / "fatbin.bin"
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", nvq.LIB_PATH, str(fb)], check=True)
    out = subprocess.run(["/opt/rocm/llvm/bin/clang-offload-bundler", "--list", "--type=o",
                          f"--input={fb}"], capture_output=True, text=True, check=True)
    targets = [t for t in out.stdout.split() if "amdgcn" in t]
    assert targets and all(t.endswith("gfx950") for t in targets), targets


def test_sizes():
    assert nvq.nvq_nvfp4_weight_bytes(4864, 896) == 4864 * 896 * 9 // 16
    assert nvq.nvq_nvfp4_weight_bytes(34816, 5120) == 34816 * 5120 * 9 // 16
    assert nvq.nvq_nvfp4_weight_bytes(7, 64) == 16 * 128 * 9 // 16      # padded to a 16 x 128 tile
    assert nvq.nvq_nvfp4_weight_bytes(17, 192) == 32 * 256 * 9 // 16
    assert nvq.nvq_nvfp4_weight_bytes(7, 96) == 0          # K % 64 != 0
    assert nvq.nvq_nvfp4_weight_bytes(0, 64) == 0
    assert nvq.nvq_q4_1_weight_bytes(4096, 4096) == 4096 * 4096 * 5 // 8
    assert nvq.nvq_q4_1_weight_bytes(3, 32) == 3 * 20
    assert nvq.nvq_q4_1_weight_bytes(3, 48) == 0
    # K-split workspace of the two-term GEMM (M > 16): fp32 partial tiles (one per
    # 512-thread work item: 256 x 256 tiles with 128 accumulators per thread for
    # M > 128, 256 x 128 with 64 for M <= 128, 256 x 64 with 32 for M <= 64), for the
    # tiles of an incomplete last round over 256 compute units, split up to 16 ways (at
    # most one per 64-k stage)
    tile_bytes, m128_bytes, mid_bytes = 512 * 128 * 4, 512 * 64 * 4, 512 * 32 * 4
    ws = nvq.nvq_gemm_workspace_bytes
    assert ws(nvq.NVQ_FMT_NVFP4, 2048, 17408, 5120) == 32 * 8 * tile_bytes      # 544 tiles: 32 left over
    assert ws(nvq.NVQ_FMT_NVFP4, 256, 17408, 5120) == 68 * 3 * tile_bytes       # 68 tiles, 256 // 68 = 3
    assert ws(nvq.NVQ_FMT_NVFP4, 100, 8, 640) == 1 * 10 * m128_bytes            # 1 tile, 10 stages
    assert ws(nvq.NVQ_FMT_NVFP4, 100, 8, 192) == 1 * 3 * m128_bytes             # split <= stages
    assert ws(nvq.NVQ_FMT_NVFP4, 200, 8, 640) == 1 * 10 * tile_bytes
    assert ws(nvq.NVQ_FMT_NVFP4, 256, 4096, 4096) == 16 * 16 * tile_bytes       # 16 tiles: split 16 ways
    assert ws(nvq.NVQ_FMT_NVFP4, 65, 33, 64) == 0                               # one stage: no split
    assert ws(nvq.NVQ_FMT_NVFP4, 4096, 4096, 1024) == 0                         # 256 tiles: full rounds
    assert ws(nvq.NVQ_FMT_NVFP4, 64, 17408, 5120) == 68 * 3 * mid_bytes         # 256 x 64 tiles
    assert ws(nvq.NVQ_FMT_NVFP4, 17, 300, 640) == 2 * 10 * mid_bytes
    assert ws(nvq.NVQ_FMT_NVFP4, 16, 17408, 5120) == 0                          # M <= 16: batched GEMV
    # Q4_1, split up to 16 ways: M > 128 in 128 x 256 tiles with 64 accumulators per
    # thread, 64 < M <= 128 in 128 x 128 tiles and 16 < M <= 64 in 256 x 64 tiles with 32
    q41_tile, q41_mid = 512 * 64 * 4, 512 * 32 * 4
    assert ws(nvq.NVQ_FMT_Q4_1, 2048, 4096, 4096) == 0                          # 256 tiles: full rounds
    assert ws(nvq.NVQ_FMT_Q4_1, 512, 4096, 4096) == 64 * 4 * q41_tile           # 64 tiles, 256 // 64 = 4
    assert ws(nvq.NVQ_FMT_Q4_1, 300, 19200, 256) == 44 * 4 * q41_tile           # 300 tiles: 44 left, 4 stages
    assert ws(nvq.NVQ_FMT_Q4_1, 100, 8, 640) == 1 * 10 * q41_mid                # split <= stages
    assert ws(nvq.NVQ_FMT_Q4_1, 200, 8, 640) == 1 * 10 * q41_tile
    assert ws(nvq.NVQ_FMT_Q4_1, 64, 4096, 4096) == 16 * 16 * q41_mid            # 16 tiles of 256 rows
    assert ws(nvq.NVQ_FMT_Q4_1, 17, 8, 64) == 0                                 # one stage: no split
    assert ws(nvq.NVQ_FMT_Q4_1, 16, 4096, 4096) == 0                            # M <= 16: tiled kernel
    assert ws(nvq.NVQ_FMT_Q4_1, 100, 8, 96) == 0                                # K % 64 != 0: tiled kernel
    assert ws(nvq.NVQ_FMT_NVFP4, 2048, 17408, 96) == 0                          # invalid K


def unpack_tiled(buf, N, K):
    """Inverse of the tile-interleaved layout, written from the header's description."""
    Np, Kp = -(-N // 16) * 16, -(-K // 128) * 128
    T, C = Np // 16, Kp // 128
    codes = np.zeros((Np, Kp), np.uint8)
    scales = np.zeros((Np, Kp // 16), np.uint8)
    cb = buf[: T * C * 1024].reshape(T, C, 64, 16)
    sb = buf[T * C * 1024: T * C * 1152].reshape(T, C, 64, 2)
    for t in range(T):
        for c in range(C):
            for l in range(64):
                n, g = l % 16, l // 16
                k0 = 128 * c + 32 * g
                codes[16 * t + n, k0:k0 + 32:2] = cb[t, c, l] & 0xF
                codes[16 * t + n, k0 + 1:k0 + 32:2] = cb[t, c, l] >> 4
                scales[16 * t + n, k0 // 16: k0 // 16 + 2] = sb[t, c, l]
    return codes, scales


@pytest.mark.parametrize("N,K", [(3, 128), (16, 256), (37, 320), (5, 64)])
def test_pack_nvfp4_layout(N, K):
    r = np.random.Generator(np.random.PCG64(5 + N))
    codes = r.integers(0, 16, (N, K), dtype=np.uint8)
    scales = r.integers(0, 0x7F, (N, K // 16), dtype=np.uint8)
    buf = nvq.nvq_pack_nvfp4(codes, scales)
    assert buf.size == nvq.nvq_nvfp4_weight_bytes(N, K)
    c2, s2 = unpack_tiled(buf, N, K)
    assert (c2[:N, :K] == codes).all() and (s2[:N, :K // 16] == scales).all()
    assert not c2[N:].any() and not c2[:, K:].any()           # zero padding
    assert not s2[N:].any() and not s2[:, K // 16:].any()


def test_pack_q4_1_layout():
    r = np.random.Generator(np.random.PCG64(6))
    N, K = 2, 96
    q = r.integers(0, 16, (N, K), dtype=np.uint8)
    d = r.integers(0, 65536, (N, K // 32), dtype=np.uint32).astype(np.uint16)
    m = r.integers(0, 65536, (N, K // 32), dtype=np.uint32).astype(np.uint16)
    buf = nvq.nvq_pack_q4_1(q, d, m)
    assert buf.size == N * K * 5 // 8
    cb = buf[: N * K // 2].reshape(N, K // 2)
    assert (cb & 0xF == q[:, 0::2]).all() and (cb >> 4 == q[:, 1::2]).all()
    pairs = buf[N * K // 2:].view(np.uint32).reshape(N, K // 32)
    assert ((pairs & 0xFFFF) == d).all() and ((pairs >> 16) == m).all()


@pytest.mark.parametrize("bad", ["code16", "scale_bit7", "scale_nan"])
def test_pack_nvfp4_rejects_invalid(bad):
    codes = np.zeros((1, 64), np.uint8)
    scales = np.full((1, 4), 0x38, np.uint8)
    if bad == "code16":
        codes[0, 5] = 16
    elif bad == "scale_bit7":
        scales[0, 2] = 0xB8
    else:
        scales[0, 1] = 0x7F
    with pytest.raises(nvq.NvqError) as e:
        nvq.nvq_pack_nvfp4(codes, scales)
    assert e.value.status == -3


def test_pack_shape_errors():
    L = nvq.lib()
    codes = np.zeros((1, 96), np.uint8)
    scales = np.zeros((1, 6), np.uint8)
    dst = np.zeros(128, np.uint8)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert L.nvq_pack_nvfp4(p(codes), p(scales), 1, 96, p(dst)) == -2
    assert L.nvq_pack_nvfp4(None, p(scales), 1, 64, p(dst)) == -1
    assert "NULL" in nvq.last_error()


# Fake but well-aligned "device" addresses: validation must reject the call before
# any of them is dereferenced or any HIP call is made.
A16 = ctypes.c_void_p(0x10000)
A2 = ctypes.c_void_p(0x20002)
MIS = ctypes.c_void_p(0x30004)


def test_gemv_validation_without_gpu():
    L = nvq.lib()
    st = None
    assert L.nvq_gemv_nvfp4(None, 1.0, A16, A16, 1, 8, 64, A16, st) == -1
    assert L.nvq_gemv_nvfp4(A16, 1.0, A16, A16, 1, 8, 96, A16, st) == -2     # K % 64
    assert L.nvq_gemv_nvfp4(A16, 1.0, A16, A16, 0, 8, 64, A16, st) == -2     # M = 0
    assert L.nvq_gemv_nvfp4(A16, 1.0, A16, A16, 16, 8, 64, A16, st) == -2    # M > 15
    assert L.nvq_gemv_nvfp4(A16, 1.0, A16, A16, 1, 0, 64, A16, st) == -2     # N = 0
    assert L.nvq_gemv_nvfp4(MIS, 1.0, A16, A16, 1, 8, 64, A16, st) == -4     # w alignment
    assert L.nvq_gemv_nvfp4(A16, 1.0, A16, ctypes.c_void_p(0x20001), 1, 8, 64, A16, st) == -4
    assert L.nvq_gemv_q4_1(A16, A16, A16, None, 1, 8, 32, A16, st) == -1     # bsum16 required
    assert L.nvq_gemv_nvfp4(A16, 1.0, A16, A16, 3, 8, (1 << 31) - 64, A16, st) == -2  # batched: M*K < 2^32
    assert L.nvq_gemv_q4_1(A16, A16, A16, A2, 1, 8, 48, A16, st) == -2       # K % 32


def test_gemm_validation_without_gpu():
    L = nvq.lib()
    assert L.nvq_gemm_nvfp4(A16, 1.0, A16, A16, 15, 8, 64, A16, None, 0, None) == -2   # M < 16
    assert L.nvq_gemm_nvfp4(A16, 1.0, A16, A16, 16, 8, 32, A16, None, 0, None) == -2   # K % 64
    assert L.nvq_gemm_nvfp4(A16, 1.0, A16, A16, 16, 8, 64, MIS, None, 0, None) == -4   # y alignment
    # M > 16 with K-split parts needs a workspace: missing -> NVQ_ERR_WORKSPACE before any device call
    assert L.nvq_gemm_workspace_bytes(0, 100, 8, 640) > 0
    assert L.nvq_gemm_nvfp4(A16, 1.0, A16, A16, 100, 8, 640, A16, None, 0, None) == -7
    assert L.nvq_gemm_nvfp4(A16, 1.0, A16, A16, 100, 8, 640, A16, A16, 16, None) == -7   # too small
    assert L.nvq_gemm_q4_1(A16, A16, A16, A2, 8, 8, 32, A16, None, 0, None) == -2
    assert L.nvq_gemm_q4_1(A16, A16, A16, A2, 100, 8, 640, A16, None, 0, None) == -7   # K-split parts
    assert L.nvq_gemm_q4_1(A16, A16, A16, A2, 100, 8, 640, A16, MIS, 1 << 21, None) == -4  # ws alignment
    assert L.nvq_quantize_act_q8_0(A16, 1, 48, A16, A16, None, None) == -2
    assert L.nvq_quantize_act_q8_0(MIS, 1, 64, A16, A16, None, None) == -4
    assert L.nvq_quantize_act_q8_0(None, 1, 64, A16, A16, None, None) == -1
    assert L.nvq_debug_isums(7, 0, A16, A16, 1, 8, 64, A16, None) == -3
    assert L.nvq_debug_isums(0, 9, A16, A16, 1, 8, 64, A16, None) == -3
    assert L.nvq_debug_isums(1, 2, A16, A16, 1, 8, 64, A16, None) == -3    # dot4 path is NVFP4 only
    assert L.nvq_gemv_nvfp4_dot4(A16, 1.0, A16, A16, 16, 8, 64, A16, None) == -2
    assert L.nvq_debug_isums(1, 0, A16, A16, 1, 8, 48, A16, None) == -2


def test_routed_gemv_validation_without_gpu():
    """Argument checks of the expert-routed GEMV return before any device call."""
    L = nvq.lib()
    f = L.nvq_gemv_nvfp4_routed
    #   w    scales ids  E  A  q    d    M  N  K   y
    assert f(A16, A16, A16, 0, 6, A16, A16, 1, 8, 64, A16, None) == -2       # no experts
    assert f(A16, A16, A16, 4, 0, A16, A16, 1, 8, 64, A16, None) == -2       # no routing slot
    assert f(A16, A16, A16, 4, 6, A16, A16, 1, 8, 48, A16, None) == -2       # K % 64
    assert f(A16, A16, A16, 4, 6, A16, A16, 20000, 8, 64, A16, None) == -2   # M * n_active > 65535
    assert f(A16, A16, A16, 4, 6, A16, A16, 1, 8, 98304, A16, None) == -2    # beyond the LDS table
    assert f(A16, None, A16, 4, 6, A16, A16, 1, 8, 64, A16, None) == -1      # w_scales
    assert f(A16, A16, None, 4, 6, A16, A16, 1, 8, 64, A16, None) == -1      # ids
    assert f(A16, A16, A2, 4, 6, A16, A16, 1, 8, 64, A16, None) == -4        # ids alignment
    assert f(A16, A16, A16, 4, 6, A16, A16, 1, 8, 64, MIS, None) == -4       # y alignment


def test_status_strings():
    for s, name in [(0, "NVQ_OK"), (-1, "NVQ_ERR_NULL"), (-2, "NVQ_ERR_SHAPE"), (-3, "NVQ_ERR_RANGE"),
                    (-4, "NVQ_ERR_ALIGN"), (-5, "NVQ_ERR_DEVICE"), (-6, "NVQ_ERR_HIP"),
                    (-7, "NVQ_ERR_WORKSPACE")]:
        assert nvq.status_str(s) == name
