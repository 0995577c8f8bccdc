"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, the sizes and packers follow the documented layout, and every
argument error is reported before any HIP call (so these run on a CPU host)."""
import ctypes
import json
import os
import re
import subprocess

import numpy as np
import pytest

import gemm_q8_act_amd as nvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvq.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))


def declared_symbols():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(nvq_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


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
    # K-split workspace of the GEMM kernels (M > 16): fp32 partial tiles (one per
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
    # Q4_1 (integer-MFMA kernel), split up to 16 ways: M > 512 in 128 x 256 tiles with 64
    # accumulators per thread, 64 < M <= 512 in 128 x 128 tiles and 16 < M <= 64 in
    # 256 x 64 tiles with 32
    q41_tile, q41_mid = 512 * 64 * 4, 512 * 32 * 4
    assert ws(nvq.NVQ_FMT_Q4_1, 2048, 4096, 4096) == 0                          # 256 tiles: full rounds
    assert ws(nvq.NVQ_FMT_Q4_1, 1024, 4096, 4096) == 128 * 2 * q41_tile         # 128 tiles, 256 // 128 = 2
    assert ws(nvq.NVQ_FMT_Q4_1, 512, 4096, 4096) == 128 * 2 * q41_mid           # 128 x 128 tiles
    assert ws(nvq.NVQ_FMT_Q4_1, 300, 12800, 256) == 44 * 4 * q41_mid            # 300 tiles: 44 left, 4 stages
    assert ws(nvq.NVQ_FMT_Q4_1, 300, 19200, 256) == 0                           # 450 tiles: 194 left, 256 // 194 = 1
    assert ws(nvq.NVQ_FMT_Q4_1, 100, 8, 640) == 1 * 10 * q41_mid                # split <= stages
    assert ws(nvq.NVQ_FMT_Q4_1, 200, 8, 640) == 2 * 10 * q41_mid
    assert ws(nvq.NVQ_FMT_Q4_1, 600, 8, 640) == 3 * 10 * q41_tile
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


def test_q4_k_block_size_matches_type_table():
    # the GGML type table of the llama.cpp 2-bit GGUF tutorial: Q4_K = 256 values in 144 bytes
    facts = json.load(open(os.path.join(ROOT, "tests", "golden", "page_facts.json")))["q4_k_block"]
    vb, bb = facts["values_per_block"], facts["bytes_per_block"]
    assert nvq.nvq_q4_k_weight_bytes(1, vb) == bb
    assert nvq.nvq_q4_k_weight_bytes(4096, 4096) == 4096 * (4096 // vb) * bb
    assert nvq.nvq_q4_k_weight_bytes(3, 128) == 0          # K % 256 != 0
    assert nvq.nvq_q4_k_weight_bytes(0, 256) == 0


def test_pack_q4_k_layout():
    # decode the documented layout independently: codes as Q4_1, then per (row, 256
    # weights) 16 bytes = d, dmin, and 16 6-bit fields (sc_0..7, mn_0..7) of a 96-bit
    # little-endian number
    r = np.random.Generator(np.random.PCG64(7))
    N, K = 3, 512
    q = r.integers(0, 16, (N, K), dtype=np.uint8)
    sc = r.integers(0, 64, (N, K // 32), dtype=np.uint8)
    mn = r.integers(0, 64, (N, K // 32), dtype=np.uint8)
    d = r.integers(0, 65536, (N, K // 256), dtype=np.uint32).astype(np.uint16)
    dm = r.integers(0, 65536, (N, K // 256), dtype=np.uint32).astype(np.uint16)
    buf = nvq.nvq_pack_q4_k(q, sc, mn, d, dm)
    assert buf.size == N * K * 144 // 256
    cb = buf[: N * K // 2].reshape(N, K // 2)
    assert (cb & 0xF == q[:, 0::2]).all() and (cb >> 4 == q[:, 1::2]).all()
    hdr = buf[N * K // 2:].reshape(N, K // 256, 16)
    assert (hdr[..., 0:2].copy().view(np.uint16)[..., 0] == d).all()
    assert (hdr[..., 2:4].copy().view(np.uint16)[..., 0] == dm).all()
    for n in range(N):
        for b in range(K // 256):
            big = int.from_bytes(bytes(hdr[n, b, 4:16]), "little")
            fields = [(big >> (6 * f)) & 63 for f in range(16)]
            assert fields[:8] == list(sc[n, 8 * b: 8 * b + 8]) and fields[8:] == list(mn[n, 8 * b: 8 * b + 8])


def test_iq4_xs_block_size_matches_type_table():
    # the GGML type table of the llama.cpp 2-bit GGUF tutorial: IQ4_XS = 256 values in 136 bytes
    facts = json.load(open(os.path.join(ROOT, "tests", "golden", "page_facts.json")))["iq4_xs_block"]
    vb, bb = facts["values_per_block"], facts["bytes_per_block"]
    assert nvq.nvq_iq4_xs_weight_bytes(1, vb) == bb
    assert nvq.nvq_iq4_xs_weight_bytes(4096, 4096) == 4096 * (4096 // vb) * bb
    assert nvq.nvq_iq4_xs_weight_bytes(3, 128) == 0


def test_pack_iq4_xs_layout():
    # codes as Q4_1, then per (row, 256 weights) 8 bytes = d and 8 6-bit fields (ls_0..7)
    # of a 48-bit little-endian number
    r = np.random.Generator(np.random.PCG64(8))
    N, K = 3, 512
    q = r.integers(0, 16, (N, K), dtype=np.uint8)
    ls = r.integers(0, 64, (N, K // 32), dtype=np.uint8)
    d = r.integers(0, 65536, (N, K // 256), dtype=np.uint32).astype(np.uint16)
    buf = nvq.nvq_pack_iq4_xs(q, ls, d)
    assert buf.size == N * K * 136 // 256
    cb = buf[: N * K // 2].reshape(N, K // 2)
    assert (cb & 0xF == q[:, 0::2]).all() and (cb >> 4 == q[:, 1::2]).all()
    hdr = buf[N * K // 2:].reshape(N, K // 256, 8)
    assert (hdr[..., 0:2].copy().view(np.uint16)[..., 0] == d).all()
    for n in range(N):
        for b in range(K // 256):
            big = int.from_bytes(bytes(hdr[n, b, 2:8]), "little")
            assert [(big >> (6 * j)) & 63 for j in range(8)] == list(ls[n, 8 * b: 8 * b + 8])


@pytest.mark.parametrize("bad", ["code16", "scale64"])
def test_pack_iq4_xs_rejects_invalid(bad):
    q = np.zeros((1, 256), np.uint8)
    ls = np.zeros((1, 8), np.uint8)
    if bad == "code16":
        q[0, 9] = 16
    else:
        ls[0, 5] = 64
    with pytest.raises(nvq.NvqError) as e:
        nvq.nvq_pack_iq4_xs(q, ls, np.zeros((1, 1), np.uint16))
    assert e.value.status == -3


@pytest.mark.parametrize("bad", ["code16", "scale64", "min64"])
def test_pack_q4_k_rejects_invalid(bad):
    q = np.zeros((1, 256), np.uint8)
    sc = np.zeros((1, 8), np.uint8)
    mn = np.zeros((1, 8), np.uint8)
    d = np.zeros((1, 1), np.uint16)
    if bad == "code16":
        q[0, 7] = 16
    elif bad == "scale64":
        sc[0, 3] = 64
    else:
        mn[0, 6] = 64
    with pytest.raises(nvq.NvqError) as e:
        nvq.nvq_pack_q4_k(q, sc, mn, d, d)
    assert e.value.status == -3


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


def _code_bits_word(q32, bit):
    """The documented high-bit word of 32 codes: bit e = bit `bit` of code 2e, bit
    16 + e = that of code 2e + 1 (independent restatement for the layout tests)."""
    w = 0
    for e in range(16):
        w |= ((int(q32[2 * e]) >> bit) & 1) << e
        w |= ((int(q32[2 * e + 1]) >> bit) & 1) << (16 + e)
    return w


def test_pack_q5_k_layout():
    # low nibbles as Q4_1, the Q4_K headers, then per 32 weights the fifth-bit word
    r = np.random.Generator(np.random.PCG64(9))
    N, K = 3, 512
    q = r.integers(0, 32, (N, K), dtype=np.uint8)
    sc = r.integers(0, 64, (N, K // 32), dtype=np.uint8)
    mn = r.integers(0, 64, (N, K // 32), dtype=np.uint8)
    d = r.integers(0, 65536, (N, K // 256), dtype=np.uint32).astype(np.uint16)
    dm = r.integers(0, 65536, (N, K // 256), dtype=np.uint32).astype(np.uint16)
    buf = nvq.nvq_pack_q5_k(q, sc, mn, d, dm)
    assert buf.size == N * K * 176 // 256 == nvq.nvq_q5_k_weight_bytes(N, K)
    cb = buf[: N * K // 2].reshape(N, K // 2)
    assert (cb & 0xF == q[:, 0::2] & 15).all() and (cb >> 4 == q[:, 1::2] & 15).all()
    # the headers are byte-identical with the Q4_K packer's for the same scales
    ref4 = nvq.nvq_pack_q4_k(q & 15, sc, mn, d, dm)
    assert (buf[N * K // 2: N * K // 2 + N * K // 16] == ref4[N * K // 2:]).all()
    hb = buf[N * K // 2 + N * K // 16:].copy().view(np.uint32).reshape(N, K // 32)
    for n in range(N):
        for b in range(K // 32):
            assert int(hb[n, b]) == _code_bits_word(q[n, 32 * b: 32 * b + 32], 4)


def test_pack_q6_k_layout():
    # low nibbles, int8 scales [N][K/16], two high-bit words per 32 weights, then d
    r = np.random.Generator(np.random.PCG64(10))
    N, K = 3, 512
    q = r.integers(0, 64, (N, K), dtype=np.uint8)
    sc = r.integers(-128, 128, (N, K // 16)).astype(np.int8)
    d = r.integers(0, 65536, (N, K // 256), dtype=np.uint32).astype(np.uint16)
    buf = nvq.nvq_pack_q6_k(q, sc, d)
    assert buf.size == N * K * 210 // 256 == nvq.nvq_q6_k_weight_bytes(N, K)
    o1, o2, o3 = N * K // 2, N * K // 2 + N * K // 16, N * K // 2 + N * K // 16 + N * K // 4
    cb = buf[:o1].reshape(N, K // 2)
    assert (cb & 0xF == q[:, 0::2] & 15).all() and (cb >> 4 == q[:, 1::2] & 15).all()
    assert (buf[o1:o2].view(np.int8).reshape(N, K // 16) == sc).all()
    hb = buf[o2:o3].copy().view(np.uint32).reshape(N, K // 32, 2)
    for n in range(N):
        for b in range(K // 32):
            assert int(hb[n, b, 0]) == _code_bits_word(q[n, 32 * b: 32 * b + 32], 4)
            assert int(hb[n, b, 1]) == _code_bits_word(q[n, 32 * b: 32 * b + 32], 5)
    assert (buf[o3:].copy().view(np.uint16).reshape(N, K // 256) == d).all()


def test_q5_k_q6_k_sizes():
    assert nvq.nvq_q5_k_weight_bytes(1, 256) == 176 and nvq.nvq_q6_k_weight_bytes(1, 256) == 210
    assert nvq.nvq_q5_k_weight_bytes(4096, 4096) == 4096 * 16 * 176
    assert nvq.nvq_q6_k_weight_bytes(4096, 4096) == 4096 * 16 * 210
    assert nvq.nvq_q5_k_weight_bytes(3, 128) == 0 and nvq.nvq_q6_k_weight_bytes(0, 256) == 0


@pytest.mark.parametrize("bad", ["code32", "scale64", "min64"])
def test_pack_q5_k_rejects_invalid(bad):
    q = np.zeros((1, 256), np.uint8)
    sc = np.zeros((1, 8), np.uint8)
    mn = np.zeros((1, 8), np.uint8)
    d = np.zeros((1, 1), np.uint16)
    if bad == "code32":
        q[0, 200] = 32
    elif bad == "scale64":
        sc[0, 3] = 64
    else:
        mn[0, 6] = 64
    with pytest.raises(nvq.NvqError) as e:
        nvq.nvq_pack_q5_k(q, sc, mn, d, d)
    assert e.value.status == -3


def test_pack_q6_k_rejects_invalid():
    q = np.zeros((1, 256), np.uint8)
    q[0, 255] = 64
    with pytest.raises(nvq.NvqError) as e:
        nvq.nvq_pack_q6_k(q, np.zeros((1, 16), np.int8), np.zeros((1, 1), np.uint16))
    assert e.value.status == -3


def test_packers_write_nothing_on_error():
    # every packer checks its whole input before writing: a bad last code leaves dst as it was
    L = nvq.lib()
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    N, K = 2, 256
    z32, z256 = np.zeros((N, K // 32), np.uint8), np.zeros((N, K // 256), np.uint16)
    cases = {
        "q4_1": (15, lambda q, dst: L.nvq_pack_q4_1(p(q), p(np.zeros((N, K // 32), np.uint16)),
                                                    p(np.zeros((N, K // 32), np.uint16)), N, K, p(dst))),
        "q4_k": (15, lambda q, dst: L.nvq_pack_q4_k(p(q), p(z32), p(z32), p(z256), p(z256), N, K, p(dst))),
        "q5_k": (31, lambda q, dst: L.nvq_pack_q5_k(p(q), p(z32), p(z32), p(z256), p(z256), N, K, p(dst))),
        "q6_k": (63, lambda q, dst: L.nvq_pack_q6_k(p(q), p(np.zeros((N, K // 16), np.int8)), p(z256), N, K, p(dst))),
        "iq4_xs": (15, lambda q, dst: L.nvq_pack_iq4_xs(p(q), p(z32), p(z256), N, K, p(dst))),
    }
    for name, (cmax, fn) in cases.items():
        q = np.full((N, K), cmax, np.uint8)
        q[-1, -1] = cmax + 1
        dst = np.full(N * K, 0xA5, np.uint8)
        assert fn(q, dst) == -3, name
        assert (dst == 0xA5).all(), name


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
    assert L.nvq_debug_isums(2, 0, A16, A16, 1, 8, 128, A16, None) == -2   # Q4_K: K % 256
    # Q4_K entries: K % 256, bsum16 required, M ranges, workspace for the integer-MFMA kernel
    assert L.nvq_gemv_q4_k(A16, A16, A16, A2, 1, 8, 128, A16, None) == -2
    assert L.nvq_gemv_q4_k(A16, A16, A16, None, 1, 8, 256, A16, None) == -1
    assert L.nvq_gemv_q4_k(A16, A16, A16, A2, 16, 8, 256, A16, None) == -2
    assert L.nvq_gemm_q4_k(A16, A16, A16, A2, 15, 8, 256, A16, None, 0, None) == -2
    assert L.nvq_gemm_workspace_bytes(2, 100, 8, 768) > 0
    assert L.nvq_gemm_workspace_bytes(2, 100, 8, 640) == 0                  # K % 256 != 0
    assert L.nvq_gemm_q4_k(A16, A16, A16, A2, 100, 8, 768, A16, None, 0, None) == -7
    # IQ4_XS entries: the value table is required, K % 256, workspace; generic debug entry rejects the format
    assert L.nvq_gemv_iq4_xs(A16, None, A16, A16, 1, 8, 256, A16, None) == -1
    assert L.nvq_gemv_iq4_xs(A16, A16, A16, A16, 1, 8, 128, A16, None) == -2
    assert L.nvq_gemm_iq4_xs(A16, A16, A16, A16, 15, 8, 256, A16, None, 0, None) == -2
    assert L.nvq_gemm_workspace_bytes(3, 100, 8, 768) == L.nvq_gemm_workspace_bytes(2, 100, 8, 768) > 0
    assert L.nvq_gemm_iq4_xs(A16, A16, A16, A16, 100, 8, 768, A16, None, 0, None) == -7
    assert L.nvq_debug_isums(3, 0, A16, A16, 1, 8, 256, A16, None) == -3
    assert L.nvq_debug_isums_iq4_xs(None, 0, A16, A16, 1, 8, 256, A16, None) == -1
    assert L.nvq_debug_isums_iq4_xs(A16, 2, A16, A16, 1, 8, 256, A16, None) == -3


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


# ---- measurement probes: every argument error is reported before any HIP call ----

ERR_NULL, ERR_SHAPE, ERR_RANGE, ERR_ALIGN = -1, -2, -3, -4  # include/nvq.h


def test_probe_rejects():
    L = nvq.lib()
    P = ctypes.c_void_p
    buf = P(16 * 1024)  # never dereferenced: validation fails first
    sink = P(4096)
    # read: NULL, alignment, size, block count
    assert L.nvq_probe_read(None, 1024, 4, sink, None) == ERR_NULL
    assert L.nvq_probe_read(P(16 * 1024 + 8), 1024, 4, sink, None) == ERR_ALIGN
    assert L.nvq_probe_read(buf, 1000, 4, sink, None) == ERR_SHAPE
    assert L.nvq_probe_read(buf, 0, 4, sink, None) == ERR_SHAPE
    assert L.nvq_probe_read(buf, 1024, 0, sink, None) == ERR_SHAPE
    assert L.nvq_probe_read(buf, 1024, 65537, sink, None) == ERR_SHAPE
    # gemv loads: shape, splits, launch shape
    assert L.nvq_probe_gemv_loads(buf, 64, 100, 1, 4, 5, sink, None) == ERR_SHAPE
    assert L.nvq_probe_gemv_loads(buf, 64, 256, 3, 4, 5, sink, None) == ERR_RANGE  # 2 chunks < 3 splits
    assert L.nvq_probe_gemv_loads(buf, 64, 5120, 9, 4, 5, sink, None) == ERR_RANGE
    assert L.nvq_probe_gemv_loads(buf, 64, 5120, 1, 6, 5, sink, None) == ERR_RANGE
    assert L.nvq_probe_gemv_loads(buf, 64, 5120, 1, 8, 4, sink, None) == ERR_RANGE
    assert L.nvq_probe_gemv_loads(None, 64, 5120, 1, 8, 5, sink, None) == ERR_NULL
    # mfma: blocks, iterations
    assert L.nvq_probe_mfma(0, 10, 0, sink, None) == ERR_SHAPE
    assert L.nvq_probe_mfma(8, 0, 0, sink, None) == ERR_SHAPE
    assert L.nvq_probe_mfma(8, 10, 0, None, None) == ERR_NULL
    assert "blocks" in nvq.last_error() or "NULL" in nvq.last_error()


def test_q5_k_q6_k_validation_without_gpu():
    L = nvq.lib()
    st = None
    # K % 256, M range, bsum16 (Q5_K only), workspace
    assert L.nvq_gemv_q5_k(A16, A16, A2, A2, 1, 8, 128, A16, st) == -2
    assert L.nvq_gemv_q5_k(A16, A16, A2, None, 1, 8, 256, A16, st) == -1
    assert L.nvq_gemv_q5_k(A16, A16, A2, A2, 16, 8, 256, A16, st) == -2
    assert L.nvq_gemv_q6_k(A16, A16, A2, 1, 8, 320, A16, st) == -2
    assert L.nvq_gemv_q6_k(A16, MIS, A2, 1, 8, 256, A16, st) == -4
    need = nvq.nvq_gemm_workspace_bytes(nvq.NVQ_FMT_Q6_K, 40, 4096, 4096)
    assert need > 0 and need == nvq.nvq_gemm_workspace_bytes(nvq.NVQ_FMT_Q5_K, 40, 4096, 4096)
    assert L.nvq_gemm_q6_k(A16, A16, A2, 40, 4096, 4096, A16, None, 0, st) == -7
    assert L.nvq_gemm_q5_k(A16, A16, A2, A2, 40, 4096, 4096, A16, None, need - 1, st) == -7
    assert L.nvq_gemm_q5_k(A16, A16, A2, A2, 8, 64, 256, A16, None, 0, st) == -2   # M < 16
    assert L.nvq_debug_isums(nvq.NVQ_FMT_Q6_K, 1, A16, A16, 1, 8, 320, A16, st) == -2
    assert L.nvq_debug_isums(6, 1, A16, A16, 1, 8, 256, A16, st) == -3

