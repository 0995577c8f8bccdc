"""Pins of the oracle: checks that tie every oracle function to something other
than itself -- library decoders (torch float8, numpy float16), brute force on
small inputs with numpy float64 matmul, closed-form special cases, constructed
rounding ties, and the bias identity the NVFP4 page states.

``battery(oracle)`` runs every pin and returns a list of (name, ok, detail).  The
pin tests assert all pass; the planted-mistake tests assert that each deliberately
broken oracle fails at least one of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def page_facts() -> dict:
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Independent references
# ---------------------------------------------------------------------------

def minifloat(bits: int, ebits: int, mbits: int, bias: int) -> float:
    """Generic sign/exponent/mantissa decode of a finite minifloat code (no inf/NaN
    handling).  Validated below against torch's float8 decoders and numpy float16
    before it is used as the reference for E2M1."""
    s = (bits >> (ebits + mbits)) & 1
    e = (bits >> mbits) & ((1 << ebits) - 1)
    m = bits & ((1 << mbits) - 1)
    if e == 0:
        v = m * 2.0 ** (1 - bias - mbits)
    else:
        v = ((1 << mbits) + m) * 2.0 ** (e - bias - mbits)
    return -v if s else v


def _library_minifloat_check() -> list[str]:
    """The generic decoder agrees with three library decoders on all their finite codes."""
    import torch

    bad = []
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    for dt, eb, mb, bias in ((torch.float8_e4m3fn, 4, 3, 7), (torch.float8_e5m2, 5, 2, 15)):
        vals = codes.view(dt).to(torch.float64).numpy()
        for b in range(256):
            if math.isfinite(vals[b]) and minifloat(b, eb, mb, bias) != vals[b]:
                bad.append(f"{dt} code {b}")
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    for b in range(0, 65536, 7):
        if math.isfinite(h[b]) and minifloat(b, 5, 10, 15) != h[b]:
            bad.append(f"float16 code {b}")
    return bad


def e2m1_ref(code: int) -> float:
    return minifloat(code, 2, 1, 1)


def ue4m3_ref_table() -> np.ndarray:
    import torch

    return torch.arange(128, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------------------
# Small synthetic cases (independent of the synth module on purpose: pins use
# their own tiny, hand-shaped inputs)
# ---------------------------------------------------------------------------

def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _nvfp4_case(seed, M, N, K):
    r = _rng(seed)
    codes = r.integers(0, 16, (N, K), dtype=np.uint8)
    e = r.integers(-4, 5, (N, K // 16))
    m = r.integers(0, 8, (N, K // 16))
    scales = (((e + 7) << 3) | m).astype(np.uint8)
    x = r.standard_normal((M, K)).astype(np.float32)
    return codes, scales, x


# ---------------------------------------------------------------------------
# The battery
# ---------------------------------------------------------------------------

def battery(o) -> list[tuple[str, bool, str]]:
    out: list[tuple[str, bool, str]] = []

    def pin(name, ok, detail=""):
        out.append((name, bool(ok), detail))

    facts = page_facts()

    # P1: E2M1 against the library-validated generic minifloat decoder
    lib_bad = _library_minifloat_check()
    pin("minifloat_reference_matches_libraries", not lib_bad, ",".join(lib_bad[:5]))
    bad = [c for c in range(16) if o.e2m1(c) != e2m1_ref(c)]
    pin("e2m1_closed_form", not bad, f"codes {bad}")

    # P2: the page's biased LUT range and the sign symmetry of the 4-bit code
    L = [2.0 * o.e2m1(c) for c in range(16)]
    ints = all(float(v).is_integer() for v in L)
    bias = facts["bias_trick"]["lut_bias"]
    lo, hi = facts["bias_trick"]["unsigned_code_min"], facts["bias_trick"]["unsigned_code_max"]
    rng_ok = ints and min(L) + bias == lo and max(L) + bias == hi
    sym = all(L[c + 8] == -L[c] for c in range(8))
    mono = all(L[c] < L[c + 1] for c in range(7))
    pin("lut_range_0_24_and_symmetry", rng_ok and sym and mono, f"L={L}")

    # P3/P4: UE4M3 against torch's E4M3 decoder; invalid bytes are NaN; anchors
    ref = ue4m3_ref_table()
    bad = [b for b in range(127) if o.ue4m3(b) != ref[b]]
    nan_ok = all(math.isnan(o.ue4m3(b)) for b in [0x7F] + list(range(0x80, 0x100)))
    pin("ue4m3_vs_library", not bad and nan_ok, f"bad {bad[:8]}")
    anchors = {0x38: 1.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x7E: 448.0, 0x00: 0.0}
    pin("ue4m3_anchors", all(o.ue4m3(b) == v for b, v in anchors.items()))

    # P5: binary16 -> double, exhaustive against numpy
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref16 = f16_bits_to_f64(allb)
    got = np.array([o.f16_to_f64(int(b)) for b in allb], np.float64)
    same = (got == ref16) | (np.isnan(got) & np.isnan(ref16))
    pin("f16_to_f64_exhaustive", bool(same.all()), f"{int((~same).sum())} mismatches")

    # P6: float -> binary16 (RNE, subnormals, overflow) against numpy on a varied set
    r = _rng(11)
    xs = [np.float32(v) for v in (0.0, -0.0, 1.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9,
                                   2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26,
                                   2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11,
                                   1.0 + 3 * 2.0 ** -11, -(1.0 + 2.0 ** -11), 5 * 2.0 ** -25)]
    bits = r.integers(0, 2 ** 32, 4000, dtype=np.uint64).astype(np.uint32)
    expo = r.integers(127 - 30, 127 + 18, 4000).astype(np.uint32)
    bits = (bits & np.uint32(0x807FFFFF)) | (expo << np.uint32(23))
    xs += list(bits.view(np.float32))
    k = r.integers(0, 2048, 300)
    xs += list(np.float32((2 * k + 1) * 2.0 ** -25))               # subnormal ties
    xs += list(np.float32((1024 + k) * 2.0 ** -10 + 2.0 ** -11))    # normal ties near 1
    xs = np.array(xs, np.float32)
    with np.errstate(over="ignore"):
        want = xs.astype(np.float16).view(np.uint16)
    got = np.array([o.f32_to_f16(float(v)) for v in xs], np.uint16)
    pin("f32_to_f16_vs_library", bool((got == want).all()), f"{int((got != want).sum())} mismatches")

    # P7: Q8_0 on constructed blocks with exactly known answers
    blk = np.zeros(32, np.float32)
    blk[:10] = [127.0, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 126.5, -3.5, 4.5]
    q, d16, bs = o.quantize_q8_0(blk[None, :])
    exp_q = [127, 2, 4, -2, 0, 2, 0, 126, -4, 4] + [0] * 22
    ok7 = list(q[0]) == exp_q and int(d16[0, 0]) == 0x3C00
    ok7 &= int(bs[0, 0]) == sum(exp_q[:16]) and int(bs[0, 1]) == sum(exp_q[16:])
    blk2 = np.zeros(32, np.float32)
    blk2[:3] = [63.5, 1.25, 0.75]          # d32 = 0.5: 2.5 -> 2, 1.5 -> 2
    q2, d2, _ = o.quantize_q8_0(blk2[None, :])
    ok7 &= list(q2[0, :3]) == [127, 2, 2] and int(d2[0, 0]) == 0x3800
    q3, d3, b3 = o.quantize_q8_0(np.zeros((1, 64), np.float32))
    ok7 &= not q3.any() and not d3.any() and not b3.any()
    blk4 = -blk                            # sign symmetry
    q4, _, _ = o.quantize_q8_0(blk4[None, :])
    ok7 &= list(q4[0]) == [-v for v in exp_q]
    pin("q8_0_constructed_ties", ok7, f"q={list(q[0][:10])} d={hex(int(d16[0,0]))}")

    # P7b: float32 subnormal blocks.  amax = 50 * 2^-149 gives d32 = amax / 127 below
    # half the least subnormal, so d32 rounds to 0: the block stores d = 0 and q = 0
    # like an all-zero block.  amax = 127 * 2^-149 gives d32 = 2^-149 exactly, a
    # non-zero divisor, so the codes are the integers x / 2^-149 themselves.
    tiny = np.float32(2.0 ** -149)
    blk5 = np.zeros(64, np.float32)
    blk5[:4] = [50 * tiny, -50 * tiny, 7 * tiny, -tiny]
    blk5[32:36] = [127 * tiny, -5 * tiny, 64 * tiny, 0.0]
    d32a = np.float32(blk5[0] / np.float32(127.0))
    d32b = np.float32(blk5[32] / np.float32(127.0))
    q5, d5, b5 = o.quantize_q8_0(blk5[None, :])
    ok7b = d32a == 0.0 and d32b == tiny
    ok7b &= not q5[0, :32].any() and int(d5[0, 0]) == 0 and int(b5[0, 0]) == 0 and int(b5[0, 1]) == 0
    ok7b &= list(q5[0, 32:36]) == [127, -5, 64, 0] and int(d5[0, 1]) == 0
    pin("q8_0_underflowing_scale", ok7b, f"q={list(q5[0, :4])} {list(q5[0, 32:36])} d={list(d5[0])}")

    # P8: Q8_0 on random rows: properties + numpy float32 / float16 cross-check
    x = _rng(12).standard_normal((5, 96)).astype(np.float32) * np.float32(3.0)
    x[1, 40] = 0.0
    x[2, 0:32] *= np.float32(1e-4)          # tiny block: binary16 subnormal scale
    q, d16, bs = o.quantize_q8_0(x)
    xb = x.reshape(5, 3, 32)
    amax = np.abs(xb).max(axis=2)
    d32 = (amax / np.float32(127.0)).astype(np.float32)
    t = (xb / d32[:, :, None]).astype(np.float32)
    q_ref = np.clip(np.rint(t), -127, 127).astype(np.int8).reshape(5, 96)
    d_ref = d32.astype(np.float16).view(np.uint16)
    b_ref = q_ref.astype(np.int32).reshape(5, 6, 16).sum(axis=2)
    ok8 = (q == q_ref).all() and (d16 == d_ref).all() and (bs == b_ref).all()
    at = np.argmax(np.abs(xb), axis=2)
    qb = q.reshape(5, 3, 32)
    peaks = np.take_along_axis(qb, at[:, :, None], axis=2)[:, :, 0]
    ok8 &= (np.abs(peaks) == 127).all() and (np.abs(q.astype(int)) <= 127).all()
    pin("q8_0_random_vs_numpy", ok8, "")

    # P9: the divisor is the float32 d32, not the rounded binary16 d
    amax = np.float32(1.0)
    d32 = np.float32(amax / np.float32(127.0))
    d16v = float(np.float32(d32).astype(np.float16))
    xv = np.float32(100.4999 * float(d32))
    blk = np.zeros(32, np.float32)
    blk[0], blk[1] = amax, xv
    qv, _, _ = o.quantize_q8_0(blk[None, :])
    via32 = int(np.rint(np.float32(xv) / d32))
    via16 = int(np.rint(np.float32(xv) / np.float32(d16v)))
    pin("q8_0_divides_by_float32_d", via32 != via16 and int(qv[0, 1]) == via32,
        f"q={int(qv[0,1])} via32={via32} via16={via16}")

    # P10: integer per-16 sums against brute force with the reference E2M1
    codes, scales, x = _nvfp4_case(13, 3, 5, 128)
    q, d16, bs = o.quantize_q8_0(x)
    Lref = np.array([int(2 * e2m1_ref(c)) for c in range(16)], np.int64)
    W_int = Lref[codes]                                    # [N, K]
    isum_ref = (q.astype(np.int64)[:, None, :] * W_int[None, :, :]).reshape(3, 5, 8, 16).sum(axis=3)
    isums = o.isums_nvfp4(codes, q)
    pin("isums_nvfp4_bruteforce", (isums == isum_ref).all())

    # P11: the page's bias identity over each 16-subblock
    U = W_int + bias
    biased = (q.astype(np.int64)[:, None, :] * U[None, :, :]).reshape(3, 5, 8, 16).sum(axis=3)
    rhs = biased - bias * bs.astype(np.int64)[:, None, :]
    pin("bias_identity", (rhs == isums).all() and U.min() >= lo and U.max() <= hi)

    # P12: products against float64 dequantize-then-matmul
    for (seed, M, N, K, S) in ((14, 3, 7, 256, 1.0), (15, 2, 4, 1024, 1.7341)):
        codes, scales, x = _nvfp4_case(seed, M, N, K)
        q, d16, _ = o.quantize_q8_0(x)
        E = np.array([e2m1_ref(c) for c in range(16)])[codes]
        Uv = ue4m3_ref_table()[scales]
        Wd = np.float64(np.float32(S)) * np.repeat(Uv, 16, axis=1) * E
        Ad = np.repeat(f16_bits_to_f64(d16), 32, axis=1) * q.astype(np.float64)
        yref = Ad @ Wd.T
        aref = np.abs(Ad) @ np.abs(Wd).T
        y, awa = o.matmul_nvfp4(codes, scales, S, q, d16)
        ulp = np.spacing(np.abs(yref).astype(np.float32))
        ok = (np.abs(y.astype(np.float64) - yref) <= ulp).all()
        ok &= np.allclose(awa, aref, rtol=1e-12, atol=0)
        pin(f"matmul_nvfp4_bruteforce_{K}", ok, f"max err {np.abs(y - yref).max():.3g}")

    # P13: closed-form special cases
    codes = np.zeros((2, 64), np.uint8)
    scales = np.full((2, 4), 0x38, np.uint8)
    codes[1, 37] = 0x7                     # E2M1 6.0 at k=37
    scales[1, 2] = 0x4B                    # UE4M3 (1 + 3/8) * 2^2 = 5.5
    x = np.zeros((1, 64), np.float32)
    x[0, 37] = 3.0
    x[0, 33] = -7.0                        # same 32-block, amax 7 -> d32 = 7/127
    q, d16, _ = o.quantize_q8_0(x)
    y, _ = o.matmul_nvfp4(codes, scales, 0.5, q, d16)
    closed = np.float32(0.5 * 5.5 * 6.0 * float(f16_bits_to_f64(d16[0, 1])) * int(q[0, 37]))
    ok13 = y[0, 0] == 0.0 and y[0, 1] == closed and int(q[0, 37]) == int(np.rint(np.float32(3.0) / np.float32(np.float32(7.0) / np.float32(127.0))))
    codes, scales, x = _nvfp4_case(16, 2, 3, 128)
    q, d16, _ = o.quantize_q8_0(x)
    zc = np.where(codes < 8, 0, 8).astype(np.uint8)   # every code is +0 or -0
    yz, _ = o.matmul_nvfp4(zc, scales, 1.0, q, d16)
    ok13 &= not yz.any()
    y1, _ = o.matmul_nvfp4(codes, scales, 1.0, q, d16)
    y2, _ = o.matmul_nvfp4(codes, scales, 2.0, q, d16)
    ok13 &= (y2 == 2 * y1).all()
    ysub, _ = o.matmul_nvfp4(codes, scales, 1.0, q, d16, cols=[2, 0])
    ok13 &= (ysub[:, 0] == y1[:, 2]).all() and (ysub[:, 1] == y1[:, 0]).all()
    pin("matmul_nvfp4_special_cases", ok13, f"y={y[0]} closed={closed}")

    # P16: expert-routed product against float64 dequantize-then-matmul per (token,
    # slot); an out-of-range id gives a NaN row; relabelling the experts (storage order
    # permuted, ids mapped) changes nothing
    r = _rng(18)
    E, A, M, N, K = 4, 3, 2, 5, 128
    codes = r.integers(0, 16, (E, N, K), dtype=np.uint8)
    ee = r.integers(-4, 5, (E, N, K // 16))
    mm = r.integers(0, 8, (E, N, K // 16))
    scales = (((ee + 7) << 3) | mm).astype(np.uint8)
    wsc = r.uniform(0.5, 2.0, E).astype(np.float32)
    x = r.standard_normal((M, K)).astype(np.float32)
    q, d16, _ = o.quantize_q8_0(x)
    ids = np.array([[2, 0, 2], [3, 1, 7]], np.int32)       # a repeated expert; 7 is invalid
    y, awa = o.matmul_nvfp4_routed(codes, scales, wsc, ids, q, d16)
    Ad = np.repeat(f16_bits_to_f64(d16), 32, axis=1) * q.astype(np.float64)
    Etab = np.array([e2m1_ref(c) for c in range(16)])
    ok16 = True
    for mi in range(M):
        for a in range(A):
            e = int(ids[mi, a])
            if not 0 <= e < E:
                ok16 &= bool(np.isnan(y[mi, a]).all()) and not awa[mi, a].any()
                continue
            Wd = np.float64(wsc[e]) * np.repeat(ue4m3_ref_table()[scales[e]], 16, axis=1) * Etab[codes[e]]
            yref = Wd @ Ad[mi]
            ok16 &= bool((np.abs(y[mi, a].astype(np.float64) - yref) <= np.spacing(np.abs(yref).astype(np.float32))).all())
            ok16 &= bool(np.allclose(awa[mi, a], np.abs(Wd) @ np.abs(Ad[mi]), rtol=1e-12, atol=0))
    perm = np.array([3, 0, 1, 2])                            # new slot i holds old expert perm[i]
    inv = np.argsort(perm)
    ids_p = np.where((ids >= 0) & (ids < E), inv[np.clip(ids, 0, E - 1)], ids).astype(np.int32)
    y_p, _ = o.matmul_nvfp4_routed(codes[perm], scales[perm], wsc[perm], ids_p, q, d16)
    ok16 &= bool(((y_p == y) | (np.isnan(y_p) & np.isnan(y))).all())
    pin("matmul_nvfp4_routed_bruteforce_and_relabel", ok16)

    # P14/P15: Q4_1
    r = _rng(17)
    M, N, K = 3, 5, 128
    qw = r.integers(0, 16, (N, K), dtype=np.uint8)
    dw = r.uniform(1e-3, 2e-2, (N, K // 32)).astype(np.float16).view(np.uint16)
    mw = r.uniform(-0.1, 0.0, (N, K // 32)).astype(np.float16).view(np.uint16)
    x = r.standard_normal((M, K)).astype(np.float32)
    q, d16, bs = o.quantize_q8_0(x)
    isum_ref = (q.astype(np.int64)[:, None, :] * qw.astype(np.int64)[None]).reshape(M, N, K // 16, 16).sum(axis=3)
    pin("isums_q4_1_bruteforce", (o.isums_q4_1(qw, q) == isum_ref).all())
    Wd = np.repeat(f16_bits_to_f64(dw), 32, axis=1) * qw + np.repeat(f16_bits_to_f64(mw), 32, axis=1)
    Ad = np.repeat(f16_bits_to_f64(d16), 32, axis=1) * q.astype(np.float64)
    yref = Ad @ Wd.T
    y, awa = o.matmul_q4_1(qw, dw, mw, q, d16)
    ok15 = (np.abs(y.astype(np.float64) - yref) <= np.spacing(np.abs(yref).astype(np.float32))).all()
    ok15 &= np.allclose(awa, np.abs(Ad) @ np.abs(Wd).T, rtol=1e-12, atol=0)
    y0, _ = o.matmul_q4_1(qw, np.zeros_like(dw), mw, q, d16)
    bs32 = bs.astype(np.int64).reshape(M, K // 32, 2).sum(axis=2)
    ref0 = (f16_bits_to_f64(d16) * bs32) @ f16_bits_to_f64(mw).T
    ok15 &= (np.abs(y0 - ref0) <= np.spacing(np.abs(ref0).astype(np.float32))).all()
    pin("matmul_q4_1_bruteforce_and_zero_scale", ok15)

    # P16: Q4_K -- brute force on its own definition (numpy float64, the block size of
    # the GGML type table), the reduction to Q4_1 when every per-32 scale d*sc and min
    # dmin*mn is a binary16 value, and the zero-min case
    facts = page_facts()["q4_k_block"]
    SB = facts["values_per_block"]
    r = _rng(18)
    M, N, K = 3, 4, 2 * SB
    qw = r.integers(0, 16, (N, K), dtype=np.uint8)
    sc = r.integers(0, 64, (N, K // 32), dtype=np.uint8)
    mn = r.integers(0, 64, (N, K // 32), dtype=np.uint8)
    dd = r.uniform(2e-5, 3e-4, (N, K // SB)).astype(np.float16).view(np.uint16)
    dm = r.uniform(0.0, 1.6e-3, (N, K // SB)).astype(np.float16).view(np.uint16)
    x = r.standard_normal((M, K)).astype(np.float32)
    q, d16, bs = o.quantize_q8_0(x)
    Wd = (np.repeat(f16_bits_to_f64(dd), SB, axis=1) * np.repeat(sc.astype(np.float64), 32, axis=1) * qw
          - np.repeat(f16_bits_to_f64(dm), SB, axis=1) * np.repeat(mn.astype(np.float64), 32, axis=1))
    Ad = np.repeat(f16_bits_to_f64(d16), 32, axis=1) * q.astype(np.float64)
    yref = Ad @ Wd.T
    y, awa = o.matmul_q4_k(qw, sc, mn, dd, dm, q, d16)
    ok16k = (np.abs(y.astype(np.float64) - yref) <= np.spacing(np.abs(yref).astype(np.float32))).all()
    ok16k &= np.allclose(awa, np.abs(Ad) @ np.abs(Wd).T, rtol=1e-12, atol=0)
    # powers of two d = 2^-12, dmin = 2^-9: d*sc and dmin*mn are binary16 values
    dp = np.full((N, K // SB), 2.0 ** -12, np.float16).view(np.uint16)
    mp = np.full((N, K // SB), 2.0 ** -9, np.float16).view(np.uint16)
    dw41 = (2.0 ** -12 * sc.astype(np.float64)).astype(np.float16).view(np.uint16)
    mw41 = (-(2.0 ** -9) * mn.astype(np.float64)).astype(np.float16).view(np.uint16)
    yk, _ = o.matmul_q4_k(qw, sc, mn, dp, mp, q, d16)
    y1, _ = o.matmul_q4_1(qw, dw41, mw41, q, d16)
    ok16k &= bool((yk == y1).all())
    ymin0, _ = o.matmul_q4_k(qw, sc, np.zeros_like(mn), dd, dm, q, d16)
    ref0 = Ad @ (Wd + np.repeat(f16_bits_to_f64(dm), SB, axis=1) * np.repeat(mn.astype(np.float64), 32, axis=1)).T
    ok16k &= bool((np.abs(ymin0.astype(np.float64) - ref0) <= np.spacing(np.abs(ref0).astype(np.float32))).all())
    pin("matmul_q4_k_bruteforce_q4_1_reduction_zero_min", bool(ok16k))

    # P17: IQ4_XS -- per-16 sums and y by brute force on its definition (a seeded int8
    # value table), the reduction to Q4_1 when the table is the affine c - 8 and every
    # per-32 scale is a binary16 value, and invariance under relabelling the table
    facts = page_facts()["iq4_xs_block"]
    SB = facts["values_per_block"]
    r = _rng(19)
    M, N, K = 3, 4, 2 * SB
    qw = r.integers(0, 16, (N, K), dtype=np.uint8)
    ls = r.integers(0, 64, (N, K // 32), dtype=np.uint8)
    dd = r.uniform(1e-4, 1e-3, (N, K // SB)).astype(np.float16).view(np.uint16)
    table = np.sort(r.choice(np.arange(-128, 128), 16, replace=False)).astype(np.int8)
    x = r.standard_normal((M, K)).astype(np.float32)
    q, d16, bs = o.quantize_q8_0(x)
    Vq = table.astype(np.int64)[qw]
    isum_ref = (q.astype(np.int64)[:, None, :] * Vq[None]).reshape(M, N, K // 16, 16).sum(axis=3)
    ok17 = bool((o.isums_iq4_xs(qw, table, q) == isum_ref).all())
    Wd = (np.repeat(f16_bits_to_f64(dd), SB, axis=1) * np.repeat(ls.astype(np.float64) - 32.0, 32, axis=1)
          * Vq.astype(np.float64))
    Ad = np.repeat(f16_bits_to_f64(d16), 32, axis=1) * q.astype(np.float64)
    yref = Ad @ Wd.T
    y, awa = o.matmul_iq4_xs(qw, ls, dd, table, q, d16)
    ok17 &= bool((np.abs(y.astype(np.float64) - yref) <= np.spacing(np.abs(yref).astype(np.float32))).all())
    ok17 &= bool(np.allclose(awa, np.abs(Ad) @ np.abs(Wd).T, rtol=1e-12, atol=0))
    aff = (np.arange(16) - 8).astype(np.int8)
    dp = np.full((N, K // SB), 2.0 ** -10, np.float16).view(np.uint16)
    D = 2.0 ** -10 * (ls.astype(np.float64) - 32.0)
    yx, _ = o.matmul_iq4_xs(qw, ls, dp, aff, q, d16)
    y1, _ = o.matmul_q4_1(qw, D.astype(np.float16).view(np.uint16), (-8.0 * D).astype(np.float16).view(np.uint16),
                          q, d16)
    ok17 &= bool((yx == y1).all())
    perm = r.permutation(16)                                   # new table slot i holds old entry perm[i]
    yp, _ = o.matmul_iq4_xs(np.argsort(perm).astype(np.uint8)[qw], ls, dd, table[perm], q, d16)
    ok17 &= bool((yp == y).all())
    pin("iq4_xs_bruteforce_q4_1_reduction_relabel", ok17)

    # P18: Q5_K (no block or rule in the pages: the GGML format's reading, 256-weight
    # super-blocks) -- per-16 sums and y by brute force on its definition, and the split
    # of each 5-bit code c = c_lo + 16 c_hi: the product equals the Q4_K product of the
    # low nibbles plus that of the fifth bits with scale 16 d and no min (the fifth bit
    # weighs 16, the min is applied once)
    SB = 256
    r = _rng(20)
    M, N, K = 3, 4, 2 * SB
    qw = r.integers(0, 32, (N, K), dtype=np.uint8)
    sc = r.integers(0, 64, (N, K // 32), dtype=np.uint8)
    mn = r.integers(0, 64, (N, K // 32), dtype=np.uint8)
    dd = r.uniform(1e-5, 1.5e-4, (N, K // SB)).astype(np.float16).view(np.uint16)
    dm = r.uniform(0.0, 1.6e-3, (N, K // SB)).astype(np.float16).view(np.uint16)
    x = r.standard_normal((M, K)).astype(np.float32)
    q, d16, bs = o.quantize_q8_0(x)
    isum_ref = (q.astype(np.int64)[:, None, :] * qw.astype(np.int64)[None]).reshape(M, N, K // 16, 16).sum(axis=3)
    ok18 = bool((o.isums_q5_k(qw, q) == isum_ref).all())
    Wd = (np.repeat(f16_bits_to_f64(dd), SB, axis=1) * np.repeat(sc.astype(np.float64), 32, axis=1) * qw
          - np.repeat(f16_bits_to_f64(dm), SB, axis=1) * np.repeat(mn.astype(np.float64), 32, axis=1))
    Ad = np.repeat(f16_bits_to_f64(d16), 32, axis=1) * q.astype(np.float64)
    yref = Ad @ Wd.T
    y, awa = o.matmul_q5_k(qw, sc, mn, dd, dm, q, d16)
    ok18 &= bool((np.abs(y.astype(np.float64) - yref) <= np.spacing(np.abs(yref).astype(np.float32))).all())
    ok18 &= bool(np.allclose(awa, np.abs(Ad) @ np.abs(Wd).T, rtol=1e-12, atol=0))
    d16x = (f16_bits_to_f64(dd) * 16.0).astype(np.float16).view(np.uint16)    # exact: a power of two
    ylo, _ = o.matmul_q4_k(qw & 15, sc, mn, dd, dm, q, d16)
    yhi, _ = o.matmul_q4_k(qw >> 4, sc, np.zeros_like(mn), d16x, np.zeros_like(dm), q, d16)
    ysplit = ylo.astype(np.float64) + yhi.astype(np.float64)
    ok18 &= bool((np.abs(y.astype(np.float64) - ysplit) <= 4 * np.spacing(np.abs(awa).astype(np.float32))).all())
    pin("q5_k_bruteforce_and_fifth_bit_split", ok18)

    # P19: Q6_K (the GGML format's reading) -- per-16 sums and y by brute force on its
    # definition (one signed scale per 16 weights, codes offset by 32), the reduction to
    # Q4_K when every code lies in 32..47 and the two 16-scales of each 32-block are equal
    # (codes c - 32, mins 0), and the sign symmetry c -> 64 - c, which negates y exactly
    r = _rng(21)
    M, N, K = 3, 4, 2 * SB
    qw = r.integers(0, 64, (N, K), dtype=np.uint8)
    sc = r.integers(-128, 128, (N, K // 16)).astype(np.int8)
    dd = r.uniform(2e-6, 3e-5, (N, K // SB)).astype(np.float16).view(np.uint16)
    x = r.standard_normal((M, K)).astype(np.float32)
    q, d16, bs = o.quantize_q8_0(x)
    Cq = qw.astype(np.int64) - 32
    isum_ref = (q.astype(np.int64)[:, None, :] * Cq[None]).reshape(M, N, K // 16, 16).sum(axis=3)
    ok19 = bool((o.isums_q6_k(qw, q) == isum_ref).all())
    Wd = (np.repeat(f16_bits_to_f64(dd), SB, axis=1) * np.repeat(sc.astype(np.float64), 16, axis=1)
          * Cq.astype(np.float64))
    Ad = np.repeat(f16_bits_to_f64(d16), 32, axis=1) * q.astype(np.float64)
    yref = Ad @ Wd.T
    y, awa = o.matmul_q6_k(qw, sc, dd, q, d16)
    ok19 &= bool((np.abs(y.astype(np.float64) - yref) <= np.spacing(np.abs(yref).astype(np.float32))).all())
    ok19 &= bool(np.allclose(awa, np.abs(Ad) @ np.abs(Wd).T, rtol=1e-12, atol=0))
    c4 = r.integers(32, 48, (N, K), dtype=np.uint8)
    s32 = r.integers(0, 64, (N, K // 32), dtype=np.uint8)
    y6, _ = o.matmul_q6_k(c4, np.repeat(s32, 2, axis=1).astype(np.int8), dd, q, d16)
    y4, _ = o.matmul_q4_k(c4 - 32, s32, np.zeros_like(s32), dd, np.zeros_like(dd), q, d16)
    ok19 &= bool((y6 == y4).all())
    c1 = r.integers(1, 64, (N, K), dtype=np.uint8)
    yp, _ = o.matmul_q6_k(c1, sc, dd, q, d16)
    yn, _ = o.matmul_q6_k((64 - c1.astype(np.int32)).astype(np.uint8), sc, dd, q, d16)
    ok19 &= bool((yn == -yp).all())
    pin("q6_k_bruteforce_q4_k_reduction_sign_symmetry", ok19)
    return out
