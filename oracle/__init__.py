"""Plain-C oracle for the NVFP4, Q4_1, Q4_K, Q5_K, Q6_K and IQ4_XS x Q8_0 quantized matrix product.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never calls
it and shares no code with it; the oracle in turn knows nothing of the GPU
library's packed layout.  It works on the logical representation:

* NVFP4 weights: ``codes`` uint8 [N, K] (one 4-bit E2M1 code per byte, 0..15),
  ``scales`` uint8 [N, K/16] (UE4M3), one float32 per-tensor scale.
* Q4_1 weights: ``qw`` uint8 [N, K] (0..15), ``dw``/``mw`` uint16 [N, K/32]
  (binary16 bits of d and m).
* Q4_K weights: ``qw`` uint8 [N, K] (0..15), ``sc``/``mn`` uint8 [N, K/32] (6-bit
  sub-block scales and mins), ``d``/``dmin`` uint16 [N, K/256] (binary16 bits).
* Q5_K weights: as Q4_K with ``qw`` 0..31.
* Q6_K weights: ``qw`` uint8 [N, K] (0..63, used as qw - 32), ``sc`` int8 [N, K/16],
  ``d`` uint16 [N, K/256].
* IQ4_XS weights: ``qw`` uint8 [N, K] (0..15, indices into ``table`` int8 [16]),
  ``ls`` uint8 [N, K/32] (6-bit sub-block scales, used as ls - 32), ``d`` uint16
  [N, K/256].
* Q8_0 activations: ``q`` int8 [M, K], ``d16`` uint16 [M, K/32], ``bsum16``
  int16 [M, K/16].

The arithmetic lives in ``nvq_oracle.c`` (scalar C99, double accumulation); this
file only marshals numpy arrays through ctypes and compiles the C source with gcc.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_DIR, "nvq_oracle.c")
LIB_PATH = os.path.join(_DIR, "libnvq_oracle.so")
# Plain scalar build: no vectorisation, no FMA contraction, no fast-math.
CFLAGS = ["-std=c99", "-O2", "-fno-tree-vectorize", "-ffp-contract=off", "-fPIC", "-shared"]


def build(out: str = LIB_PATH, src: str = SRC, extra_flags=()) -> str:
    """Compile the oracle into a shared library (gcc, plain scalar flags)."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra_flags, "-I", _DIR, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library not built: {path} (run oracle.build())")
        lib = ctypes.CDLL(path)
        lib.nvqo_e2m1.restype = ctypes.c_double
        lib.nvqo_e2m1.argtypes = [ctypes.c_int]
        lib.nvqo_ue4m3.restype = ctypes.c_double
        lib.nvqo_ue4m3.argtypes = [ctypes.c_int]
        lib.nvqo_f16_to_f64.restype = ctypes.c_double
        lib.nvqo_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.nvqo_f32_to_f16.restype = ctypes.c_uint16
        lib.nvqo_f32_to_f16.argtypes = [ctypes.c_float]
        lib.nvqo_quantize_q8_0.restype = None
        lib.nvqo_quantize_q8_0.argtypes = [_P, _I64, _I64, _P, _P, _P]
        for name in ("nvqo_isums_nvfp4", "nvqo_isums_q4_1"):
            f = getattr(lib, name)
            f.restype = None
            f.argtypes = [_P, _P, _I64, _I64, _I64, _P]
        lib.nvqo_matmul_nvfp4.restype = None
        lib.nvqo_matmul_nvfp4.argtypes = [_P, _P, ctypes.c_float, _P, _P, _I64, _I64, _I64,
                                          _P, _I64, _P, _P]
        lib.nvqo_matmul_nvfp4_routed.restype = None
        lib.nvqo_matmul_nvfp4_routed.argtypes = [_P, _P, _P, _P, _I64, _I64, _P, _P, _I64, _I64, _I64,
                                                 _P, _I64, _P, _P]
        lib.nvqo_matmul_q4_1.restype = None
        lib.nvqo_matmul_q4_1.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _P]
        lib.nvqo_isums_iq4_xs.restype = None
        lib.nvqo_isums_iq4_xs.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P]
        lib.nvqo_matmul_iq4_xs.restype = None
        lib.nvqo_matmul_iq4_xs.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _P]
        lib.nvqo_matmul_q4_k.restype = None
        lib.nvqo_matmul_q4_k.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _P]
        lib.nvqo_matmul_q5_k.restype = None
        lib.nvqo_matmul_q5_k.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _P]
        lib.nvqo_isums_q6_k.restype = None
        lib.nvqo_isums_q6_k.argtypes = [_P, _P, _I64, _I64, _I64, _P]
        lib.nvqo_matmul_q6_k.restype = None
        lib.nvqo_matmul_q6_k.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _P]
        self.lib = lib
        self.path = path

    # -- element decodes ------------------------------------------------------
    def e2m1(self, code: int) -> float:
        return self.lib.nvqo_e2m1(int(code))

    def ue4m3(self, byte: int) -> float:
        return self.lib.nvqo_ue4m3(int(byte))

    def f16_to_f64(self, bits: int) -> float:
        return self.lib.nvqo_f16_to_f64(int(bits))

    def f32_to_f16(self, x: float) -> int:
        return int(self.lib.nvqo_f32_to_f16(float(np.float32(x))))

    # -- Q8_0 --------------------------------------------------------------------
    def quantize_q8_0(self, x: np.ndarray):
        x = np.ascontiguousarray(x, dtype=np.float32)
        M, K = x.shape
        assert K % 32 == 0
        q = np.empty((M, K), np.int8)
        d16 = np.empty((M, K // 32), np.uint16)
        bsum = np.empty((M, K // 16), np.int16)
        self.lib.nvqo_quantize_q8_0(_ptr(x), M, K, _ptr(q), _ptr(d16), _ptr(bsum))
        return q, d16, bsum

    # -- NVFP4 -------------------------------------------------------------------
    def isums_nvfp4(self, codes: np.ndarray, q: np.ndarray) -> np.ndarray:
        codes = np.ascontiguousarray(codes, np.uint8)
        q = np.ascontiguousarray(q, np.int8)
        N, K = codes.shape
        M = q.shape[0]
        out = np.empty((M, N, K // 16), np.int32)
        self.lib.nvqo_isums_nvfp4(_ptr(codes), _ptr(q), M, N, K, _ptr(out))
        return out

    def matmul_nvfp4(self, codes, scales, w_scale, q, d16, cols=None):
        """Returns (y float32 [M, ncols], abs_wa float64 [M, ncols])."""
        codes = np.ascontiguousarray(codes, np.uint8)
        scales = np.ascontiguousarray(scales, np.uint8)
        q = np.ascontiguousarray(q, np.int8)
        d16 = np.ascontiguousarray(d16, np.uint16)
        N, K = codes.shape
        M = q.shape[0]
        c = None if cols is None else np.ascontiguousarray(cols, np.int64)
        nc = N if c is None else len(c)
        y = np.empty((M, nc), np.float32)
        awa = np.empty((M, nc), np.float64)
        self.lib.nvqo_matmul_nvfp4(_ptr(codes), _ptr(scales), float(np.float32(w_scale)), _ptr(q),
                                   _ptr(d16), M, N, K, _ptr(c), nc, _ptr(y), _ptr(awa))
        return y, awa

    def matmul_nvfp4_routed(self, codes, scales, w_scales, ids, q, d16, cols=None):
        """codes [E, N, K], scales [E, N, K/16], w_scales [E], ids int32 [M, A].
        Returns (y float32 [M, A, ncols], abs_wa float64 [M, A, ncols])."""
        codes = np.ascontiguousarray(codes, np.uint8)
        scales = np.ascontiguousarray(scales, np.uint8)
        w_scales = np.ascontiguousarray(w_scales, np.float32)
        ids = np.ascontiguousarray(ids, np.int32)
        q = np.ascontiguousarray(q, np.int8)
        d16 = np.ascontiguousarray(d16, np.uint16)
        E, N, K = codes.shape
        M, A = ids.shape
        c = None if cols is None else np.ascontiguousarray(cols, np.int64)
        nc = N if c is None else len(c)
        y = np.empty((M, A, nc), np.float32)
        awa = np.empty((M, A, nc), np.float64)
        self.lib.nvqo_matmul_nvfp4_routed(_ptr(codes), _ptr(scales), _ptr(w_scales), _ptr(ids), E, A,
                                          _ptr(q), _ptr(d16), M, N, K, _ptr(c), nc, _ptr(y), _ptr(awa))
        return y, awa

    # -- Q4_1 --------------------------------------------------------------------
    def isums_q4_1(self, qw: np.ndarray, q: np.ndarray) -> np.ndarray:
        qw = np.ascontiguousarray(qw, np.uint8)
        q = np.ascontiguousarray(q, np.int8)
        N, K = qw.shape
        M = q.shape[0]
        out = np.empty((M, N, K // 16), np.int32)
        self.lib.nvqo_isums_q4_1(_ptr(qw), _ptr(q), M, N, K, _ptr(out))
        return out

    def matmul_q4_1(self, qw, dw, mw, q, d16, cols=None):
        qw = np.ascontiguousarray(qw, np.uint8)
        dw = np.ascontiguousarray(dw, np.uint16)
        mw = np.ascontiguousarray(mw, np.uint16)
        q = np.ascontiguousarray(q, np.int8)
        d16 = np.ascontiguousarray(d16, np.uint16)
        N, K = qw.shape
        M = q.shape[0]
        c = None if cols is None else np.ascontiguousarray(cols, np.int64)
        nc = N if c is None else len(c)
        y = np.empty((M, nc), np.float32)
        awa = np.empty((M, nc), np.float64)
        self.lib.nvqo_matmul_q4_1(_ptr(qw), _ptr(dw), _ptr(mw), _ptr(q), _ptr(d16), M, N, K,
                                  _ptr(c), nc, _ptr(y), _ptr(awa))
        return y, awa

    # -- Q4_K --------------------------------------------------------------------
    def isums_q4_k(self, qw: np.ndarray, q: np.ndarray) -> np.ndarray:
        """Per-16 sums of unsigned codes times activation codes: those of Q4_1."""
        return self.isums_q4_1(qw, q)

    def matmul_q4_k(self, qw, sc, mn, d, dmin, q, d16, cols=None):
        qw = np.ascontiguousarray(qw, np.uint8)
        sc = np.ascontiguousarray(sc, np.uint8)
        mn = np.ascontiguousarray(mn, np.uint8)
        d = np.ascontiguousarray(d, np.uint16)
        dmin = np.ascontiguousarray(dmin, np.uint16)
        q = np.ascontiguousarray(q, np.int8)
        d16 = np.ascontiguousarray(d16, np.uint16)
        N, K = qw.shape
        M = q.shape[0]
        assert K % 256 == 0 and sc.shape == (N, K // 32) and d.shape == (N, K // 256)
        c = None if cols is None else np.ascontiguousarray(cols, np.int64)
        nc = N if c is None else len(c)
        y = np.empty((M, nc), np.float32)
        awa = np.empty((M, nc), np.float64)
        self.lib.nvqo_matmul_q4_k(_ptr(qw), _ptr(sc), _ptr(mn), _ptr(d), _ptr(dmin), _ptr(q), _ptr(d16),
                                  M, N, K, _ptr(c), nc, _ptr(y), _ptr(awa))
        return y, awa

    # -- Q5_K --------------------------------------------------------------------
    def isums_q5_k(self, qw: np.ndarray, q: np.ndarray) -> np.ndarray:
        """Per-16 sums of the unsigned 5-bit codes times activation codes."""
        return self.isums_q4_1(qw, q)

    def matmul_q5_k(self, qw, sc, mn, d, dmin, q, d16, cols=None):
        qw = np.ascontiguousarray(qw, np.uint8)
        sc = np.ascontiguousarray(sc, np.uint8)
        mn = np.ascontiguousarray(mn, np.uint8)
        d = np.ascontiguousarray(d, np.uint16)
        dmin = np.ascontiguousarray(dmin, np.uint16)
        q = np.ascontiguousarray(q, np.int8)
        d16 = np.ascontiguousarray(d16, np.uint16)
        N, K = qw.shape
        M = q.shape[0]
        assert K % 256 == 0 and sc.shape == (N, K // 32) and d.shape == (N, K // 256)
        c = None if cols is None else np.ascontiguousarray(cols, np.int64)
        nc = N if c is None else len(c)
        y = np.empty((M, nc), np.float32)
        awa = np.empty((M, nc), np.float64)
        self.lib.nvqo_matmul_q5_k(_ptr(qw), _ptr(sc), _ptr(mn), _ptr(d), _ptr(dmin), _ptr(q), _ptr(d16),
                                  M, N, K, _ptr(c), nc, _ptr(y), _ptr(awa))
        return y, awa

    # -- Q6_K --------------------------------------------------------------------
    def isums_q6_k(self, qw: np.ndarray, q: np.ndarray) -> np.ndarray:
        """Per-16 sums of (code - 32) times activation codes."""
        qw = np.ascontiguousarray(qw, np.uint8)
        q = np.ascontiguousarray(q, np.int8)
        N, K = qw.shape
        M = q.shape[0]
        out = np.empty((M, N, K // 16), np.int32)
        self.lib.nvqo_isums_q6_k(_ptr(qw), _ptr(q), M, N, K, _ptr(out))
        return out

    def matmul_q6_k(self, qw, sc, d, q, d16, cols=None):
        qw = np.ascontiguousarray(qw, np.uint8)
        sc = np.ascontiguousarray(sc, np.int8)
        d = np.ascontiguousarray(d, np.uint16)
        q = np.ascontiguousarray(q, np.int8)
        d16 = np.ascontiguousarray(d16, np.uint16)
        N, K = qw.shape
        M = q.shape[0]
        assert K % 256 == 0 and sc.shape == (N, K // 16) and d.shape == (N, K // 256)
        c = None if cols is None else np.ascontiguousarray(cols, np.int64)
        nc = N if c is None else len(c)
        y = np.empty((M, nc), np.float32)
        awa = np.empty((M, nc), np.float64)
        self.lib.nvqo_matmul_q6_k(_ptr(qw), _ptr(sc), _ptr(d), _ptr(q), _ptr(d16), M, N, K,
                                  _ptr(c), nc, _ptr(y), _ptr(awa))
        return y, awa

    # -- IQ4_XS ------------------------------------------------------------------
    def isums_iq4_xs(self, qw: np.ndarray, table: np.ndarray, q: np.ndarray) -> np.ndarray:
        qw = np.ascontiguousarray(qw, np.uint8)
        table = np.ascontiguousarray(table, np.int8)
        q = np.ascontiguousarray(q, np.int8)
        N, K = qw.shape
        M = q.shape[0]
        assert table.shape == (16,)
        out = np.empty((M, N, K // 16), np.int32)
        self.lib.nvqo_isums_iq4_xs(_ptr(qw), _ptr(table), _ptr(q), M, N, K, _ptr(out))
        return out

    def matmul_iq4_xs(self, qw, ls, d, table, q, d16, cols=None):
        qw = np.ascontiguousarray(qw, np.uint8)
        ls = np.ascontiguousarray(ls, np.uint8)
        d = np.ascontiguousarray(d, np.uint16)
        table = np.ascontiguousarray(table, np.int8)
        q = np.ascontiguousarray(q, np.int8)
        d16 = np.ascontiguousarray(d16, np.uint16)
        N, K = qw.shape
        M = q.shape[0]
        assert K % 256 == 0 and ls.shape == (N, K // 32) and d.shape == (N, K // 256) and table.shape == (16,)
        c = None if cols is None else np.ascontiguousarray(cols, np.int64)
        nc = N if c is None else len(c)
        y = np.empty((M, nc), np.float32)
        awa = np.empty((M, nc), np.float64)
        self.lib.nvqo_matmul_iq4_xs(_ptr(qw), _ptr(ls), _ptr(d), _ptr(table), _ptr(q), _ptr(d16), M, N, K,
                                    _ptr(c), nc, _ptr(y), _ptr(awa))
        return y, awa

    # -- several host threads over disjoint output columns --------------------
    def matmul_threads(self, fmt: str, weights: tuple, q, d16, cols, threads: int):
        """Run matmul_<fmt> over ``cols`` split into ``threads`` disjoint slices, one
        host thread each (ctypes releases the GIL during the C call).  The per-output
        arithmetic is exactly the single-thread oracle's."""
        cols = np.asarray(cols, np.int64)
        parts = [p for p in np.array_split(cols, max(1, threads)) if len(p)]
        res = [None] * len(parts)
        fn = {"nvfp4": self.matmul_nvfp4, "q4_1": self.matmul_q4_1, "q4_k": self.matmul_q4_k}[fmt]

        def run(i):
            res[i] = fn(*weights, q, d16, cols=parts[i])

        ts = [threading.Thread(target=run, args=(i,)) for i in range(len(parts))]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        y = np.concatenate([r[0] for r in res], axis=1)
        awa = np.concatenate([r[1] for r in res], axis=1)
        return y, awa


_default: Oracle | None = None


def load(path: str = LIB_PATH) -> Oracle:
    """Load the oracle library, building it first if it is missing."""
    global _default
    if path == LIB_PATH:
        if _default is None:
            if not os.path.exists(LIB_PATH):
                build()
            _default = Oracle(LIB_PATH)
        return _default
    return Oracle(path)
