"""gemm_q8_act_amd -- Python binding of libnvq, the MI355X (gfx950) library for
NVFP4 x Q8_0 and Q4_1 x Q8_0 quantized matrix products.

This module only marshals arguments: every step of the computation runs in the
HIP kernels of ``libnvq.so`` behind the C ABI declared in ``include/nvq.h``.  The
functions keep the C names.  Device buffers are torch tensors (torch is used for
device memory and streams only); their data pointers and the current HIP stream
are passed straight through.  There is no fallback: if the library is missing
every call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_DIR, "libnvq.so")

NVQ_OK = 0
NVQ_FMT_NVFP4 = 0
NVQ_FMT_Q4_1 = 1
NVQ_PATH_GEMV = 0
NVQ_PATH_GEMM = 1
NVQ_PATH_GEMV_DOT4 = 2
NVQ_GEMV_MAX_M = 15

# Every symbol include/nvq.h declares.
EXPORTS = (
    "nvq_nvfp4_weight_bytes", "nvq_q4_1_weight_bytes", "nvq_gemm_workspace_bytes",
    "nvq_pack_nvfp4", "nvq_pack_q4_1", "nvq_quantize_act_q8_0", "nvq_gemv_nvfp4", "nvq_gemv_nvfp4_dot4",
    "nvq_gemv_nvfp4_routed", "nvq_gemm_nvfp4", "nvq_gemv_q4_1", "nvq_gemm_q4_1", "nvq_debug_isums",
    "nvq_status_str", "nvq_last_error",
)


class NvqError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {status_str(status)} ({status}): {detail}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libnvq.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libnvq.so not built at {LIB_PATH}; run gemm_q8_act_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, SZ, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        sigs = {
            "nvq_nvfp4_weight_bytes": (SZ, [I64, I64]),
            "nvq_q4_1_weight_bytes": (SZ, [I64, I64]),
            "nvq_gemm_workspace_bytes": (SZ, [ctypes.c_int, I64, I64, I64]),
            "nvq_pack_nvfp4": (ctypes.c_int, [P, P, I64, I64, P]),
            "nvq_pack_q4_1": (ctypes.c_int, [P, P, P, I64, I64, P]),
            "nvq_quantize_act_q8_0": (ctypes.c_int, [P, I64, I64, P, P, P, P]),
            "nvq_gemv_nvfp4": (ctypes.c_int, [P, F, P, P, I64, I64, I64, P, P]),
            "nvq_gemv_nvfp4_dot4": (ctypes.c_int, [P, F, P, P, I64, I64, I64, P, P]),
            "nvq_gemv_nvfp4_routed": (ctypes.c_int, [P, P, P, I64, I64, P, P, I64, I64, I64, P, P]),
            "nvq_gemm_nvfp4": (ctypes.c_int, [P, F, P, P, I64, I64, I64, P, P, SZ, P]),
            "nvq_gemv_q4_1": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, P]),
            "nvq_gemm_q4_1": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, P, SZ, P]),
            "nvq_debug_isums": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, P, P, I64, I64, I64, P, P]),
            "nvq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
            "nvq_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_str(s: int) -> str:
    return lib().nvq_status_str(int(s)).decode()


def last_error() -> str:
    return lib().nvq_last_error().decode()


def _check(status: int, where: str) -> None:
    if status != NVQ_OK:
        raise NvqError(status, where, last_error())


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t):
    """Device address of a torch tensor (or None)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libnvq must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, *tensors):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch

    dev = next((t.device for t in tensors if t is not None and t.is_cuda), None)
    if dev is None:
        return None
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, dtype, shape, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


# ---------------------------------------------------------------------------
# sizes and packers (host)
# ---------------------------------------------------------------------------

def nvq_nvfp4_weight_bytes(N: int, K: int) -> int:
    return int(lib().nvq_nvfp4_weight_bytes(N, K))


def nvq_q4_1_weight_bytes(N: int, K: int) -> int:
    return int(lib().nvq_q4_1_weight_bytes(N, K))


def nvq_gemm_workspace_bytes(fmt: int, M: int, N: int, K: int) -> int:
    return int(lib().nvq_gemm_workspace_bytes(fmt, M, N, K))


def nvq_pack_nvfp4(codes: np.ndarray, ue4m3: np.ndarray) -> np.ndarray:
    """codes uint8 [N, K] (0..15), ue4m3 uint8 [N, K/16] -> packed uint8 buffer."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    ue4m3 = np.ascontiguousarray(ue4m3, dtype=np.uint8)
    N, K = codes.shape
    if ue4m3.shape != (N, K // 16):
        raise ValueError("ue4m3 must be [N, K/16]")
    nbytes = nvq_nvfp4_weight_bytes(N, K)
    out = np.empty(max(nbytes, 1), np.uint8)
    _check(lib().nvq_pack_nvfp4(codes.ctypes.data_as(ctypes.c_void_p), ue4m3.ctypes.data_as(ctypes.c_void_p),
                                N, K, out.ctypes.data_as(ctypes.c_void_p)), "nvq_pack_nvfp4")
    return out[:nbytes]


def nvq_pack_q4_1(q: np.ndarray, d_f16: np.ndarray, m_f16: np.ndarray) -> np.ndarray:
    """q uint8 [N, K] (0..15), d_f16 / m_f16 uint16 [N, K/32] -> packed uint8 buffer."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    d_f16 = np.ascontiguousarray(d_f16, dtype=np.uint16)
    m_f16 = np.ascontiguousarray(m_f16, dtype=np.uint16)
    N, K = q.shape
    if d_f16.shape != (N, K // 32) or m_f16.shape != (N, K // 32):
        raise ValueError("d_f16 and m_f16 must be [N, K/32]")
    nbytes = nvq_q4_1_weight_bytes(N, K)
    out = np.empty(max(nbytes, 1), np.uint8)
    _check(lib().nvq_pack_q4_1(q.ctypes.data_as(ctypes.c_void_p), d_f16.ctypes.data_as(ctypes.c_void_p),
                               m_f16.ctypes.data_as(ctypes.c_void_p), N, K,
                               out.ctypes.data_as(ctypes.c_void_p)), "nvq_pack_q4_1")
    return out[:nbytes]


# ---------------------------------------------------------------------------
# device entry points (torch tensors on the GPU)
# ---------------------------------------------------------------------------

def nvq_quantize_act_q8_0(x, q, d_f16, bsum16=None, stream=None) -> None:
    """x float32 [M, K] -> q int8 [M, K], d_f16 int16/uint16 bits [M, K/32], bsum16 int16 [M, K/16]."""
    import torch

    M, K = x.shape
    _need(x, torch.float32, (M, K), "x")
    _need(q, torch.int8, (M, K), "q")
    if d_f16 is None or tuple(d_f16.shape) != (M, K // 32) or d_f16.element_size() != 2:
        raise ValueError("d_f16 must be a 2-byte tensor [M, K/32]")
    if bsum16 is not None:
        _need(bsum16, torch.int16, (M, K // 16), "bsum16")
    _check(lib().nvq_quantize_act_q8_0(_ptr(x), M, K, _ptr(q), _ptr(d_f16), _ptr(bsum16),
                                       _stream(stream, x)), "nvq_quantize_act_q8_0")


def _weights(w, nbytes, name):
    import torch

    if w is None or w.dtype != torch.uint8 or w.numel() < nbytes:
        raise ValueError(f"{name}: packed uint8 weight buffer of >= {nbytes} bytes required")


def _acts(q, d_f16):
    import torch

    M, K = q.shape
    _need(q, torch.int8, (M, K), "q")
    if d_f16 is None or tuple(d_f16.shape) != (M, K // 32) or d_f16.element_size() != 2:
        raise ValueError("d_f16 must be a 2-byte tensor [M, K/32]")
    return M, K


def nvq_gemv_nvfp4(w, w_scale: float, q, d_f16, y, stream=None) -> None:
    import torch

    M, K = _acts(q, d_f16)
    N = y.shape[1]
    _need(y, torch.float32, (M, N), "y")
    _weights(w, nvq_nvfp4_weight_bytes(N, K), "w")
    _check(lib().nvq_gemv_nvfp4(_ptr(w), float(w_scale), _ptr(q), _ptr(d_f16), M, N, K, _ptr(y),
                                _stream(stream, y)), "nvq_gemv_nvfp4")


def nvq_gemv_nvfp4_routed(w, w_scales, ids, q, d_f16, y, stream=None) -> None:
    """w: uint8, n_experts packed [N][K] matrices back to back; w_scales float32
    [n_experts]; ids int32 [M, n_active]; q, d_f16 [M, K]; y float32 [M, n_active, N]."""
    import torch

    M, K = _acts(q, d_f16)
    E = w_scales.shape[0]
    _need(w_scales, torch.float32, (E,), "w_scales")
    A = ids.shape[1] if ids is not None and ids.dim() == 2 else -1
    _need(ids, torch.int32, (M, A), "ids")
    N = y.shape[2]
    _need(y, torch.float32, (M, A, N), "y")
    _weights(w, E * nvq_nvfp4_weight_bytes(N, K), "w")
    _check(lib().nvq_gemv_nvfp4_routed(_ptr(w), _ptr(w_scales), _ptr(ids), E, A, _ptr(q), _ptr(d_f16), M, N, K,
                                       _ptr(y), _stream(stream, y)), "nvq_gemv_nvfp4_routed")


def nvq_gemv_nvfp4_dot4(w, w_scale: float, q, d_f16, y, stream=None) -> None:
    import torch

    M, K = _acts(q, d_f16)
    N = y.shape[1]
    _need(y, torch.float32, (M, N), "y")
    _weights(w, nvq_nvfp4_weight_bytes(N, K), "w")
    _check(lib().nvq_gemv_nvfp4_dot4(_ptr(w), float(w_scale), _ptr(q), _ptr(d_f16), M, N, K, _ptr(y),
                                     _stream(stream, y)), "nvq_gemv_nvfp4_dot4")


def nvq_gemm_nvfp4(w, w_scale: float, q, d_f16, y, workspace=None, stream=None) -> None:
    import torch

    M, K = _acts(q, d_f16)
    N = y.shape[1]
    _need(y, torch.float32, (M, N), "y")
    _weights(w, nvq_nvfp4_weight_bytes(N, K), "w")
    if workspace is None:  # the split-K partial tiles; torch's caching allocator makes this cheap
        need = lib().nvq_gemm_workspace_bytes(NVQ_FMT_NVFP4, M, N, K)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=y.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().nvq_gemm_nvfp4(_ptr(w), float(w_scale), _ptr(q), _ptr(d_f16), M, N, K, _ptr(y),
                                _ptr(workspace), ws_bytes, _stream(stream, y)), "nvq_gemm_nvfp4")


def nvq_gemv_q4_1(w, q, d_f16, bsum16, y, stream=None) -> None:
    import torch

    M, K = _acts(q, d_f16)
    N = y.shape[1]
    _need(y, torch.float32, (M, N), "y")
    _need(bsum16, torch.int16, (M, K // 16), "bsum16")
    _weights(w, nvq_q4_1_weight_bytes(N, K), "w")
    _check(lib().nvq_gemv_q4_1(_ptr(w), _ptr(q), _ptr(d_f16), _ptr(bsum16), M, N, K, _ptr(y),
                               _stream(stream, y)), "nvq_gemv_q4_1")


def nvq_gemm_q4_1(w, q, d_f16, bsum16, y, workspace=None, stream=None) -> None:
    import torch

    M, K = _acts(q, d_f16)
    N = y.shape[1]
    _need(y, torch.float32, (M, N), "y")
    _need(bsum16, torch.int16, (M, K // 16), "bsum16")
    _weights(w, nvq_q4_1_weight_bytes(N, K), "w")
    if workspace is None:
        need = lib().nvq_gemm_workspace_bytes(NVQ_FMT_Q4_1, M, N, K)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=y.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().nvq_gemm_q4_1(_ptr(w), _ptr(q), _ptr(d_f16), _ptr(bsum16), M, N, K, _ptr(y),
                               _ptr(workspace), ws_bytes, _stream(stream, y)), "nvq_gemm_q4_1")


def nvq_debug_isums(fmt: int, path: int, w, q, N: int, isums, stream=None) -> None:
    """isums int32 [M, N, K/16]: integer per-16 sums from the chosen production path."""
    import torch

    M, K = q.shape
    _need(q, torch.int8, (M, K), "q")
    _need(isums, torch.int32, (M, N, K // 16), "isums")
    nbytes = nvq_nvfp4_weight_bytes(N, K) if fmt == NVQ_FMT_NVFP4 else nvq_q4_1_weight_bytes(N, K)
    _weights(w, nbytes, "w")
    _check(lib().nvq_debug_isums(int(fmt), int(path), _ptr(w), _ptr(q), M, N, K, _ptr(isums),
                                 _stream(stream, q)), "nvq_debug_isums")
