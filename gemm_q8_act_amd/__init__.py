"""gemm_q8_act_amd -- Python binding of libnvq, the MI355X (gfx950) library for
NVFP4, Q4_1, Q4_K and IQ4_XS x Q8_0 quantized matrix products.

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
NVQ_FMT_Q4_K = 2
NVQ_FMT_IQ4_XS = 3
NVQ_FMT_Q5_K = 4
NVQ_FMT_Q6_K = 5
NVQ_PATH_GEMV = 0
NVQ_PATH_GEMM = 1
NVQ_PATH_GEMV_DOT4 = 2
NVQ_GEMV_MAX_M = 15

# Every symbol include/nvq.h and include/nvq_probe.h declare.
EXPORTS = (
    "nvq_nvfp4_weight_bytes", "nvq_q4_1_weight_bytes", "nvq_q4_k_weight_bytes", "nvq_iq4_xs_weight_bytes",
    "nvq_gemm_workspace_bytes",
    "nvq_pack_nvfp4", "nvq_pack_q4_1", "nvq_pack_q4_k", "nvq_pack_iq4_xs", "nvq_quantize_act_q8_0", "nvq_gemv_nvfp4",
    "nvq_gemv_nvfp4_fused", "nvq_gemv_nvfp4_dot4",
    "nvq_gemv_nvfp4_routed", "nvq_gemm_nvfp4", "nvq_gemm_nvfp4_noalloc", "nvq_gemv_q4_1", "nvq_gemm_q4_1",
    "nvq_gemv_q4_k", "nvq_gemm_q4_k", "nvq_gemv_iq4_xs", "nvq_gemm_iq4_xs", "nvq_debug_isums",
    "nvq_debug_isums_iq4_xs",
    "nvq_q5_k_weight_bytes", "nvq_q6_k_weight_bytes", "nvq_pack_q5_k", "nvq_pack_q6_k",
    "nvq_gemv_q5_k", "nvq_gemm_q5_k", "nvq_gemv_q6_k", "nvq_gemm_q6_k",
    "nvq_status_str", "nvq_last_error",
    "nvq_probe_read", "nvq_probe_gemv_loads", "nvq_probe_mfma",
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
        # torch first: it loads its own HIP runtime (soname libamdhip64.so.7), which
        # libnvq's dependency then resolves to, so the process has one runtime and the
        # library sees torch's devices, memory and streams.  Loaded the other way round,
        # torch would bring a second runtime and libnvq's would find no device.
        import torch  # noqa: F401

        L = ctypes.CDLL(LIB_PATH)
        P, I64, SZ, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        sigs = {
            "nvq_nvfp4_weight_bytes": (SZ, [I64, I64]),
            "nvq_q4_1_weight_bytes": (SZ, [I64, I64]),
            "nvq_q4_k_weight_bytes": (SZ, [I64, I64]),
            "nvq_iq4_xs_weight_bytes": (SZ, [I64, I64]),
            "nvq_gemm_workspace_bytes": (SZ, [ctypes.c_int, I64, I64, I64]),
            "nvq_pack_nvfp4": (ctypes.c_int, [P, P, I64, I64, P]),
            "nvq_pack_q4_1": (ctypes.c_int, [P, P, P, I64, I64, P]),
            "nvq_pack_q4_k": (ctypes.c_int, [P, P, P, P, P, I64, I64, P]),
            "nvq_pack_iq4_xs": (ctypes.c_int, [P, P, P, I64, I64, P]),
            "nvq_quantize_act_q8_0": (ctypes.c_int, [P, I64, I64, P, P, P, P]),
            "nvq_gemv_nvfp4": (ctypes.c_int, [P, F, P, P, I64, I64, I64, P, P]),
            "nvq_gemv_nvfp4_fused": (ctypes.c_int, [P, F, P, I64, I64, P, P, P, P]),
            "nvq_gemv_nvfp4_dot4": (ctypes.c_int, [P, F, P, P, I64, I64, I64, P, P]),
            "nvq_gemv_nvfp4_routed": (ctypes.c_int, [P, P, P, I64, I64, P, P, I64, I64, I64, P, P]),
            "nvq_gemm_nvfp4": (ctypes.c_int, [P, F, P, P, I64, I64, I64, P, P, SZ, P]),
            "nvq_gemm_nvfp4_noalloc": (ctypes.c_int, [P, F, P, P, I64, I64, I64, P, P]),
            "nvq_gemv_q4_1": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, P]),
            "nvq_gemm_q4_1": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, P, SZ, P]),
            "nvq_gemv_q4_k": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, P]),
            "nvq_gemm_q4_k": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, P, SZ, P]),
            "nvq_gemv_iq4_xs": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, P]),
            "nvq_gemm_iq4_xs": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, P, SZ, P]),
            "nvq_debug_isums_iq4_xs": (ctypes.c_int, [P, ctypes.c_int, P, P, I64, I64, I64, P, P]),
            "nvq_debug_isums": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, P, P, I64, I64, I64, P, P]),
            "nvq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
            "nvq_last_error": (ctypes.c_char_p, []),
            "nvq_q5_k_weight_bytes": (SZ, [I64, I64]),
            "nvq_q6_k_weight_bytes": (SZ, [I64, I64]),
            "nvq_pack_q5_k": (ctypes.c_int, [P, P, P, P, P, I64, I64, P]),
            "nvq_pack_q6_k": (ctypes.c_int, [P, P, P, I64, I64, P]),
            "nvq_gemv_q5_k": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, P]),
            "nvq_gemm_q5_k": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, P, SZ, P]),
            "nvq_gemv_q6_k": (ctypes.c_int, [P, P, P, I64, I64, I64, P, P]),
            "nvq_gemm_q6_k": (ctypes.c_int, [P, P, P, I64, I64, I64, P, P, SZ, P]),
            "nvq_probe_read": (ctypes.c_int, [P, SZ, ctypes.c_int, P, P]),
            "nvq_probe_gemv_loads": (ctypes.c_int, [P, I64, I64, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]),
            "nvq_probe_mfma": (ctypes.c_int, [ctypes.c_int, I64, ctypes.c_int, P, P]),
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


def nvq_q4_k_weight_bytes(N: int, K: int) -> int:
    return int(lib().nvq_q4_k_weight_bytes(N, K))


def nvq_iq4_xs_weight_bytes(N: int, K: int) -> int:
    return int(lib().nvq_iq4_xs_weight_bytes(N, K))


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


def nvq_gemv_nvfp4_fused(w, w_scale: float, x, y, q_out=None, d_out=None, stream=None) -> None:
    """One token: x float32 [1, K] (or [K]) -> y float32 [1, N] (or [N]), Q8_0
    quantization inside the GEMV launch; q_out int8 [.., K] / d_out 2-byte [.., K/32]
    optionally receive the codes and scales."""
    import torch

    K = x.shape[-1]
    N = y.shape[-1]
    if x.numel() != K or y.numel() != N:
        raise ValueError("nvq_gemv_nvfp4_fused takes one token: x [K] or [1, K], y [N] or [1, N]")
    _need(x, torch.float32, tuple(x.shape), "x")
    _need(y, torch.float32, tuple(y.shape), "y")
    if (q_out is None) != (d_out is None):
        raise ValueError("q_out and d_out are given together or not at all")
    if q_out is not None:
        if q_out.dtype != torch.int8 or q_out.numel() != K:
            raise ValueError("q_out: int8 tensor of K elements required")
        if d_out.element_size() != 2 or d_out.numel() != K // 32:
            raise ValueError("d_out: 2-byte tensor of K/32 elements required")
    _weights(w, nvq_nvfp4_weight_bytes(N, K), "w")
    _check(lib().nvq_gemv_nvfp4_fused(_ptr(w), float(w_scale), _ptr(x), N, K, _ptr(y), _ptr(q_out), _ptr(d_out),
                                      _stream(stream, y)), "nvq_gemv_nvfp4_fused")


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


def nvq_gemm_nvfp4_noalloc(w, w_scale: float, q, d_f16, y, stream=None) -> None:
    """nvq_gemm_nvfp4 with its K-split partials in the library's static per-GPU scratch
    (nothing allocated; calls on one GPU must not overlap in time)."""
    import torch

    M, K = _acts(q, d_f16)
    N = y.shape[1]
    _need(y, torch.float32, (M, N), "y")
    _weights(w, nvq_nvfp4_weight_bytes(N, K), "w")
    _check(lib().nvq_gemm_nvfp4_noalloc(_ptr(w), float(w_scale), _ptr(q), _ptr(d_f16), M, N, K, _ptr(y),
                                        _stream(stream, y)), "nvq_gemm_nvfp4_noalloc")


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


def nvq_pack_q4_k(q: np.ndarray, sc: np.ndarray, mn: np.ndarray, d_f16: np.ndarray,
                  dmin_f16: np.ndarray) -> np.ndarray:
    """q uint8 [N, K] (0..15), sc / mn uint8 [N, K/32] (0..63), d_f16 / dmin_f16 uint16
    [N, K/256] -> packed uint8 buffer."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    sc = np.ascontiguousarray(sc, dtype=np.uint8)
    mn = np.ascontiguousarray(mn, dtype=np.uint8)
    d_f16 = np.ascontiguousarray(d_f16, dtype=np.uint16)
    dmin_f16 = np.ascontiguousarray(dmin_f16, dtype=np.uint16)
    N, K = q.shape
    if sc.shape != (N, K // 32) or mn.shape != (N, K // 32):
        raise ValueError("sc and mn must be [N, K/32]")
    if d_f16.shape != (N, K // 256) or dmin_f16.shape != (N, K // 256):
        raise ValueError("d_f16 and dmin_f16 must be [N, K/256]")
    nbytes = nvq_q4_k_weight_bytes(N, K)
    out = np.empty(max(nbytes, 1), np.uint8)
    _check(lib().nvq_pack_q4_k(*(a.ctypes.data_as(ctypes.c_void_p) for a in (q, sc, mn, d_f16, dmin_f16)), N, K,
                               out.ctypes.data_as(ctypes.c_void_p)), "nvq_pack_q4_k")
    return out[:nbytes]


def nvq_gemv_q4_k(w, q, d_f16, bsum16, y, stream=None) -> None:
    import torch

    M, K = _acts(q, d_f16)
    N = y.shape[1]
    _need(y, torch.float32, (M, N), "y")
    _need(bsum16, torch.int16, (M, K // 16), "bsum16")
    _weights(w, nvq_q4_k_weight_bytes(N, K), "w")
    _check(lib().nvq_gemv_q4_k(_ptr(w), _ptr(q), _ptr(d_f16), _ptr(bsum16), M, N, K, _ptr(y),
                               _stream(stream, y)), "nvq_gemv_q4_k")


def nvq_gemm_q4_k(w, q, d_f16, bsum16, y, workspace=None, stream=None) -> None:
    import torch

    M, K = _acts(q, d_f16)
    N = y.shape[1]
    _need(y, torch.float32, (M, N), "y")
    _need(bsum16, torch.int16, (M, K // 16), "bsum16")
    _weights(w, nvq_q4_k_weight_bytes(N, K), "w")
    if workspace is None:
        need = lib().nvq_gemm_workspace_bytes(NVQ_FMT_Q4_K, M, N, K)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=y.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().nvq_gemm_q4_k(_ptr(w), _ptr(q), _ptr(d_f16), _ptr(bsum16), M, N, K, _ptr(y),
                               _ptr(workspace), ws_bytes, _stream(stream, y)), "nvq_gemm_q4_k")


def nvq_q5_k_weight_bytes(N: int, K: int) -> int:
    return int(lib().nvq_q5_k_weight_bytes(N, K))


def nvq_q6_k_weight_bytes(N: int, K: int) -> int:
    return int(lib().nvq_q6_k_weight_bytes(N, K))


def nvq_pack_q5_k(q: np.ndarray, sc: np.ndarray, mn: np.ndarray, d_f16: np.ndarray,
                  dmin_f16: np.ndarray) -> np.ndarray:
    """q uint8 [N, K] (0..31), sc / mn uint8 [N, K/32] (0..63), d_f16 / dmin_f16 uint16
    [N, K/256] -> packed uint8 buffer."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    sc = np.ascontiguousarray(sc, dtype=np.uint8)
    mn = np.ascontiguousarray(mn, dtype=np.uint8)
    d_f16 = np.ascontiguousarray(d_f16, dtype=np.uint16)
    dmin_f16 = np.ascontiguousarray(dmin_f16, dtype=np.uint16)
    N, K = q.shape
    if sc.shape != (N, K // 32) or mn.shape != (N, K // 32):
        raise ValueError("sc and mn must be [N, K/32]")
    if d_f16.shape != (N, K // 256) or dmin_f16.shape != (N, K // 256):
        raise ValueError("d_f16 and dmin_f16 must be [N, K/256]")
    nbytes = nvq_q5_k_weight_bytes(N, K)
    out = np.empty(max(nbytes, 1), np.uint8)
    _check(lib().nvq_pack_q5_k(*(a.ctypes.data_as(ctypes.c_void_p) for a in (q, sc, mn, d_f16, dmin_f16)), N, K,
                               out.ctypes.data_as(ctypes.c_void_p)), "nvq_pack_q5_k")
    return out[:nbytes]


def nvq_pack_q6_k(q: np.ndarray, sc: np.ndarray, d_f16: np.ndarray) -> np.ndarray:
    """q uint8 [N, K] (0..63), sc int8 [N, K/16], d_f16 uint16 [N, K/256] -> packed uint8
    buffer."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    sc = np.ascontiguousarray(sc, dtype=np.int8)
    d_f16 = np.ascontiguousarray(d_f16, dtype=np.uint16)
    N, K = q.shape
    if sc.shape != (N, K // 16) or d_f16.shape != (N, K // 256):
        raise ValueError("sc must be [N, K/16] and d_f16 [N, K/256]")
    nbytes = nvq_q6_k_weight_bytes(N, K)
    out = np.empty(max(nbytes, 1), np.uint8)
    _check(lib().nvq_pack_q6_k(*(a.ctypes.data_as(ctypes.c_void_p) for a in (q, sc, d_f16)), N, K,
                               out.ctypes.data_as(ctypes.c_void_p)), "nvq_pack_q6_k")
    return out[:nbytes]


def nvq_gemv_q5_k(w, q, d_f16, bsum16, y, stream=None) -> None:
    import torch

    M, K = _acts(q, d_f16)
    N = y.shape[1]
    _need(y, torch.float32, (M, N), "y")
    _need(bsum16, torch.int16, (M, K // 16), "bsum16")
    _weights(w, nvq_q5_k_weight_bytes(N, K), "w")
    _check(lib().nvq_gemv_q5_k(_ptr(w), _ptr(q), _ptr(d_f16), _ptr(bsum16), M, N, K, _ptr(y),
                               _stream(stream, y)), "nvq_gemv_q5_k")


def nvq_gemm_q5_k(w, q, d_f16, bsum16, y, workspace=None, stream=None) -> None:
    import torch

    M, K = _acts(q, d_f16)
    N = y.shape[1]
    _need(y, torch.float32, (M, N), "y")
    _need(bsum16, torch.int16, (M, K // 16), "bsum16")
    _weights(w, nvq_q5_k_weight_bytes(N, K), "w")
    if workspace is None:
        need = lib().nvq_gemm_workspace_bytes(NVQ_FMT_Q5_K, M, N, K)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=y.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().nvq_gemm_q5_k(_ptr(w), _ptr(q), _ptr(d_f16), _ptr(bsum16), M, N, K, _ptr(y),
                               _ptr(workspace), ws_bytes, _stream(stream, y)), "nvq_gemm_q5_k")


def nvq_gemv_q6_k(w, q, d_f16, y, stream=None) -> None:
    import torch

    M, K = _acts(q, d_f16)
    N = y.shape[1]
    _need(y, torch.float32, (M, N), "y")
    _weights(w, nvq_q6_k_weight_bytes(N, K), "w")
    _check(lib().nvq_gemv_q6_k(_ptr(w), _ptr(q), _ptr(d_f16), M, N, K, _ptr(y), _stream(stream, y)),
           "nvq_gemv_q6_k")


def nvq_gemm_q6_k(w, q, d_f16, y, workspace=None, stream=None) -> None:
    import torch

    M, K = _acts(q, d_f16)
    N = y.shape[1]
    _need(y, torch.float32, (M, N), "y")
    _weights(w, nvq_q6_k_weight_bytes(N, K), "w")
    if workspace is None:
        need = lib().nvq_gemm_workspace_bytes(NVQ_FMT_Q6_K, M, N, K)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=y.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().nvq_gemm_q6_k(_ptr(w), _ptr(q), _ptr(d_f16), M, N, K, _ptr(y), _ptr(workspace), ws_bytes,
                               _stream(stream, y)), "nvq_gemm_q6_k")


def nvq_pack_iq4_xs(q: np.ndarray, ls: np.ndarray, d_f16: np.ndarray) -> np.ndarray:
    """q uint8 [N, K] (0..15), ls uint8 [N, K/32] (0..63), d_f16 uint16 [N, K/256] ->
    packed uint8 buffer (the value table is passed to the products)."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    ls = np.ascontiguousarray(ls, dtype=np.uint8)
    d_f16 = np.ascontiguousarray(d_f16, dtype=np.uint16)
    N, K = q.shape
    if ls.shape != (N, K // 32) or d_f16.shape != (N, K // 256):
        raise ValueError("ls must be [N, K/32] and d_f16 [N, K/256]")
    nbytes = nvq_iq4_xs_weight_bytes(N, K)
    out = np.empty(max(nbytes, 1), np.uint8)
    _check(lib().nvq_pack_iq4_xs(*(a.ctypes.data_as(ctypes.c_void_p) for a in (q, ls, d_f16)), N, K,
                                 out.ctypes.data_as(ctypes.c_void_p)), "nvq_pack_iq4_xs")
    return out[:nbytes]


def _table(table) -> np.ndarray:
    t = np.ascontiguousarray(table, dtype=np.int8)
    if t.shape != (16,):
        raise ValueError("table must hold 16 int8 values")
    return t


def nvq_gemv_iq4_xs(w, table, q, d_f16, y, stream=None) -> None:
    import torch

    t = _table(table)
    M, K = _acts(q, d_f16)
    N = y.shape[1]
    _need(y, torch.float32, (M, N), "y")
    _weights(w, nvq_iq4_xs_weight_bytes(N, K), "w")
    _check(lib().nvq_gemv_iq4_xs(_ptr(w), t.ctypes.data_as(ctypes.c_void_p), _ptr(q), _ptr(d_f16), M, N, K, _ptr(y),
                                 _stream(stream, y)), "nvq_gemv_iq4_xs")


def nvq_gemm_iq4_xs(w, table, q, d_f16, y, workspace=None, stream=None) -> None:
    import torch

    t = _table(table)
    M, K = _acts(q, d_f16)
    N = y.shape[1]
    _need(y, torch.float32, (M, N), "y")
    _weights(w, nvq_iq4_xs_weight_bytes(N, K), "w")
    if workspace is None:
        need = lib().nvq_gemm_workspace_bytes(NVQ_FMT_IQ4_XS, M, N, K)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=y.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().nvq_gemm_iq4_xs(_ptr(w), t.ctypes.data_as(ctypes.c_void_p), _ptr(q), _ptr(d_f16), M, N, K, _ptr(y),
                                 _ptr(workspace), ws_bytes, _stream(stream, y)), "nvq_gemm_iq4_xs")


def nvq_debug_isums_iq4_xs(table, path: int, w, q, N: int, isums, stream=None) -> None:
    """isums int32 [M, N, K/16]: sum of table[code] * q per 16, from the dispatched kernel."""
    import torch

    t = _table(table)
    M, K = q.shape
    _need(q, torch.int8, (M, K), "q")
    _need(isums, torch.int32, (M, N, K // 16), "isums")
    _weights(w, nvq_iq4_xs_weight_bytes(N, K), "w")
    _check(lib().nvq_debug_isums_iq4_xs(t.ctypes.data_as(ctypes.c_void_p), int(path), _ptr(w), _ptr(q), M, N, K,
                                        _ptr(isums), _stream(stream, q)), "nvq_debug_isums_iq4_xs")


def nvq_debug_isums(fmt: int, path: int, w, q, N: int, isums, stream=None) -> None:
    """isums int32 [M, N, K/16]: integer per-16 sums from the chosen production path."""
    import torch

    M, K = q.shape
    _need(q, torch.int8, (M, K), "q")
    _need(isums, torch.int32, (M, N, K // 16), "isums")
    nbytes = {NVQ_FMT_NVFP4: nvq_nvfp4_weight_bytes, NVQ_FMT_Q4_1: nvq_q4_1_weight_bytes,
              NVQ_FMT_Q4_K: nvq_q4_k_weight_bytes}.get(fmt, nvq_q4_1_weight_bytes)(N, K)
    _weights(w, nbytes, "w")
    _check(lib().nvq_debug_isums(int(fmt), int(path), _ptr(w), _ptr(q), M, N, K, _ptr(isums),
                                 _stream(stream, q)), "nvq_debug_isums")


# ---------------------------------------------------------------------------
# measurement probes (include/nvq_probe.h): ceilings, not part of the product path
# ---------------------------------------------------------------------------

def nvq_probe_read(src, blocks: int, sink, stream=None) -> None:
    """Stream every byte of the device tensor ``src`` (size a multiple of 16) with
    16-byte non-temporal loads over ``blocks`` blocks of 256 threads; ``sink``: int32
    or uint32 device tensor of >= 4 * blocks elements."""
    nbytes = src.numel() * src.element_size()
    if sink.element_size() != 4 or sink.numel() < 4 * blocks:
        raise ValueError("sink: 4-byte tensor of at least 4 * blocks elements required")
    _check(lib().nvq_probe_read(_ptr(src), nbytes, int(blocks), _ptr(sink), _stream(stream, src)), "nvq_probe_read")


def nvq_probe_gemv_loads(w, N: int, K: int, splits: int, waves: int, batch: int, sink, stream=None) -> None:
    """The weight loads of the single-token decode GEMV over packed NVFP4 ``w`` (N x K)
    and nothing else; ``sink``: 4-byte device tensor of >= waves * ceil(N/16) * splits
    elements."""
    _weights(w, nvq_nvfp4_weight_bytes(N, K), "w")
    if sink.element_size() != 4 or sink.numel() < waves * ((N + 15) // 16) * splits:
        raise ValueError("sink: 4-byte tensor of at least waves * ceil(N/16) * splits elements required")
    _check(lib().nvq_probe_gemv_loads(_ptr(w), int(N), int(K), int(splits), int(waves), int(batch), _ptr(sink),
                                      _stream(stream, w)), "nvq_probe_gemv_loads")


def nvq_probe_mfma(blocks: int, iters: int, random_operands: bool, out, stream=None) -> None:
    """Back-to-back v_mfma_f32_32x32x16_f16 on register operands; ``out``: float32
    device tensor of >= 256 * blocks elements.  Flops per call:
    blocks * 4 * 12 * iters * 32768."""
    import torch

    if out.dtype != torch.float32 or out.numel() < 256 * blocks:
        raise ValueError("out: float32 tensor of at least 256 * blocks elements required")
    _check(lib().nvq_probe_mfma(int(blocks), int(iters), 1 if random_operands else 0, _ptr(out), _stream(stream, out)),
           "nvq_probe_mfma")
