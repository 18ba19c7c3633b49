"""Python binding of libsvdq: the SVDQuant W4A4 linear layer on MI355X (gfx950).

Argument marshalling only: every step of the layer runs in libsvdq (the host
packing step in its C++ code, the activation step and the linear in its HIP
kernels).  There is no fallback: if the library cannot be loaded, or the GPU
is not a gfx950, the calls raise.

Functions mirror the C ABI in include/svdq.h:

    pack_weights(W, act_absmax, rank=32, prec=INT4)            host, numpy in/out
    pack_residual(W, smooth, down, up, prec=INT4)              host, numpy in/out
    quantize_act(X, smooth, down, prec=INT4, ...)              device, torch tensors
    w4a4_linear(xq, xscale, h, wq, wscale, up, bias, ...)      device, torch tensors
    w4a4_linear_requant(...)                                    device, torch tensors
    w4a4_linear_qkv_norm_rope(...)                              device, torch tensors
    awq_pack_weights(W)                                         host, numpy in/out
    awq_w4a16_linear(X, wq, wscale, bias, ...)                  device, torch tensors

Device tensors: X bf16 [M][K], smooth fp32 [K], down bf16 [32][K],
up bf16 [N][32], bias bf16 [N] or None, xq uint8 [M][K/2],
xscale fp32 [M][K/64] (INT4) or uint8 [M][K/32] (MXFP4), h fp32 [M][32],
Y bf16 [M][N].  Calls are enqueued on the current torch stream (or `stream`).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libsvdq.so")

INT4 = 0
MXFP4 = 1
EPI_NONE = 0
EPI_GELU_TANH = 1
RANK = 32

STATUS = {
    0: "SVDQ_OK", -1: "SVDQ_ERR_INVALID_ARG", -2: "SVDQ_ERR_SHAPE", -3: "SVDQ_ERR_MISALIGNED",
    -4: "SVDQ_ERR_UNSUPPORTED", -5: "SVDQ_ERR_UNSUPPORTED_DEVICE", -6: "SVDQ_ERR_NONFINITE",
    -7: "SVDQ_ERR_HIP",
}
EXPORTS = ("svdq_status_string", "svdq_version", "svdq_check_device", "svdq_pack_weights",
           "svdq_pack_residual", "svdq_quantize_act", "svdq_w4a4_linear", "svdq_requant_workspace_bytes",
           "svdq_w4a4_linear_requant", "svdq_w4a4_linear_qkv_norm_rope", "svdq_awq_pack_weights",
           "svdq_awq_w4a16_linear", "svdq_w4a4_linear_splitk_workspace_bytes", "svdq_w4a4_linear_splitk")


class SvdqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


_lib = None


def lib():
    """Load libsvdq.so (building it in-tree only when it is absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from .build import build
            build()
        L = ctypes.CDLL(LIB_PATH)
        P, I = ctypes.c_void_p, ctypes.c_int
        L.svdq_status_string.restype = ctypes.c_char_p
        L.svdq_status_string.argtypes = [I]
        L.svdq_version.restype = I
        L.svdq_version.argtypes = []
        L.svdq_check_device.restype = I
        L.svdq_check_device.argtypes = []
        L.svdq_pack_weights.restype = I
        L.svdq_pack_weights.argtypes = [P, P, I, I, I, I, P, P, P, P, P]
        L.svdq_pack_residual.restype = I
        L.svdq_pack_residual.argtypes = [P, P, P, P, I, I, I, I, P, P]
        L.svdq_quantize_act.restype = I
        L.svdq_quantize_act.argtypes = [P, I, I, P, P, I, I, P, P, P, P]
        L.svdq_w4a4_linear.restype = I
        L.svdq_w4a4_linear.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P, P]
        L.svdq_w4a4_linear_splitk_workspace_bytes.restype = ctypes.c_size_t
        L.svdq_w4a4_linear_splitk_workspace_bytes.argtypes = [I, I, I, I]
        L.svdq_w4a4_linear_splitk.restype = I
        L.svdq_w4a4_linear_splitk.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P, P, ctypes.c_size_t, P]
        L.svdq_requant_workspace_bytes.restype = ctypes.c_size_t
        L.svdq_requant_workspace_bytes.argtypes = [I, I, I, I]
        L.svdq_w4a4_linear_requant.restype = I
        L.svdq_w4a4_linear_requant.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, P, P,
                                               ctypes.c_size_t, P]
        L.svdq_w4a4_linear_qkv_norm_rope.restype = I
        L.svdq_w4a4_linear_qkv_norm_rope.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P, P, ctypes.c_float, P, P,
                                                     P, P]
        L.svdq_awq_pack_weights.restype = I
        L.svdq_awq_pack_weights.argtypes = [P, I, I, P, P]
        L.svdq_awq_w4a16_linear.restype = I
        L.svdq_awq_w4a16_linear.argtypes = [P, P, P, P, I, I, I, P, P]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().svdq_status_string(int(status)).decode()


def version() -> int:
    return lib().svdq_version()


def _check(st: int, where: str):
    if st != 0:
        raise SvdqError(st, where)


def check_device() -> None:
    _check(lib().svdq_check_device(), "svdq_check_device")


def group_of(prec: int) -> int:
    return 64 if prec == INT4 else 32


# ------------------------------------------------------------------ host calls

def _np(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, ctypes.c_void_p(a.ctypes.data)


def pack_weights(W: np.ndarray, act_absmax: np.ndarray, rank: int = RANK, prec: int = INT4) -> dict:
    """Smoothing, top-r SVD and residual packing of one layer (host)."""
    W, pW = _np(W, np.uint16)
    a, pa = _np(act_absmax, np.float32)
    N, K = W.shape
    g = group_of(prec)
    smooth = np.zeros(K, np.float32)
    down = np.zeros((rank, K), np.uint16)
    up = np.zeros((N, rank), np.uint16)
    wq = np.zeros((N, K // 2), np.uint8)
    wscale = np.zeros((N, max(K // g, 0)), np.float32 if prec == INT4 else np.uint8)
    st = lib().svdq_pack_weights(pW, pa, N, K, rank, prec, smooth.ctypes.data, down.ctypes.data,
                                 up.ctypes.data, wq.ctypes.data, wscale.ctypes.data)
    _check(st, "svdq_pack_weights")
    return dict(smooth=smooth, down=down, up=up, wq=wq, wscale=wscale)


def pack_residual(W, smooth, down, up, prec: int = INT4):
    W, pW = _np(W, np.uint16)
    s, ps = _np(smooth, np.float32)
    d, pd = _np(down, np.uint16)
    u, pu = _np(up, np.uint16)
    N, K = W.shape
    g = group_of(prec)
    wq = np.zeros((N, K // 2), np.uint8)
    wscale = np.zeros((N, max(K // g, 0)), np.float32 if prec == INT4 else np.uint8)
    st = lib().svdq_pack_residual(pW, ps, pd, pu, N, K, d.shape[0], prec, wq.ctypes.data,
                                  wscale.ctypes.data)
    _check(st, "svdq_pack_residual")
    return wq, wscale


# ---------------------------------------------------------------- device calls

def _torch():
    import torch
    return torch


def _dev(t, dtypes, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def quantize_act(X, smooth, down, prec: int = INT4, xq=None, xscale=None, h=None, stream=None):
    """Fused smoothing + 4-bit quantization + down projection (one kernel)."""
    torch = _torch()
    M, K = X.shape
    r = down.shape[0]
    g = group_of(prec)
    dev = X.device
    if xq is None:
        xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    if xscale is None:
        xscale = torch.empty((M, K // g), dtype=torch.float32 if prec == INT4 else torch.uint8, device=dev)
    if h is None:
        h = torch.empty((M, r), dtype=torch.float32, device=dev)
    st = lib().svdq_quantize_act(
        _dev(X, (torch.bfloat16, torch.int16), "X"), M, K,
        _dev(smooth, (torch.float32,), "smooth"), _dev(down, (torch.bfloat16, torch.int16), "down"), r,
        prec, _dev(xq, (torch.uint8,), "xq"), _dev(xscale, (torch.float32, torch.uint8), "xscale"),
        _dev(h, (torch.float32,), "h"), _stream(stream))
    _check(st, "svdq_quantize_act")
    return xq, xscale, h


def w4a4_linear(xq, xscale, h, wq, wscale, up, bias, prec: int = INT4, epi: int = EPI_NONE,
                Y=None, stream=None):
    """4-bit product + low-rank up projection + bias (+ GELU) -> bf16 (one kernel)."""
    torch = _torch()
    M = xq.shape[0]
    K = xq.shape[1] * 2
    N = wq.shape[0]
    r = up.shape[1]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    pbias = None if bias is None else _dev(bias, (torch.bfloat16, torch.int16), "bias")
    st = lib().svdq_w4a4_linear(
        _dev(xq, (torch.uint8,), "xq"), _dev(xscale, (torch.float32, torch.uint8), "xscale"),
        _dev(h, (torch.float32,), "h"), _dev(wq, (torch.uint8,), "wq"),
        _dev(wscale, (torch.float32, torch.uint8), "wscale"), _dev(up, (torch.bfloat16, torch.int16), "up"),
        pbias, M, N, K, r, prec, epi, _dev(Y, (torch.bfloat16, torch.int16), "Y"), _stream(stream))
    _check(st, "svdq_w4a4_linear")
    return Y


def linear_splitk_workspace_bytes(M: int, N: int, K: int, prec: int = MXFP4) -> int:
    """Device scratch bytes that w4a4_linear_splitk needs on the current
    device (0 when the shape is not split)."""
    return int(lib().svdq_w4a4_linear_splitk_workspace_bytes(M, N, K, prec))


def w4a4_linear_splitk(xq, xscale, h, wq, wscale, up, bias, prec: int = MXFP4, epi: int = EPI_NONE,
                       Y=None, work=None, stream=None):
    """w4a4_linear with K split across work items when the tiles cannot fill
    the chip (fp32 partial sums in `work`, summed in slice order).  When
    `work` is None this binding allocates it with torch; pass a preallocated
    tensor of linear_splitk_workspace_bytes(...) bytes in a serving loop."""
    torch = _torch()
    M = xq.shape[0]
    K = xq.shape[1] * 2
    N = wq.shape[0]
    r = up.shape[1]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    need = linear_splitk_workspace_bytes(M, N, K, prec)
    if work is None and need > 0:
        work = torch.empty(need // 4, dtype=torch.float32, device=xq.device)
    pwork = None if work is None else _dev(work, (torch.float32, torch.uint8), "work")
    nbytes = 0 if work is None else work.numel() * work.element_size()
    pbias = None if bias is None else _dev(bias, (torch.bfloat16, torch.int16), "bias")
    st = lib().svdq_w4a4_linear_splitk(
        _dev(xq, (torch.uint8,), "xq"), _dev(xscale, (torch.float32, torch.uint8), "xscale"),
        _dev(h, (torch.float32,), "h"), _dev(wq, (torch.uint8,), "wq"),
        _dev(wscale, (torch.float32, torch.uint8), "wscale"), _dev(up, (torch.bfloat16, torch.int16), "up"),
        pbias, M, N, K, r, prec, epi, _dev(Y, (torch.bfloat16, torch.int16), "Y"), pwork, nbytes,
        _stream(stream))
    _check(st, "svdq_w4a4_linear_splitk")
    return Y


def requant_workspace_bytes(M: int, N: int, rank: int = RANK, prec: int = INT4) -> int:
    """Device scratch bytes that w4a4_linear_requant needs."""
    return int(lib().svdq_requant_workspace_bytes(M, N, rank, prec))


def w4a4_linear_requant(xq, xscale, h, wq, wscale, up, bias, smooth2, down2, prec: int = INT4,
                        epi: int = EPI_NONE, out=None, work=None, stream=None):
    """w4a4_linear whose epilogue writes the next layer's activation codes,
    scales and h (smooth2, down2 of that layer) instead of Y.  Returns
    (xq2, xscale2, h2)."""
    torch = _torch()
    M = xq.shape[0]
    K = xq.shape[1] * 2
    N = wq.shape[0]
    r = up.shape[1]
    dev = xq.device
    if out is None:
        scales = (torch.empty((M, max(N // 64, 1)), dtype=torch.float32, device=dev) if prec == INT4
                  else torch.empty((M, max(N // 32, 1)), dtype=torch.uint8, device=dev))
        out = (torch.empty((M, N // 2), dtype=torch.uint8, device=dev), scales,
               torch.empty((M, r), dtype=torch.float32, device=dev))
    xq2, xs2, h2 = out
    nbytes = requant_workspace_bytes(M, N, r, prec)
    if work is None:
        work = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=dev)
    pbias = None if bias is None else _dev(bias, (torch.bfloat16, torch.int16), "bias")
    st = lib().svdq_w4a4_linear_requant(
        _dev(xq, (torch.uint8,), "xq"), _dev(xscale, (torch.float32, torch.uint8), "xscale"),
        _dev(h, (torch.float32,), "h"), _dev(wq, (torch.uint8,), "wq"),
        _dev(wscale, (torch.float32, torch.uint8), "wscale"), _dev(up, (torch.bfloat16, torch.int16), "up"),
        pbias, M, N, K, r, prec, epi, _dev(smooth2, (torch.float32,), "smooth2"),
        _dev(down2, (torch.bfloat16, torch.int16), "down2"), _dev(xq2, (torch.uint8,), "xq2"),
        _dev(xs2, (torch.float32, torch.uint8), "xscale2"), _dev(h2, (torch.float32,), "h2"),
        _dev(work, (torch.uint8, torch.float32), "work"), work.numel() * work.element_size(), _stream(stream))
    _check(st, "svdq_w4a4_linear_requant")
    return xq2, xs2, h2


def w4a4_linear_qkv_norm_rope(xq, xscale, h, wq, wscale, up, bias, norm_q, norm_k, eps: float, rope_cos,
                              rope_sin, prec: int = INT4, Y=None, stream=None):
    """w4a4_linear of a fused QKV projection (N = 3 H 128) with the Q/K
    RMS-norm and rotary embedding applied in its epilogue (one kernel)."""
    torch = _torch()
    M = xq.shape[0]
    K = xq.shape[1] * 2
    N = wq.shape[0]
    r = up.shape[1]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    pbias = None if bias is None else _dev(bias, (torch.bfloat16, torch.int16), "bias")
    st = lib().svdq_w4a4_linear_qkv_norm_rope(
        _dev(xq, (torch.uint8,), "xq"), _dev(xscale, (torch.float32, torch.uint8), "xscale"),
        _dev(h, (torch.float32,), "h"), _dev(wq, (torch.uint8,), "wq"),
        _dev(wscale, (torch.float32, torch.uint8), "wscale"), _dev(up, (torch.bfloat16, torch.int16), "up"),
        pbias, M, N, K, r, prec, _dev(norm_q, (torch.bfloat16, torch.int16), "norm_q"),
        _dev(norm_k, (torch.bfloat16, torch.int16), "norm_k"), float(eps),
        _dev(rope_cos, (torch.float32,), "rope_cos"), _dev(rope_sin, (torch.float32,), "rope_sin"),
        _dev(Y, (torch.bfloat16, torch.int16), "Y"), _stream(stream))
    _check(st, "svdq_w4a4_linear_qkv_norm_rope")
    return Y


def awq_pack_weights(W: np.ndarray):
    """Weight-only AWQ W4A16 packing (host): bf16 bits [N][K] ->
    (wq uint8 [N][K/2], wscale fp32 [N][K/64])."""
    W, pW = _np(W, np.uint16)
    N, K = W.shape
    wq = np.zeros((N, K // 2), np.uint8)
    wscale = np.zeros((N, max(K // 64, 0)), np.float32)
    st = lib().svdq_awq_pack_weights(pW, N, K, wq.ctypes.data, wscale.ctypes.data)
    _check(st, "svdq_awq_pack_weights")
    return wq, wscale


def awq_w4a16_linear(X, wq, wscale, bias=None, Y=None, stream=None):
    """Weight-only 4-bit linear with bf16 activations -> bf16 (one kernel)."""
    torch = _torch()
    M, K = X.shape
    N = wq.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    pbias = None if bias is None else _dev(bias, (torch.bfloat16, torch.int16), "bias")
    st = lib().svdq_awq_w4a16_linear(
        _dev(X, (torch.bfloat16, torch.int16), "X"), _dev(wq, (torch.uint8,), "wq"),
        _dev(wscale, (torch.float32,), "wscale"), pbias, M, N, K,
        _dev(Y, (torch.bfloat16, torch.int16), "Y"), _stream(stream))
    _check(st, "svdq_awq_w4a16_linear")
    return Y


def to_device(packed: dict, device="cuda") -> dict:
    """Copy packed numpy arrays to device tensors with the dtypes the calls expect."""
    torch = _torch()
    out = {}
    for k, v in packed.items():
        t = torch.from_numpy(np.ascontiguousarray(v))
        if v.dtype == np.uint16:
            t = t.view(torch.int16).view(torch.bfloat16)
        out[k] = t.to(device)
    return out


def bf16_tensor(bits: np.ndarray, device="cuda"):
    """uint16 bf16 bits (numpy) -> torch bfloat16 tensor on `device`."""
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(
        torch.bfloat16).to(device)


def bf16_bits(t) -> np.ndarray:
    """torch bfloat16 tensor -> uint16 bits (numpy, host)."""
    torch = _torch()
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
