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
# SVDQ_LIBRARY names another build of the same library (the sanitizer
# tests load an address/undefined-behaviour-sanitized build this way)
LIB_PATH = os.environ.get("SVDQ_LIBRARY") or os.path.join(PKG_DIR, "libsvdq.so")

INT4 = 0
MXFP4 = 1
EPI_NONE = 0
EPI_GELU_TANH = 1
RANK = 32

STATUS = {
    0: "SVDQ_OK", -1: "SVDQ_ERR_INVALID_ARG", -2: "SVDQ_ERR_SHAPE", -3: "SVDQ_ERR_MISALIGNED",
    -4: "SVDQ_ERR_UNSUPPORTED", -5: "SVDQ_ERR_UNSUPPORTED_DEVICE", -6: "SVDQ_ERR_NONFINITE",
    -7: "SVDQ_ERR_HIP", -8: "SVDQ_ERR_SCRATCH",
}
EXPORTS = ("svdq_status_string", "svdq_version", "svdq_check_device", "svdq_pack_weights",
           "svdq_pack_residual", "svdq_quantize_act", "svdq_w4a4_linear", "svdq_requant_workspace_bytes",
           "svdq_w4a4_linear_requant", "svdq_w4a4_linear_qkv_norm_rope", "svdq_awq_pack_weights",
           "svdq_awq_w4a16_linear", "svdq_w4a4_linear_splitk_workspace_bytes", "svdq_w4a4_linear_splitk",
           "svdq_nf4_codebook", "svdq_nf4_pack_weights", "svdq_nf4_dequantize", "svdq_nf4_w4a16_linear",
           "svdq_w4a4_linear_splitk_noalloc")


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
        L.svdq_w4a4_linear_splitk_noalloc.restype = I
        L.svdq_w4a4_linear_splitk_noalloc.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P, P]
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
        L.svdq_nf4_codebook.restype = I
        L.svdq_nf4_codebook.argtypes = [P]
        L.svdq_nf4_pack_weights.restype = I
        L.svdq_nf4_pack_weights.argtypes = [P, I, I, P, P, P]
        L.svdq_nf4_dequantize.restype = I
        L.svdq_nf4_dequantize.argtypes = [P, P, P, I, I, P, P]
        L.svdq_nf4_w4a16_linear.restype = I
        L.svdq_nf4_w4a16_linear.argtypes = [P, P, P, P, P, I, I, I, P, P]
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
    prec = _prec(prec)
    W, pW = _np(W, np.uint16)
    a, pa = _np(act_absmax, np.float32)
    if W.ndim != 2:
        raise ValueError(f"W must have 2 dimensions, got shape {W.shape}")
    N, K = W.shape
    if a.shape != (K,):
        raise ValueError(f"act_absmax has shape {a.shape}, expected {(K,)}")
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
    prec = _prec(prec)
    if W.ndim != 2 or d.ndim != 2:
        raise ValueError("W and down must have 2 dimensions")
    N, K = W.shape
    r = d.shape[0]
    for arr, want, name in ((s, (K,), "smooth"), (d, (r, K), "down"), (u, (N, r), "up")):
        if arr.shape != want:
            raise ValueError(f"{name} has shape {arr.shape}, expected {want}")
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


def _chk(t, dtypes, name, shape=None):
    """Type, dtype, shape (when given) and contiguity of a tensor argument."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptrs(*specs):
    """Pointers of device tensors given as (tensor, dtypes, name[, shape])
    (None for an absent optional tensor).  Every tensor's type, dtype, shape
    and contiguity are checked before any device check, so a wrong shape is
    reported the same way with or without a GPU."""
    for sp in specs:
        if sp is not None:
            _chk(*sp)
    out = []
    for sp in specs:
        if sp is None:
            out.append(None)
            continue
        t, name = sp[0], sp[2]
        if t.device.type != "cuda":
            raise TypeError(f"{name} must be a device tensor")
        out.append(ctypes.c_void_p(t.data_ptr()))
    return out


def _prec(prec: int) -> int:
    if prec not in (INT4, MXFP4):
        raise ValueError(f"prec must be INT4 ({INT4}) or MXFP4 ({MXFP4}), got {prec}")
    return prec


def _scale_dtypes(prec: int):
    """The one scale dtype each precision takes: fp32 (INT4), E8M0 bytes (MXFP4)."""
    torch = _torch()
    return (torch.float32,) if prec == INT4 else (torch.uint8,)


def _ndim(t, n, name):
    if getattr(t, "ndim", None) != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(getattr(t, 'shape', ()))}")


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def quantize_act(X, smooth, down, prec: int = INT4, xq=None, xscale=None, h=None, stream=None):
    """Fused smoothing + 4-bit quantization + down projection (one kernel)."""
    torch = _torch()
    prec = _prec(prec)
    _ndim(X, 2, "X")
    _ndim(down, 2, "down")
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
    bf = (torch.bfloat16, torch.int16)
    pX, ps, pd, pq, pxs, ph = _ptrs(
        (X, bf, "X"), (smooth, (torch.float32,), "smooth", (K,)), (down, bf, "down", (r, K)),
        (xq, (torch.uint8,), "xq", (M, K // 2)), (xscale, _scale_dtypes(prec), "xscale", (M, K // g)),
        (h, (torch.float32,), "h", (M, r)))
    st = lib().svdq_quantize_act(pX, M, K, ps, pd, r, prec, pq, pxs, ph, _stream(stream))
    _check(st, "svdq_quantize_act")
    return xq, xscale, h


def _linear_specs(xq, xscale, h, wq, wscale, up, bias, prec):
    """Shapes of the product's operands: M, K from xq, N from wq, r from up;
    every other operand must agree with them."""
    torch = _torch()
    prec = _prec(prec)
    for t, name in ((xq, "xq"), (xscale, "xscale"), (h, "h"), (wq, "wq"), (wscale, "wscale"), (up, "up")):
        _ndim(t, 2, name)
    M, K = xq.shape[0], xq.shape[1] * 2
    N, r = wq.shape[0], up.shape[1]
    g = group_of(prec)
    bf = (torch.bfloat16, torch.int16)
    specs = [(xq, (torch.uint8,), "xq"), (xscale, _scale_dtypes(prec), "xscale", (M, K // g)),
             (h, (torch.float32,), "h", (M, r)), (wq, (torch.uint8,), "wq", (N, K // 2)),
             (wscale, _scale_dtypes(prec), "wscale", (N, K // g)), (up, bf, "up", (N, r)),
             None if bias is None else (bias, bf, "bias", (N,))]
    return M, N, K, r, specs


def w4a4_linear(xq, xscale, h, wq, wscale, up, bias, prec: int = INT4, epi: int = EPI_NONE,
                Y=None, stream=None):
    """4-bit product + low-rank up projection + bias (+ GELU) -> bf16 (one kernel)."""
    torch = _torch()
    M, N, K, r, specs = _linear_specs(xq, xscale, h, wq, wscale, up, bias, prec)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    *ptrs, pY = _ptrs(*specs, (Y, (torch.bfloat16, torch.int16), "Y", (M, N)))
    st = lib().svdq_w4a4_linear(*ptrs, M, N, K, r, prec, epi, pY, _stream(stream))
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
    M, N, K, r, specs = _linear_specs(xq, xscale, h, wq, wscale, up, bias, prec)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    need = linear_splitk_workspace_bytes(M, N, K, prec)
    if work is None and need > 0:
        work = torch.empty(need // 4, dtype=torch.float32, device=xq.device)
    wspec = None if work is None else (work, (torch.float32, torch.uint8), "work")
    *ptrs, pY, pwork = _ptrs(*specs, (Y, (torch.bfloat16, torch.int16), "Y", (M, N)), wspec)
    nbytes = 0 if work is None else work.numel() * work.element_size()
    st = lib().svdq_w4a4_linear_splitk(*ptrs, M, N, K, r, prec, epi, pY, pwork, nbytes, _stream(stream))
    _check(st, "svdq_w4a4_linear_splitk")
    return Y


NOALLOC_SCRATCH_BYTES = 64 << 20


def w4a4_linear_splitk_noalloc(xq, xscale, h, wq, wscale, up, bias, prec: int = MXFP4, epi: int = EPI_NONE,
                               Y=None, stream=None):
    """w4a4_linear_splitk without a workspace: the slice sums go to the
    library's static per-GPU scratch buffer (NOALLOC_SCRATCH_BYTES), so the
    library allocates nothing.  Calls that overlap in time on one GPU race.
    With Y given, this binding allocates nothing either."""
    torch = _torch()
    M, N, K, r, specs = _linear_specs(xq, xscale, h, wq, wscale, up, bias, prec)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    *ptrs, pY = _ptrs(*specs, (Y, (torch.bfloat16, torch.int16), "Y", (M, N)))
    st = lib().svdq_w4a4_linear_splitk_noalloc(*ptrs, M, N, K, r, prec, epi, pY, _stream(stream))
    _check(st, "svdq_w4a4_linear_splitk_noalloc")
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
    M, N, K, r, specs = _linear_specs(xq, xscale, h, wq, wscale, up, bias, prec)
    g = group_of(prec)
    dev = xq.device
    if out is None:
        scales = (torch.empty((M, N // 64), dtype=torch.float32, device=dev) if prec == INT4
                  else torch.empty((M, N // 32), dtype=torch.uint8, device=dev))
        out = (torch.empty((M, N // 2), dtype=torch.uint8, device=dev), scales,
               torch.empty((M, r), dtype=torch.float32, device=dev))
    xq2, xs2, h2 = out
    nbytes = requant_workspace_bytes(M, N, r, prec)
    if work is None:
        work = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=dev)
    bf = (torch.bfloat16, torch.int16)
    ptrs = _ptrs(*specs, (smooth2, (torch.float32,), "smooth2", (N,)), (down2, bf, "down2", (r, N)),
                 (xq2, (torch.uint8,), "xq2", (M, N // 2)), (xs2, _scale_dtypes(prec), "xscale2", (M, N // g)),
                 (h2, (torch.float32,), "h2", (M, r)), (work, (torch.uint8, torch.float32), "work"))
    st = lib().svdq_w4a4_linear_requant(*ptrs[:7], M, N, K, r, prec, epi, *ptrs[7:],
                                        work.numel() * work.element_size(), _stream(stream))
    _check(st, "svdq_w4a4_linear_requant")
    return xq2, xs2, h2


def w4a4_linear_qkv_norm_rope(xq, xscale, h, wq, wscale, up, bias, norm_q, norm_k, eps: float, rope_cos,
                              rope_sin, prec: int = INT4, Y=None, stream=None):
    """w4a4_linear of a fused QKV projection (N = 3 H 128) with the Q/K
    RMS-norm and rotary embedding applied in its epilogue (one kernel)."""
    torch = _torch()
    M, N, K, r, specs = _linear_specs(xq, xscale, h, wq, wscale, up, bias, prec)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    bf = (torch.bfloat16, torch.int16)
    ptrs = _ptrs(*specs, (norm_q, bf, "norm_q", (128,)), (norm_k, bf, "norm_k", (128,)),
                 (rope_cos, (torch.float32,), "rope_cos", (M, 64)), (rope_sin, (torch.float32,), "rope_sin", (M, 64)),
                 (Y, bf, "Y", (M, N)))
    st = lib().svdq_w4a4_linear_qkv_norm_rope(*ptrs[:7], M, N, K, r, prec, ptrs[7], ptrs[8], float(eps),
                                              *ptrs[9:], _stream(stream))
    _check(st, "svdq_w4a4_linear_qkv_norm_rope")
    return Y


def awq_pack_weights(W: np.ndarray):
    """Weight-only AWQ W4A16 packing (host): bf16 bits [N][K] ->
    (wq uint8 [N][K/2], wscale fp32 [N][K/64])."""
    W, pW = _np(W, np.uint16)
    if W.ndim != 2:
        raise ValueError(f"W must have 2 dimensions, got shape {W.shape}")
    N, K = W.shape
    wq = np.zeros((N, K // 2), np.uint8)
    wscale = np.zeros((N, max(K // 64, 0)), np.float32)
    st = lib().svdq_awq_pack_weights(pW, N, K, wq.ctypes.data, wscale.ctypes.data)
    _check(st, "svdq_awq_pack_weights")
    return wq, wscale


def awq_w4a16_linear(X, wq, wscale, bias=None, Y=None, stream=None):
    """Weight-only 4-bit linear with bf16 activations -> bf16 (one kernel)."""
    torch = _torch()
    for t, name in ((X, "X"), (wq, "wq"), (wscale, "wscale")):
        _ndim(t, 2, name)
    M, K = X.shape
    N = wq.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    bf = (torch.bfloat16, torch.int16)
    pX, pq, ps, pb, pY = _ptrs((X, bf, "X"), (wq, (torch.uint8,), "wq", (N, K // 2)),
                               (wscale, (torch.float32,), "wscale", (N, K // 64)),
                               None if bias is None else (bias, bf, "bias", (N,)), (Y, bf, "Y", (M, N)))
    st = lib().svdq_awq_w4a16_linear(pX, pq, ps, pb, M, N, K, pY, _stream(stream))
    _check(st, "svdq_awq_w4a16_linear")
    return Y


def nf4_codebook() -> np.ndarray:
    """The 16 NF4 levels (fp32, ascending)."""
    c = np.zeros(16, np.float32)
    _check(lib().svdq_nf4_codebook(c.ctypes.data), "svdq_nf4_codebook")
    return c


def nf4_pack_weights(W: np.ndarray):
    """NF4 weight-only packing (host): bf16 bits [N][K] -> (wq uint8 [N][K/2],
    qabs uint8 [N*K/64], chunk_scale fp32 [ceil(N*K/64/256)])."""
    W, pW = _np(W, np.uint16)
    if W.ndim != 2:
        raise ValueError(f"W must have 2 dimensions, got shape {W.shape}")
    N, K = W.shape
    nb = N * (K // 64)
    wq = np.zeros((N, K // 2), np.uint8)
    qabs = np.zeros(max(nb, 1), np.uint8)[:nb]
    chunk = np.zeros(max((nb + 255) // 256, 1), np.float32)[:(nb + 255) // 256]
    st = lib().svdq_nf4_pack_weights(pW, N, K, wq.ctypes.data, qabs.ctypes.data, chunk.ctypes.data)
    _check(st, "svdq_nf4_pack_weights")
    return wq, qabs, chunk


def _nf4_specs(wq, qabs, chunk):
    torch = _torch()
    _ndim(wq, 2, "wq")
    N, K = wq.shape[0], wq.shape[1] * 2
    nb = N * (K // 64)
    return N, K, [(wq, (torch.uint8,), "wq"), (qabs, (torch.uint8,), "qabs", (nb,)),
                  (chunk, (torch.float32,), "chunk_scale", ((nb + 255) // 256,))]


def nf4_dequantize(wq, qabs, chunk, Wd=None, stream=None):
    """The dequantized NF4 weights as a bf16 tensor [N][K] (one kernel)."""
    torch = _torch()
    N, K, specs = _nf4_specs(wq, qabs, chunk)
    if Wd is None:
        Wd = torch.empty((N, K), dtype=torch.bfloat16, device=wq.device)
    pq, pa, pc, pW = _ptrs(*specs, (Wd, (torch.bfloat16, torch.int16), "Wd", (N, K)))
    _check(lib().svdq_nf4_dequantize(pq, pa, pc, N, K, pW, _stream(stream)), "svdq_nf4_dequantize")
    return Wd


def nf4_w4a16_linear(X, wq, qabs, chunk, bias=None, Y=None, stream=None):
    """Weight-only NF4 linear with bf16 activations -> bf16 (one kernel)."""
    torch = _torch()
    N, K, specs = _nf4_specs(wq, qabs, chunk)
    _ndim(X, 2, "X")
    M = X.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    bf = (torch.bfloat16, torch.int16)
    pX, pq, pa, pc, pb, pY = _ptrs((X, bf, "X", (M, K)), *specs, None if bias is None else (bias, bf, "bias", (N,)),
                                   (Y, bf, "Y", (M, N)))
    st = lib().svdq_nf4_w4a16_linear(pX, pq, pa, pc, pb, M, N, K, pY, _stream(stream))
    _check(st, "svdq_nf4_w4a16_linear")
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
