"""TEST INFRASTRUCTURE ONLY: Python face of the fp64 CPU oracle.

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
module.  It wraps the plain C routines of svdq_oracle.c (ctypes) and adds the
one step that calls a library primitive: the top-r SVD of the smoothed
weight, done with numpy.linalg.svd (LAPACK) in float64.

Method source: "Bringing Nunchaku 4-bit Diffusion Inference to Diffusers"
(Hugging Face blog), section "Background: SVDQuant and Nunchaku" (smoothing
moves activation outliers into the weights, a small 16-bit low-rank branch
takes the hardest part of each weight matrix, the residual goes to 4 bits;
the low-rank down projection is fused with the quantization and the up
projection with the 4-bit product), and section "Native loading in
Diffusers" (rank 32, bfloat16 compute dtype, 4-bit weight groups).
The formulas, with the readings that fix what the prose leaves open, are at
the top of svdq_oracle.c.  The same file holds the weight-only AWQ W4A16
layer of those pages (section "Native loading in Diffusers": awq_w4a16,
int4, group size 64, for the modulation layers), with its readings.

Parity unpinned: the exact bits of the low-rank factors (several results are
correct: signs of singular-vector pairs, rotations inside repeated singular
values, last-bit differences between SVD algorithms); they are checked by
Eckart-Young instead.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# SVDQ_ORACLE_LIBRARY names another build of the oracle (the sanitizer tests
# load a sanitized build this way)
_LIB_PATH = os.environ.get("SVDQ_ORACLE_LIBRARY") or os.path.join(HERE, "liboracle.so")

INT4 = 0
MXFP4 = 1

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from oracle.build import build as _build
            _build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.oracle_quant_group_int4.restype = ctypes.c_float
        L.oracle_quant_group_int4.argtypes = [P, I, P, P]
        L.oracle_int4_value.restype = I
        L.oracle_int4_value.argtypes = [ctypes.c_uint8]
        L.oracle_quant_block_mxfp4.restype = ctypes.c_uint8
        L.oracle_quant_block_mxfp4.argtypes = [P, I, P]
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        L.oracle_e8m0_value.restype = ctypes.c_double
        L.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        L.oracle_pack_nibbles.argtypes = [P, I, P]
        L.oracle_smooth.argtypes = [P, P, I, I, P]
        L.oracle_residual.argtypes = [P, P, P, P, I, I, I, I, P, P, P]
        L.oracle_quant_act.argtypes = [P, I, I, P, P, I, I, P, P, P]
        L.oracle_linear.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P, I, P, P, P]
        L.oracle_gelu_tanh.restype = ctypes.c_double
        L.oracle_gelu_tanh.argtypes = [ctypes.c_double]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_qkv_norm_rope.argtypes = [P, I, I, P, P, ctypes.c_double, P, P, P]
        L.oracle_awq_code.restype = I
        L.oracle_awq_code.argtypes = [P, I]
        L.oracle_awq_pack.argtypes = [P, I, I, P, P]
        L.oracle_awq_linear.argtypes = [P, P, P, P, I, I, I, P]
        L.oracle_nf4_codebook.argtypes = [P]
        L.oracle_nf4_code.restype = I
        L.oracle_nf4_code.argtypes = [ctypes.c_float, P]
        L.oracle_nf4_pack.argtypes = [P, I, I, P, P, P]
        L.oracle_nf4_dequant.argtypes = [P, P, P, I, I, P]
        L.oracle_nf4_linear.argtypes = [P, P, P, P, P, I, I, I, P, I, P]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def group_of(prec: int) -> int:
    return 64 if prec == INT4 else 32


# ------------------------------------------------------------ group quantizers

def quant_group_int4(v, codes: bool = False):
    """(q, scale) of one INT4 group, or (q, scale, codes) with the
    sign-magnitude 4-bit codes (sign of v kept for zero)."""
    v = _c(v, np.float32)
    q = np.zeros(v.size, np.int8)
    c = np.zeros(v.size, np.uint8)
    sc = lib().oracle_quant_group_int4(_p(v), v.size, _p(q), _p(c))
    return (q, np.float32(sc), c) if codes else (q, np.float32(sc))


def int4_value(code: int) -> int:
    return lib().oracle_int4_value(code)


def quant_block_mxfp4(v) -> tuple[np.ndarray, int]:
    v = _c(v, np.float32)
    c = np.zeros(v.size, np.uint8)
    e = lib().oracle_quant_block_mxfp4(_p(v), v.size, _p(c))
    return c, int(e)


def pack_nibbles(codes) -> np.ndarray:
    """4-bit codes (one per byte) -> packed bytes, element 2i in the low nibble."""
    c = _c(codes, np.uint8)
    out = np.zeros(c.size // 2, np.uint8)
    lib().oracle_pack_nibbles(_p(c), c.size, _p(out))
    return out


def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(code)


def e8m0_value(e: int) -> float:
    return lib().oracle_e8m0_value(e)


def gelu_tanh(y: float) -> float:
    return lib().oracle_gelu_tanh(y)


def num_threads() -> int:
    return lib().oracle_num_threads()


# ------------------------------------------------------------------ bf16 (own)

def _bf16_bits_from_f64(a: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 bits: nearest-even on the float64 value, done as
    float64 -> float32 (RNE) -> bf16 (RNE on the upper 16 bits)."""
    f = np.asarray(a, np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.int64)
    keep = u >> 16
    rem = u & 0xFFFF
    up = (rem > 0x8000) | ((rem == 0x8000) & ((keep & 1) == 1))
    return (keep + up.astype(np.int64)).astype(np.uint16)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ pack steps

def smooth(W: np.ndarray, act_absmax: np.ndarray) -> np.ndarray:
    W = _c(W, np.uint16)
    a = _c(act_absmax, np.float32)
    N, K = W.shape
    s = np.zeros(K, np.float32)
    lib().oracle_smooth(_p(W), _p(a), N, K, _p(s))
    return s


def lowrank(W: np.ndarray, s: np.ndarray, r: int):
    """Top-r SVD of What_kn = W_nk / s_k (float64, numpy/LAPACK).

    Returns (down_bits [r][K], up_bits [N][r], sigma (all singular values),
    L1 = U_r S_r [K][r] float64, L2 = V_r^T [r][N] float64).  Components beyond
    the matrix rank are zero.
    """
    Wd = bf16_to_f64(W)                              # [N][K]
    What = (Wd / np.asarray(s, np.float64)[None, :]).T  # [K][N]
    U, S, Vt = np.linalg.svd(What, full_matrices=False)
    K, N = What.shape
    rr = min(r, S.size)
    L1 = np.zeros((K, r))
    L2 = np.zeros((r, N))
    L1[:, :rr] = U[:, :rr] * S[None, :rr]
    L2[:rr, :] = Vt[:rr, :]
    # sign convention (reproducibility only): largest-|.| entry of v_j positive
    for j in range(rr):
        i = int(np.argmax(np.abs(L2[j])))
        if L2[j, i] < 0:
            L2[j] = -L2[j]
            L1[:, j] = -L1[:, j]
    down = _bf16_bits_from_f64((np.asarray(s, np.float64)[:, None] * L1).T)  # [r][K]
    up = _bf16_bits_from_f64(L2.T)                                         # [N][r]
    return down, up, S, L1, L2


def residual(W, s, down, up, prec: int, want_R: bool = False):
    W = _c(W, np.uint16)
    s = _c(s, np.float32)
    down = _c(down, np.uint16)
    up = _c(up, np.uint16)
    N, K = W.shape
    r = down.shape[0]
    G = K // group_of(prec)
    wq = np.zeros((N, K // 2), np.uint8)
    wscale = np.zeros((N, G), np.float32 if prec == INT4 else np.uint8)
    R = np.zeros((N, K), np.float32) if want_R else None
    lib().oracle_residual(_p(W), _p(s), _p(down), _p(up), N, K, r, prec, _p(wq), _p(wscale), _p(R))
    return (wq, wscale, R) if want_R else (wq, wscale)


def pack_weights(W, act_absmax, r: int = 32, prec: int = INT4):
    """The whole packing step with the oracle's own SVD."""
    s = smooth(W, act_absmax)
    down, up, _, _, _ = lowrank(W, s, r)
    wq, wscale = residual(W, s, down, up, prec)
    return dict(smooth=s, down=down, up=up, wq=wq, wscale=wscale)


# ---------------------------------------------------------------- runtime steps

def quant_act(X, s, down, prec: int):
    X = _c(X, np.uint16)
    s = _c(s, np.float32)
    down = _c(down, np.uint16)
    M, K = X.shape
    r = down.shape[0]
    G = K // group_of(prec)
    xq = np.zeros((M, K // 2), np.uint8)
    xscale = np.zeros((M, G), np.float32 if prec == INT4 else np.uint8)
    h = np.zeros((M, r), np.float64)
    lib().oracle_quant_act(_p(X), M, K, _p(s), _p(down), r, prec, _p(xq), _p(xscale), _p(h))
    return xq, xscale, h


def linear(xq, xscale, h, wq, wscale, up, bias, prec: int, gelu: bool = False,
           rows=None, parts: bool = False):
    """fp64 output for the given rows (all rows by default)."""
    xq = _c(xq, np.uint8)
    wq = _c(wq, np.uint8)
    h = _c(h, np.float64)
    up = _c(up, np.uint16)
    sdt = np.float32 if prec == INT4 else np.uint8
    xscale = _c(xscale, sdt)
    wscale = _c(wscale, sdt)
    bias = None if bias is None else _c(bias, np.uint16)
    M = xq.shape[0]
    N = wq.shape[0]
    K = xq.shape[1] * 2
    r = up.shape[1]
    if rows is None:
        rows_a = None
        nrows = M
    else:
        rows_a = _c(rows, np.int32)
        nrows = rows_a.size
    y = np.zeros((nrows, N), np.float64)
    yq = np.zeros((nrows, N), np.float64) if parts else None
    ylr = np.zeros((nrows, N), np.float64) if parts else None
    lib().oracle_linear(_p(xq), _p(xscale), _p(h), _p(wq), _p(wscale), _p(up), _p(bias),
                        M, N, K, r, prec, int(bool(gelu)), _p(rows_a), nrows, _p(y), _p(yq), _p(ylr))
    return (y, yq, ylr) if parts else y


def forward(X, packed: dict, bias, prec: int, gelu: bool = False, rows=None):
    """Quantize activations, then the linear, with the given packed weights."""
    xq, xscale, h = quant_act(X, packed["smooth"], packed["down"], prec)
    y = linear(xq, xscale, h, packed["wq"], packed["wscale"], packed["up"], bias, prec,
               gelu=gelu, rows=rows)
    return y, (xq, xscale, h)


# ----------------------------------------------------------------- decoding

def unpack_int4(codes: np.ndarray) -> np.ndarray:
    """Nibble-packed sign-magnitude INT4 -> int8 (element 2i in the low nibble)."""
    n = unpack_nibbles(codes).astype(np.int16)
    out = np.where(n & 8, -(n & 7), n & 7)
    return out.astype(np.int8)


def unpack_nibbles(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = c & 0x0F
    out[..., 1::2] = c >> 4
    return out


# ----------------------------------------------------------- AWQ W4A16 (INT4)
# The weight-only family of the same pages (section "Native loading in
# Diffusers": awq_w4a16, int4, group size 64, for the memory-bound modulation
# layers); the storage layout and the readings are stated in svdq_oracle.c.

def awq_pack(W):
    """bf16 bits [N][K] (K % 256 == 0) -> (wq uint8 [N][K/2], wscale fp32 [N][K/64])."""
    W = _c(W, np.uint16)
    N, K = W.shape
    wq = np.zeros((N, K // 2), np.uint8)
    wscale = np.zeros((N, K // 64), np.float32)
    lib().oracle_awq_pack(_p(W), N, K, _p(wq), _p(wscale))
    return wq, wscale


def awq_codes(wq) -> np.ndarray:
    """Stored rows -> int8 q [N][K] in natural k order."""
    wq = _c(wq, np.uint8)
    N, KB = wq.shape
    out = np.zeros((N, 2 * KB), np.int8)
    for n in range(N):
        row = np.ascontiguousarray(wq[n])
        for k in range(2 * KB):
            out[n, k] = lib().oracle_awq_code(_p(row), k)
    return out


def awq_linear(X, wq, wscale, bias=None):
    """fp64 y [M][N] of the weight-only layer (no bf16 rounding)."""
    X = _c(X, np.uint16)
    wq = _c(wq, np.uint8)
    wscale = _c(wscale, np.float32)
    bias = None if bias is None else _c(bias, np.uint16)
    M, K = X.shape
    N = wq.shape[0]
    y = np.zeros((M, N), np.float64)
    lib().oracle_awq_linear(_p(X), _p(wq), _p(wscale), _p(bias), M, N, K, _p(y))
    return y


# ---------------------------------------- QKV projection + Q/K RMS-norm + RoPE
# The fused attention-input step (section "Quantizing models with structural
# rewrites": the engine's fused_qkv_norm_rottary); readings in svdq_oracle.c.

def qkv_norm_rope(ylin, norm_q, norm_k, eps: float, rope_cos, rope_sin):
    """fp64 linear output [M][N] (N = 3 H 128, before bf16 rounding) ->
    fp64 [M][N]: Q and K heads RMS-normalized and rotated, V rounded only."""
    y = _c(ylin, np.float64)
    M, N = y.shape
    assert N % 384 == 0
    wq_, wk_ = _c(norm_q, np.uint16), _c(norm_k, np.uint16)
    c, s = _c(rope_cos, np.float32), _c(rope_sin, np.float32)
    out = np.zeros((M, N), np.float64)
    lib().oracle_qkv_norm_rope(_p(y), M, N, _p(wq_), _p(wk_), float(eps), _p(c), _p(s), _p(out))
    return out


# ------------------------------------------------------- NF4 W4A16 (weight-only)

def nf4_codebook() -> np.ndarray:
    """The 16 fp32 NF4 levels (ascending; level 7 is 0, levels 0 and 15 are -1, 1)."""
    c = np.zeros(16, np.float32)
    lib().oracle_nf4_codebook(_p(c))
    return c


def nf4_code(x: float) -> int:
    """Code of one normalized weight x = fl32(w / absmax)."""
    c = nf4_codebook()
    return int(lib().oracle_nf4_code(ctypes.c_float(float(x)), _p(c)))


def nf4_pack(W):
    """bf16 bits [N][K] (K % 64 == 0) -> (codes uint8 [N][K/2], statistic
    codes uint8 [N*K/64], chunk scales fp32 [ceil(N*K/64 / 256)])."""
    W = _c(W, np.uint16)
    N, K = W.shape
    nb = N * (K // 64)
    wq = np.zeros((N, K // 2), np.uint8)
    qabs = np.zeros(nb, np.uint8)
    chunk = np.zeros((nb + 255) // 256, np.float32)
    lib().oracle_nf4_pack(_p(W), N, K, _p(wq), _p(qabs), _p(chunk))
    return wq, qabs, chunk


def nf4_dequant(wq, qabs, chunk, N: int, K: int) -> np.ndarray:
    """Dequantized weights w' as bf16 bits [N][K]."""
    wq, qabs, chunk = _c(wq, np.uint8), _c(qabs, np.uint8), _c(chunk, np.float32)
    out = np.zeros((N, K), np.uint16)
    lib().oracle_nf4_dequant(_p(wq), _p(qabs), _p(chunk), N, K, _p(out))
    return out


def nf4_linear(X, wq, qabs, chunk, bias, rows=None) -> np.ndarray:
    """y = X W'^T + b in fp64 ([len(rows) or M][N])."""
    X = _c(X, np.uint16)
    wq, qabs, chunk = _c(wq, np.uint8), _c(qabs, np.uint8), _c(chunk, np.float32)
    M, K = X.shape
    N = wq.shape[0]
    b = None if bias is None else _c(bias, np.uint16)
    r = None if rows is None else _c(rows, np.int32)
    R = M if r is None else r.size
    out = np.zeros((R, N), np.float64)
    lib().oracle_nf4_linear(_p(X), _p(wq), _p(qabs), _p(chunk), _p(b), M, N, K, _p(r), 0 if r is None else r.size,
                            _p(out))
    return out
