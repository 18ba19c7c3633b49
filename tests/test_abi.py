"""The C ABI: every function declared in include/svdq.h is exported, status
strings exist, and the device entry points validate their arguments (and the
device) before anything runs.  No GPU compute here."""
import ctypes
import os
import re

import numpy as np
import pytest

import w4a4_rank_corrected_quantize_amd as svdq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "svdq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(svdq_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert set(names) == set(svdq.EXPORTS)
    L = ctypes.CDLL(svdq.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    for code in svdq.STATUS:
        s = svdq.status_string(code)
        assert isinstance(s, str) and s
    assert svdq.status_string(12345) == "unknown status"
    assert svdq.version() >= 100


def _host(nbytes, offset=0):
    buf = np.zeros(nbytes + 64, np.uint8)
    base = (-buf.ctypes.data) % 16
    return buf, ctypes.c_void_p(buf.ctypes.data + base + offset)


def test_device_call_validation_order():
    """Shape / enum / rank / NULL / alignment errors come before the device check."""
    L = svdq.lib()
    _, p = _host(1 << 16)
    _, q = _host(1 << 16, offset=4)
    M, K = 16, 128
    assert L.svdq_quantize_act(p, M, 96, p, p, 32, svdq.INT4, p, p, p, None) == -2
    assert L.svdq_quantize_act(p, M, K, p, p, 16, svdq.INT4, p, p, p, None) == -4
    assert L.svdq_quantize_act(p, M, K, p, p, 32, 7, p, p, p, None) == -1
    assert L.svdq_quantize_act(None, M, K, p, p, 32, svdq.INT4, p, p, p, None) == -1
    assert L.svdq_quantize_act(p, -1, K, p, p, 32, svdq.INT4, p, p, p, None) == -1
    assert L.svdq_quantize_act(q, M, K, p, p, 32, svdq.INT4, p, p, p, None) == -3
    assert L.svdq_w4a4_linear(p, p, p, p, p, p, None, M, 12, K, 32, svdq.INT4, 0, p, None) == -2
    assert L.svdq_w4a4_linear(p, p, p, p, p, p, None, M, 16, K, 32, svdq.INT4, 5, p, None) == -1
    assert L.svdq_w4a4_linear(p, p, p, p, p, p, q, M, 16, K, 32, svdq.INT4, 0, p, None) == -3
    assert L.svdq_w4a4_linear(p, p, p, p, p, p, None, M, 16, 96, 32, svdq.MXFP4, 0, None, None) == -1
    assert L.svdq_quantize_act(None, 0, K, None, p, 32, svdq.INT4, p, p, p, None) == -1   # smooth needed


def test_requant_validation_and_workspace():
    """The fused next-layer entry point: workspace size, and its argument
    errors before the device check."""
    L = svdq.lib()
    assert L.svdq_requant_workspace_bytes(0, 256, 32, svdq.INT4) == 0
    assert L.svdq_requant_workspace_bytes(100, 256, 32, svdq.INT4) == 1 * 100 * 32 * 4
    assert L.svdq_requant_workspace_bytes(100, 320, 32, svdq.INT4) == 2 * 100 * 32 * 4
    assert L.svdq_requant_workspace_bytes(4608, 12288, 32, svdq.INT4) == 48 * 4608 * 32 * 4
    _, p = _host(1 << 20)
    _, q = _host(1 << 16, offset=4)
    M, N, K = 16, 128, 128
    W = L.svdq_requant_workspace_bytes(M, N, 32, svdq.INT4)

    def call(**kw):
        a = dict(xq=p, xs=p, h=p, wq=p, ws=p, up=p, bias=None, M=M, N=N, K=K, r=32, prec=svdq.INT4, epi=0,
                 s2=p, d2=p, xq2=p, xs2=p, h2=p, work=p, wb=W)
        a.update(kw)
        return L.svdq_w4a4_linear_requant(a["xq"], a["xs"], a["h"], a["wq"], a["ws"], a["up"], a["bias"], a["M"],
                                          a["N"], a["K"], a["r"], a["prec"], a["epi"], a["s2"], a["d2"], a["xq2"],
                                          a["xs2"], a["h2"], a["work"], a["wb"], None)
    assert call(N=96) == -2                     # N must be a multiple of 64 (the next layer's K)
    assert call(prec=svdq.MXFP4) == -4          # MXFP4 needs K % 256 == 0
    assert call(r=16) == -4
    assert call(epi=3) == -1
    assert call(wb=W - 1) == -1                 # workspace too small
    assert call(s2=None) == -1
    assert call(work=None) == -1
    assert call(d2=q) == -3
    assert call(work=q) == -3
    if not _has_gpu():
        assert call() == -5
        assert call(prec=svdq.MXFP4, K=256) == -5


def test_qkv_norm_rope_validation():
    """The fused QKV + Q/K norm + rotary entry point: argument errors before
    the device check."""
    L = svdq.lib()
    _, p = _host(1 << 16)
    _, q = _host(1 << 16, offset=4)

    def call(**kw):
        a = dict(xq=p, xs=p, h=p, wq=p, ws=p, up=p, bias=None, M=16, N=384, K=128, r=32, prec=svdq.INT4,
                 nq=p, nk=p, eps=1e-6, c=p, s=p, Y=p)
        a.update(kw)
        return L.svdq_w4a4_linear_qkv_norm_rope(a["xq"], a["xs"], a["h"], a["wq"], a["ws"], a["up"], a["bias"],
                                                a["M"], a["N"], a["K"], a["r"], a["prec"], a["nq"], a["nk"],
                                                ctypes.c_float(a["eps"]), a["c"], a["s"], a["Y"], None)
    assert call(N=256) == -2                    # N = 3 H 128
    assert call(prec=svdq.MXFP4) == -4         # INT4 only
    assert call(eps=-1.0) == -1
    assert call(eps=float("nan")) == -1
    assert call(eps=float("inf")) == -1
    assert call(r=16) == -4
    assert call(nq=None) == -1
    assert call(c=None) == -1
    assert call(s=q) == -3
    assert call(nk=q) == -3
    assert call(K=96) == -2
    if not _has_gpu():
        assert call() == -5


def test_awq_validation():
    """The weight-only AWQ W4A16 entry point: argument errors before the
    device check."""
    L = svdq.lib()
    _, p = _host(1 << 16)
    _, q = _host(1 << 16, offset=4)
    M, N, K = 2, 32, 256
    assert L.svdq_awq_w4a16_linear(p, p, p, None, M, N, 192, p, None) == -2      # K % 256
    assert L.svdq_awq_w4a16_linear(p, p, p, None, M, N, 0, p, None) == -2
    assert L.svdq_awq_w4a16_linear(p, p, p, None, -1, N, K, p, None) == -1
    assert L.svdq_awq_w4a16_linear(None, p, p, None, M, N, K, p, None) == -1
    assert L.svdq_awq_w4a16_linear(p, p, None, None, M, N, K, p, None) == -1
    assert L.svdq_awq_w4a16_linear(p, p, p, None, M, N, K, None, None) == -1
    assert L.svdq_awq_w4a16_linear(p, p, p, q, M, N, K, p, None) == -3
    assert L.svdq_awq_w4a16_linear(q, p, p, None, M, N, K, p, None) == -3
    assert L.svdq_awq_pack_weights(None, 4, 256, p, p) == -1
    if not _has_gpu():
        assert L.svdq_awq_w4a16_linear(p, p, p, None, M, N, K, p, None) == -5
        assert L.svdq_awq_w4a16_linear(None, p, p, None, 0, N, K, None, None) == -5   # empty: still checks the device


def test_splitk_validation():
    """The split-K linear: argument errors before the device check; no
    workspace is asked for without a device or for shapes it does not split."""
    L = svdq.lib()
    _, p = _host(1 << 16)
    _, q = _host(1 << 16, offset=4)

    def call(**kw):
        a = dict(xq=p, xs=p, h=p, wq=p, ws=p, up=p, bias=None, M=16, N=64, K=2048, r=32, prec=svdq.MXFP4, epi=0,
                 Y=p, work=p, wb=1 << 16)
        a.update(kw)
        return L.svdq_w4a4_linear_splitk(a["xq"], a["xs"], a["h"], a["wq"], a["ws"], a["up"], a["bias"], a["M"],
                                         a["N"], a["K"], a["r"], a["prec"], a["epi"], a["Y"], a["work"], a["wb"],
                                         None)
    assert call(N=12) == -2
    assert call(K=2040) == -2
    assert call(r=16) == -4
    assert call(epi=3) == -1
    assert call(Y=None) == -1
    assert call(work=q) == -3
    assert call(Y=q) == -3
    assert L.svdq_w4a4_linear_splitk_workspace_bytes(16, 64, 2048, svdq.INT4) == 0
    assert L.svdq_w4a4_linear_splitk_workspace_bytes(0, 64, 2048, svdq.MXFP4) == 0
    assert L.svdq_w4a4_linear_splitk_workspace_bytes(16, 64, 2040, svdq.MXFP4) == 0
    if not _has_gpu():
        assert call() == -5
        assert L.svdq_w4a4_linear_splitk_workspace_bytes(16, 64, 2048, svdq.MXFP4) == 0


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="checks the no-GPU path")
def test_no_gpu_means_unsupported_device():
    L = svdq.lib()
    _, p = _host(1 << 16)
    assert L.svdq_check_device() == -5
    assert L.svdq_quantize_act(p, 16, 128, p, p, 32, svdq.INT4, p, p, p, None) == -5
    assert L.svdq_w4a4_linear(p, p, p, p, p, p, None, 16, 16, 128, 32, svdq.INT4, 0, p, None) == -5
    with pytest.raises(svdq.SvdqError):
        svdq.check_device()


def test_matrices_of_2_30_elements_are_rejected():
    """Every matrix a call touches must hold fewer than 2^30 elements, so the
    kernels' 32-bit byte offsets (the LDS-DMA lane offsets among them) cannot
    wrap: larger shapes return SVDQ_ERR_SHAPE before the device check, and the
    split-K workspace query returns 0 for them."""
    L = svdq.lib()
    _, p = _host(1 << 16)
    big = 1 << 21                      # 2^21 rows x 512 channels = 2^30 elements
    I, MX = svdq.INT4, svdq.MXFP4
    assert L.svdq_quantize_act(p, big, 512, p, p, 32, I, p, p, p, None) == -2
    assert L.svdq_quantize_act(p, big - 1, 512, p, p, 32, I, p, p, p, None) != -2
    # weights N x K, activations M x K, output M x N
    assert L.svdq_w4a4_linear(p, p, p, p, p, p, None, 16, big, 512, 32, I, 0, p, None) == -2
    assert L.svdq_w4a4_linear(p, p, p, p, p, p, None, big, 16, 512, 32, MX, 0, p, None) == -2
    assert L.svdq_w4a4_linear(p, p, p, p, p, p, None, 1 << 15, 1 << 15, 64, 32, I, 0, p, None) == -2
    assert L.svdq_w4a4_linear_splitk(p, p, p, p, p, p, None, 16, big, 512, 32, MX, 0, p, p, 1 << 16, None) == -2
    assert L.svdq_w4a4_linear_splitk_workspace_bytes(16, big, 512, MX) == 0
    assert L.svdq_w4a4_linear_requant(p, p, p, p, p, p, None, 16, big, 512, 32, I, 0, p, p, p, p, p, p,
                                      1 << 16, None) == -2
    assert L.svdq_w4a4_linear_qkv_norm_rope(p, p, p, p, p, p, None, 16, 3 * (1 << 21), 512, 32, I, p, p,
                                            ctypes.c_float(0.0), p, p, p, None) == -2
    assert L.svdq_awq_w4a16_linear(p, p, p, None, 16, big, 512, p, None) == -2
    # host packing of an N x K weight
    assert L.svdq_awq_pack_weights(p, big, 512, p, p) == -2
    assert L.svdq_pack_residual(p, p, p, p, big, 512, 32, I, p, p) == -2
    assert L.svdq_pack_weights(p, p, big, 512, 32, I, p, p, p, p, p) == -2
