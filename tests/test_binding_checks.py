"""The Python binding checks every tensor's shape and dtype against the shapes
the call implies (M, K from the activation codes, N from the weight codes, the
rank from `up`, the scale dtype from the precision) before any library call,
so a buffer of the wrong size can never reach a kernel.  The checks run before
the device check, so these tests need no GPU: CPU tensors of the wrong shape
raise ValueError, CPU tensors of the right shape get as far as the device
check (TypeError)."""
import numpy as np
import pytest

import w4a4_rank_corrected_quantize_amd as svdq

torch = pytest.importorskip("torch")

M, K, N, R = 40, 256, 64, 32
BF, F32, U8 = torch.bfloat16, torch.float32, torch.uint8


def _z(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def _linear_set(prec):
    g = svdq.group_of(prec)
    sd = F32 if prec == svdq.INT4 else U8
    return dict(xq=_z((M, K // 2), U8), xscale=_z((M, K // g), sd), h=_z((M, R), F32),
                wq=_z((N, K // 2), U8), wscale=_z((N, K // g), sd), up=_z((N, R), BF), bias=_z((N,), BF))


def _call_linear(d, prec, **kw):
    return svdq.w4a4_linear(d["xq"], d["xscale"], d["h"], d["wq"], d["wscale"], d["up"], d["bias"], prec, **kw)


@pytest.mark.parametrize("prec", [svdq.INT4, svdq.MXFP4])
def test_linear_right_shapes_reach_the_device_check(prec):
    with pytest.raises(TypeError, match="device tensor"):
        _call_linear(_linear_set(prec), prec, Y=_z((M, N), BF))


@pytest.mark.parametrize("prec", [svdq.INT4, svdq.MXFP4])
@pytest.mark.parametrize("name,bad", [
    ("xscale", lambda p: (M, K // 32 if p == svdq.INT4 else K // 64)),   # the other precision's group count
    ("h", lambda p: (M + 1, R)),
    ("wq", lambda p: (N, K // 2 - 16)),
    ("wscale", lambda p: (N + 8, K // svdq.group_of(p))),
    ("up", lambda p: (N - 8, R)),
    ("bias", lambda p: (N + 8,)),
])
def test_linear_wrong_shape_raises(prec, name, bad):
    d = _linear_set(prec)
    d[name] = _z(bad(prec), d[name].dtype)
    with pytest.raises(ValueError, match=name):
        _call_linear(d, prec)


def test_linear_wrong_output_shape_raises():
    d = _linear_set(svdq.INT4)
    with pytest.raises(ValueError, match="Y"):
        _call_linear(d, svdq.INT4, Y=_z((M, N + 8), BF))


def test_scale_dtype_follows_precision():
    """INT4 takes fp32 scales only, MXFP4 E8M0 bytes only: a uint8 buffer sized
    for MXFP4 passed as INT4 scales would be half the bytes the kernel writes."""
    d = _linear_set(svdq.INT4)
    d["xscale"] = _z((M, K // 32), U8)
    with pytest.raises(TypeError, match="xscale"):
        _call_linear(d, svdq.INT4)
    with pytest.raises(TypeError, match="xscale"):
        svdq.quantize_act(_z((M, K), BF), _z((K,), F32), _z((R, K), BF), svdq.INT4, xscale=_z((M, K // 64), U8))
    d = _linear_set(svdq.MXFP4)
    d["wscale"] = _z((N, K // 32), F32)
    with pytest.raises(TypeError, match="wscale"):
        _call_linear(d, svdq.MXFP4)


def test_bad_precision_raises():
    with pytest.raises(ValueError, match="prec"):
        _call_linear(_linear_set(svdq.INT4), 7)


@pytest.mark.parametrize("name,shape", [("smooth", (K + 64,)), ("down", (R, K - 64)), ("xq", (M, K // 2 + 1)),
                                        ("xscale", (M - 1, K // 64)), ("h", (M, R + 1))])
def test_quantize_act_wrong_shape_raises(name, shape):
    args = dict(X=_z((M, K), BF), smooth=_z((K,), F32), down=_z((R, K), BF), xq=_z((M, K // 2), U8),
                xscale=_z((M, K // 64), F32), h=_z((M, R), F32))
    args[name] = _z(shape, args[name].dtype)
    with pytest.raises(ValueError, match=name):
        svdq.quantize_act(args["X"], args["smooth"], args["down"], svdq.INT4, xq=args["xq"],
                          xscale=args["xscale"], h=args["h"])


@pytest.mark.parametrize("name,shape", [("smooth2", (N + 64,)), ("down2", (R, N - 64)), ("xq2", (M, N)),
                                        ("xscale2", (M, N // 32)), ("h2", (M + 1, R))])
def test_requant_wrong_shape_raises(name, shape):
    d = _linear_set(svdq.INT4)
    ex = dict(smooth2=_z((N,), F32), down2=_z((R, N), BF), xq2=_z((M, N // 2), U8), xscale2=_z((M, N // 64), F32),
              h2=_z((M, R), F32))
    ex[name] = _z(shape, ex[name].dtype)
    with pytest.raises(ValueError, match=name):
        svdq.w4a4_linear_requant(d["xq"], d["xscale"], d["h"], d["wq"], d["wscale"], d["up"], d["bias"],
                                 ex["smooth2"], ex["down2"], svdq.INT4,
                                 out=(ex["xq2"], ex["xscale2"], ex["h2"]), work=_z((1 << 16,), U8))


@pytest.mark.parametrize("name,shape", [("norm_q", (64,)), ("norm_k", (256,)), ("rope_cos", (M, 32)),
                                        ("rope_sin", (M + 1, 64))])
def test_qkv_norm_rope_wrong_shape_raises(name, shape):
    n = 384
    d = _linear_set(svdq.INT4)
    d.update(wq=_z((n, K // 2), U8), wscale=_z((n, K // 64), F32), up=_z((n, R), BF), bias=_z((n,), BF))
    ex = dict(norm_q=_z((128,), BF), norm_k=_z((128,), BF), rope_cos=_z((M, 64), F32), rope_sin=_z((M, 64), F32))
    ex[name] = _z(shape, ex[name].dtype)
    with pytest.raises(ValueError, match=name):
        svdq.w4a4_linear_qkv_norm_rope(d["xq"], d["xscale"], d["h"], d["wq"], d["wscale"], d["up"], d["bias"],
                                       ex["norm_q"], ex["norm_k"], 1e-6, ex["rope_cos"], ex["rope_sin"])


@pytest.mark.parametrize("name,shape", [("wq", (N, K // 4)), ("wscale", (N, K // 32)), ("bias", (N - 1,)),
                                        ("Y", (M, N + 1))])
def test_awq_wrong_shape_raises(name, shape):
    a = dict(X=_z((M, K), BF), wq=_z((N, K // 2), U8), wscale=_z((N, K // 64), F32), bias=_z((N,), BF),
             Y=_z((M, N), BF))
    a[name] = _z(shape, a[name].dtype)
    with pytest.raises(ValueError, match=name):
        svdq.awq_w4a16_linear(a["X"], a["wq"], a["wscale"], a["bias"], Y=a["Y"])


def test_host_pack_shape_checks():
    W = np.zeros((N, K), np.uint16)
    with pytest.raises(ValueError, match="act_absmax"):
        svdq.pack_weights(W, np.ones(K + 1, np.float32))
    with pytest.raises(ValueError, match="up"):
        svdq.pack_residual(W, np.ones(K, np.float32), np.zeros((R, K), np.uint16), np.zeros((N + 1, R), np.uint16))
