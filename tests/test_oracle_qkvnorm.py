"""Pins of the oracle's QKV norm + rotary step: special cases that reduce it
to a plain division or an exact permutation, and the invariants of each part
(the normalized head has mean square ms / (ms + eps) with unit weights; a
rotation keeps every pair's length; V heads are only rounded; scaling a head
by 2 changes nothing when eps = 0)."""
import numpy as np
import pytest

from oracle import oracle as O

ONE = np.uint16(0x3F80)          # bf16 1.0


def _bf16(x):
    f = np.asarray(x, np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _case(M=3, H=2, seed=0):
    rng = np.random.default_rng(seed)
    N = 384 * H
    # bf16-exact linear outputs, so the rounding step is the identity
    y = (_bf16(rng.standard_normal((M, N)).astype(np.float32)).astype(np.uint32) << 16).view(np.float32)
    return y.astype(np.float64), N


def test_identity_rotation_unit_weights_is_rms_division():
    y, N = _case()
    M = y.shape[0]
    wq = np.full(128, ONE)
    c = np.ones((M, 64), np.float32)
    s = np.zeros((M, 64), np.float32)
    out = O.qkv_norm_rope(y, wq, wq, 0.0, c, s)
    H = N // 384
    for m in range(M):
        for hd in range(3 * H):
            yh = y[m, 128 * hd: 128 * hd + 128]
            oh = out[m, 128 * hd: 128 * hd + 128]
            if hd < 2 * H:
                rms = np.sqrt(np.mean(yh * yh))
                assert np.allclose(oh * rms, yh, rtol=1e-14, atol=0)
                assert abs(np.mean(oh * oh) - 1.0) < 1e-13
            else:
                assert np.array_equal(oh, yh)          # V: bf16-exact input passes through


def test_quarter_turn_is_an_exact_pair_swap():
    y, N = _case(seed=1)
    M = y.shape[0]
    w = _bf16(np.random.default_rng(2).uniform(0.5, 1.5, 128).astype(np.float32))
    c0, s0 = np.ones((M, 64), np.float32), np.zeros((M, 64), np.float32)
    c1, s1 = np.zeros((M, 64), np.float32), np.ones((M, 64), np.float32)
    base = O.qkv_norm_rope(y, w, w, 1e-6, c0, s0)
    turned = O.qkv_norm_rope(y, w, w, 1e-6, c1, s1)
    H = N // 384
    qk = slice(0, 256 * H)
    assert np.array_equal(turned[:, qk][:, 0::2], -base[:, qk][:, 1::2])
    assert np.array_equal(turned[:, qk][:, 1::2], base[:, qk][:, 0::2])


def test_rotation_keeps_pair_lengths_and_weights_scale_channels():
    y, N = _case(M=4, H=1, seed=3)
    M = y.shape[0]
    rng = np.random.default_rng(4)
    th = rng.uniform(0, 2 * np.pi, (M, 64))
    c, s = np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)
    # keep c^2 + s^2 = 1 exactly enough: renormalize in fp64 after fp32 rounding
    w = np.full(128, ONE)
    rot = O.qkv_norm_rope(y, w, w, 1e-6, c, s)
    flat = O.qkv_norm_rope(y, w, w, 1e-6, np.ones_like(c), np.zeros_like(s))
    cc = c.astype(np.float64) ** 2 + s.astype(np.float64) ** 2
    for hd in range(2):
        a = rot[:, 128 * hd: 128 * hd + 128]
        b = flat[:, 128 * hd: 128 * hd + 128]
        la = a[:, 0::2] ** 2 + a[:, 1::2] ** 2
        lb = (b[:, 0::2] ** 2 + b[:, 1::2] ** 2) * cc
        assert np.allclose(la, lb, rtol=1e-12, atol=1e-15)
    # a weight of 2 on channel d doubles that channel before the rotation
    w2 = w.copy()
    w2[10] = _bf16(np.float32(2.0))
    f2 = O.qkv_norm_rope(y, w2, w, 1e-6, np.ones_like(c), np.zeros_like(s))
    assert np.array_equal(f2[:, 10], 2 * flat[:, 10])
    assert np.array_equal(np.delete(f2[:, :128], 10, axis=1), np.delete(flat[:, :128], 10, axis=1))


def test_scale_invariance_without_eps_and_rounding_of_inputs():
    y, N = _case(M=2, H=1, seed=5)
    M = y.shape[0]
    w = _bf16(np.random.default_rng(6).uniform(0.5, 1.5, 128).astype(np.float32))
    th = np.random.default_rng(7).uniform(0, 2 * np.pi, (M, 64))
    c, s = np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)
    a = O.qkv_norm_rope(y, w, w, 0.0, c, s)
    b = O.qkv_norm_rope(2.0 * y, w, w, 0.0, c, s)
    assert np.allclose(a[:, :256], b[:, :256], rtol=1e-14, atol=1e-15)
    assert np.array_equal(2 * a[:, 256:], b[:, 256:])            # V scales with its input
    # the linear output is rounded to bf16 first: a perturbation below half
    # a bf16 ulp of every value changes nothing
    tiny = y * (1 + 2.0 ** -12)
    assert np.array_equal(O.qkv_norm_rope(tiny, w, w, 1e-6, c, s), O.qkv_norm_rope(y, w, w, 1e-6, c, s))


@pytest.mark.parametrize("value,eps,want", [
    (2.0, 12.0, 0.5),        # mean square 4: 1 / sqrt(4 + 12) = 1/4
    (3.0, 7.0, 0.75),        # mean square 9: 3 / sqrt(16)
    (1.0, 3.0, 0.5),         # eps three times the mean square
    (0.5, 0.0, 1.0),         # no eps: every value becomes 1
])
def test_eps_closed_forms(value, eps, want):
    """Worked by hand: a head whose 128 values all have magnitude v has mean
    square v^2, so with unit weights and no rotation each output is
    +-v / sqrt(v^2 + eps).  eps outside the square root (v / (v + eps)),
    added to the sum of squares instead of the mean (v / sqrt(v^2 + eps /
    128)) or left out would give other values in every case with eps > 0."""
    M, H = 2, 1
    y = np.full((M, 384 * H), value, np.float64)
    y[:, 1::2] *= -1.0                          # signs must pass through
    w = np.full(128, ONE)
    out = O.qkv_norm_rope(y, w, w, eps, np.ones((M, 64), np.float32), np.zeros((M, 64), np.float32))
    sign = np.where(np.arange(128) % 2 == 0, 1.0, -1.0)
    for hd in range(2):
        assert np.array_equal(out[:, 128 * hd: 128 * hd + 128], np.tile(want * sign, (M, 1)))
    assert np.array_equal(out[:, 256:], y[:, 256:])


def test_eps_with_mixed_magnitudes():
    """Half the channels 4, half 0: mean square 8; eps = 1 gives sqrt(9) = 3,
    so the outputs are 4/3 and 0 (4/3 rounded once in fp64)."""
    y = np.zeros((1, 384), np.float64)
    y[0, 0:128:2] = 4.0
    y[0, 128:256:2] = -4.0
    w = np.full(128, ONE)
    out = O.qkv_norm_rope(y, w, w, 1.0, np.ones((1, 64), np.float32), np.zeros((1, 64), np.float32))
    assert np.all(np.abs(out[0, 0:128:2] - 4.0 / 3.0) <= 2.0 ** -51)
    assert np.all(np.abs(out[0, 128:256:2] + 4.0 / 3.0) <= 2.0 ** -51)
    assert np.all(out[0, 1:256:2] == 0.0)
