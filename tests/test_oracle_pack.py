"""Pins of the oracle's packing and activation steps: the smoothing closed
form, Eckart-Young for the low-rank factors, the residual identity
X^ R + X L1 L2 = X W^T (up to the two fp32 roundings), and the activation
step against a numpy re-assembly."""
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import oracle as O
from w4a4_rank_corrected_quantize_amd import synth
from w4a4_rank_corrected_quantize_amd.synth import f32_to_bf16_bits, bf16_bits_to_f32

getcontext().prec = 60


def _small(N=96, K=192, M=40, seed=1):
    rng = np.random.default_rng(seed)
    X = f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32) *
                         np.where(rng.random(K) < 0.05, 30.0, 1.0).astype(np.float32))
    W = f32_to_bf16_bits(rng.normal(0, 0.02, (N, K)).astype(np.float32))
    return X, W


def test_smoothing_closed_form():
    rng = np.random.default_rng(3)
    N, K = 8, 512
    W = f32_to_bf16_bits((rng.standard_normal((N, K)) * 10.0 ** rng.uniform(-3, 1, K)).astype(np.float32))
    absmax = (np.abs(rng.standard_t(4, K)) * 10.0 ** rng.uniform(-2, 2, K)).astype(np.float32)
    s = O.smooth(W, absmax)
    mw = np.abs(bf16_bits_to_f32(W)).max(axis=0)
    for k in range(K):
        exact = (Decimal(float(mw[k])) / Decimal(float(absmax[k]))).sqrt()  # 1/lambda
        assert s[k] == np.float32(float(exact)) or \
            abs(float(s[k]) - float(exact)) <= float(np.spacing(np.float32(exact)))


def test_smoothing_special_cases():
    N, K = 4, 6
    W = np.zeros((N, K), np.uint16)
    Wf = np.zeros((N, K), np.float32)
    Wf[:, 0] = [0.5, -2.0, 1.0, 0.0]        # max 2
    Wf[:, 1] = 1.0
    Wf[:, 2] = 3.0
    Wf[:, 4] = 0.25
    Wf[:, 5] = 0.25
    W[:] = f32_to_bf16_bits(Wf)
    absmax = np.array([2.0, 1.0, 0.0, 5.0, 4.0, 4.0 * 30], np.float32)
    s = O.smooth(W, absmax)
    assert s[0] == 1.0                       # equal maxima -> lambda = 1
    assert s[1] == 1.0
    assert s[2] == 1.0                       # activation max 0 -> lambda = 1
    assert s[3] == 1.0                       # weight column all zero -> lambda = 1
    assert s[4] == np.float32(0.25)          # sqrt(4 / 0.25) = 4
    # an outlier channel x30 grows lambda by sqrt(30)
    assert abs(float(s[4]) / float(s[5]) - np.sqrt(30.0)) < 1e-6


def test_lowrank_eckart_young_and_orthonormality():
    X, W = _small()
    s = O.smooth(W, synth.calibration_absmax(X))
    down, up, S, L1, L2 = O.lowrank(W, s, 32)
    What = (bf16_bits_to_f32(W).astype(np.float64) / s.astype(np.float64)[None, :]).T
    err = np.sum((What - L1 @ L2) ** 2)
    assert abs(err - np.sum(S[32:] ** 2)) <= 1e-9 * np.sum(S ** 2)
    np.testing.assert_allclose(L2 @ L2.T, np.eye(32), atol=1e-12)
    G = L1.T @ L1
    np.testing.assert_allclose(np.diag(G), S[:32] ** 2, rtol=1e-10)
    np.testing.assert_allclose(G - np.diag(np.diag(G)), 0, atol=1e-9 * S[0] ** 2)
    # stored factors: down = bf16(s_k * L1_kj) laid out [r][K], up = bf16(L2^T) [N][r]
    d = bf16_bits_to_f32(down).astype(np.float64)
    np.testing.assert_allclose(d, (s.astype(np.float64)[:, None] * L1).T,
                               rtol=2.0 ** -8, atol=1e-30)
    np.testing.assert_allclose(bf16_bits_to_f32(up), L2.T, rtol=2.0 ** -8, atol=1e-30)


def test_rank_deficient_weight_leaves_tiny_residual():
    rng = np.random.default_rng(4)
    N, K = 64, 128
    # integer factors keep every entry bf16-exact, so W has rank <= 20 exactly
    A = (rng.integers(-3, 4, (N, 20)) @ rng.integers(-3, 4, (20, K))) * 2.0 ** -10
    assert np.abs(A).max() * 2 ** 10 <= 256
    W = f32_to_bf16_bits(A.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f32(W), A.astype(np.float32))
    s = np.ones(K, np.float32)
    down, up, S, _, _ = O.lowrank(W, s, 32)
    assert S[20] <= 1e-12 * S[0]
    _, _, R = O.residual(W, s, down, up, O.INT4, want_R=True)
    Wd = bf16_bits_to_f32(W).astype(np.float64)
    # only the bf16 rounding of the stored factors is left
    assert np.linalg.norm(R) <= 2.0 ** -6 * np.linalg.norm(Wd)


@pytest.mark.parametrize("prec", [O.INT4, O.MXFP4])
def test_residual_identity(prec):
    """sum_k xhat_mk R_kn + sum_k X_mk sum_j down[j][k] up[n][j] == sum_k X_mk W_nk
    up to the fp32 roundings of xhat and R."""
    X, W = _small(seed=5)
    s = O.smooth(W, synth.calibration_absmax(X))
    down, up, _, _, _ = O.lowrank(W, s, 32)
    _, _, R = O.residual(W, s, down, up, prec, want_R=True)
    Xd = bf16_bits_to_f32(X).astype(np.float64)
    xhat = (bf16_bits_to_f32(X) * s[None, :]).astype(np.float64)   # fp32 products
    Rd = R.astype(np.float64)
    lhs = xhat @ Rd.T + (Xd @ bf16_bits_to_f32(down).astype(np.float64).T) @ \
        bf16_bits_to_f32(up).astype(np.float64).T
    rhs = Xd @ bf16_bits_to_f32(W).astype(np.float64).T
    bound = 3 * 2.0 ** -24 * (np.abs(xhat) @ np.abs(Rd).T) + 1e-12 * np.abs(rhs).max()
    assert np.all(np.abs(lhs - rhs) <= bound)


@pytest.mark.parametrize("prec", [O.INT4, O.MXFP4])
def test_quant_act_reassembly(prec):
    X, W = _small(seed=6)
    s = O.smooth(W, synth.calibration_absmax(X))
    down, _, _, _, _ = O.lowrank(W, s, 32)
    xq, xscale, h = O.quant_act(X, s, down, prec)
    xhat = bf16_bits_to_f32(X) * s[None, :]             # IEEE fp32 product = fl32(exact)
    g = O.group_of(prec)
    for m in range(X.shape[0]):
        for b in range(X.shape[1] // g):
            v = xhat[m, g * b:g * b + g]
            if prec == O.INT4:
                q, sc, c = O.quant_group_int4(v, codes=True)
                assert xscale[m, b] == sc
                assert np.array_equal(xq[m, g * b // 2:(g * b + g) // 2], O.pack_nibbles(c))
            else:
                c, e = O.quant_block_mxfp4(v)
                assert xscale[m, b] == e
                assert np.array_equal(xq[m, g * b // 2:(g * b + g) // 2],
                                      ((c[0::2] & 15) | (c[1::2] << 4)).astype(np.uint8))
    ref_h = bf16_bits_to_f32(X).astype(np.float64) @ bf16_bits_to_f32(down).astype(np.float64).T
    np.testing.assert_allclose(h, ref_h, rtol=1e-12, atol=1e-12 * np.abs(ref_h).max())


def test_int4_dequant_error_bound_on_activation():
    X, W = _small(seed=7)
    s = O.smooth(W, synth.calibration_absmax(X))
    down, _, _, _, _ = O.lowrank(W, s, 32)
    xq, xscale, _ = O.quant_act(X, s, down, O.INT4)
    xhat = (bf16_bits_to_f32(X) * s[None, :]).astype(np.float64)
    q = O.unpack_int4(xq).astype(np.float64)
    sc = np.repeat(xscale.astype(np.float64), 64, axis=1)
    assert np.all(np.abs(xhat - q * sc) <= sc / 2)
