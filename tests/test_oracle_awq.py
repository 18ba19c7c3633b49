"""Pins of the oracle's weight-only AWQ W4A16 routines (INT4, group 64):
hand-worked storage bytes, the storage order being a bijection, codes and
scales equal to the pinned group quantizer, and the output equal to a plain
float64 matrix product of the decoded weights."""
import json
import os

import numpy as np
import pytest

from oracle import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_bits(x):
    f = np.asarray(x, np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "fixture values must be bf16-exact"
    return (u >> 16).astype(np.uint16)


@pytest.mark.parametrize("entry", json.load(open(os.path.join(GOLD, "awq_layout.json")))["rows"],
                         ids=lambda e: e["id"])
def test_awq_layout_golden(entry):
    K = entry["K"]
    w = np.zeros(K, np.float32)
    for k, v in entry["nonzero"].items():
        w[int(k)] = v
    wq, ws = O.awq_pack(_bf16_bits(w)[None, :])
    expect = np.full(K // 2, int(entry["other_bytes"], 16), np.uint8)
    for b, v in entry["bytes"].items():
        expect[int(b)] = int(v, 16)
    assert wq[0].tolist() == expect.tolist()
    if "scale_hex" in entry:
        assert [f"{int(v):08x}" for v in ws[0].view(np.uint32)] == entry["scale_hex"]
    else:
        a, b = entry["scale_value_over"]
        assert ws[0, entry["scale_index"]] == np.float32(a / b)
        assert np.count_nonzero(ws[0]) == 1


def test_awq_layout_is_a_bijection():
    # one distinct non-zero code per position: decoding returns every k once
    K = 512
    rng = np.random.default_rng(3)
    for _ in range(3):
        q = rng.integers(-7, 8, size=K)
        q[::64] = 7                        # absmax 7 per group -> scale 1, codes = q
        wq, ws = O.awq_pack(_bf16_bits(q.astype(np.float32))[None, :])
        assert np.all(ws == 1.0)
        assert O.awq_codes(wq)[0].tolist() == q.tolist()
    # every nibble of the row is written by exactly one k
    hits = np.zeros((K // 2, 2), int)
    for k in range(K):
        w = np.zeros(K, np.float32)
        w[k] = 1.0
        wq, _ = O.awq_pack(_bf16_bits(w)[None, :])
        changed = np.nonzero(wq[0] != 0x88)[0]
        assert changed.size == 1
        byte = int(changed[0])
        high = int(wq[0, byte] >> 4) != 8
        hits[byte, int(high)] += 1
    assert np.all(hits == 1)


def test_awq_pack_matches_group_quantizer():
    rng = np.random.default_rng(7)
    N, K = 5, 768
    W = ((rng.standard_normal((N, K)) * 0.02).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wq, ws = O.awq_pack(W)
    q = O.awq_codes(wq)
    Wf = (W.astype(np.uint32) << 16).view(np.float32)
    for n in range(N):
        for g in range(K // 64):
            qq, sc = O.quant_group_int4(Wf[n, 64 * g: 64 * g + 64])
            assert ws[n, g] == sc
            assert q[n, 64 * g: 64 * g + 64].tolist() == qq.tolist()
            # dequantization error of every weight within scale / 2
            err = np.abs(Wf[n, 64 * g: 64 * g + 64].astype(np.float64) - qq.astype(np.float64) * np.float64(sc))
            assert np.all(err <= np.float64(sc) / 2)


@pytest.mark.parametrize("M,N,K,bias", [(1, 7, 256, True), (3, 4, 512, False), (16, 3, 768, True)])
def test_awq_linear_brute_force(M, N, K, bias):
    rng = np.random.default_rng(M * 100 + N)
    Xf = rng.standard_normal((M, K)).astype(np.float32)
    X = (Xf.view(np.uint32) >> 16).astype(np.uint16)
    Wf = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W = (Wf.view(np.uint32) >> 16).astype(np.uint16)
    b = (rng.standard_normal(N).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16) if bias else None
    wq, ws = O.awq_pack(W)
    y = O.awq_linear(X, wq, ws, b)
    Xd = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Wd = O.awq_codes(wq).astype(np.float64) * np.repeat(ws.astype(np.float64), 64, axis=1)
    ref = Xd @ Wd.T
    if bias:
        ref += (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)[None, :]
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    # a zero weight row gives the bias alone
    W0 = W.copy()
    W0[0] = 0
    wq0, ws0 = O.awq_pack(W0)
    y0 = O.awq_linear(X, wq0, ws0, b)
    expect0 = 0.0 if b is None else float((b[0].astype(np.uint32) << 16).view(np.float32))
    assert np.all(y0[:, 0] == expect0)
