"""Pins of the oracle's group quantizers: hand-worked vectors, exact rational
brute force on random and adversarial near-tie groups, and the invariants
(|v - q*scale| <= scale/2, codes in range, nibble round trip)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O
from tests import _exact as E

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f32_from(x):
    if isinstance(x, str):
        return np.float32(float.fromhex(x))
    return np.float32(x)


def _group(entry, width):
    x = [_f32_from(v) for v in entry["x"]]
    s = np.float32(entry["s"]) if "s" in entry else np.float32(1)
    v = np.zeros(width, np.float32)
    v[: len(x)] = [np.float32(np.float64(a) * np.float64(s)) for a in x]
    return v


# ------------------------------------------------------------------ golden

@pytest.mark.parametrize("entry", json.load(open(os.path.join(GOLD, "int4_groups.json")))["groups"],
                         ids=lambda e: e["id"])
def test_int4_golden(entry):
    v = _group(entry, 64)
    q, scale, c = O.quant_group_int4(v, codes=True)
    assert int(np.float32(scale).view(np.uint32)) == int(entry["scale_hex"], 16)
    n = len(entry["codes"])
    assert q[:n].tolist() == entry["codes"]
    assert c[:n].tolist() == entry["nibbles"]
    assert not q[n:].any() and not c[n:].any()
    packed = O.pack_nibbles(c)
    want = bytes.fromhex(entry["bytes_hex"])
    assert packed[: len(want)].tobytes() == want
    assert not packed[len(want):].any()


@pytest.mark.parametrize("entry", json.load(open(os.path.join(GOLD, "mxfp4_blocks.json")))["blocks"],
                         ids=lambda e: e["id"])
def test_mxfp4_golden(entry):
    v = _group(entry, 32)
    codes, e = O.quant_block_mxfp4(v)
    assert e == int(entry["e8m0_hex"], 16)
    n = len(entry["codes"])
    assert codes[:n].tolist() == entry["codes"]
    assert not codes[n:].any()
    packed = (codes[0::2] & 0xF) | (codes[1::2] << 4)
    want = bytes.fromhex(entry["bytes_hex"])
    assert packed[: len(want)].astype(np.uint8).tobytes() == want


def test_mxfp4_golden_m2_dequant():
    v = np.zeros(32, np.float32)
    v[:3] = [0.3, -0.15, 0.05]
    codes, e = O.quant_block_mxfp4(v)
    deq = [O.e2m1_value(int(c)) * O.e8m0_value(e) for c in codes[:3]]
    assert deq == [0.25, -0.125, 0.0625]


# -------------------------------------------------- exact brute force, INT4

def _near_tie_groups(rng, count):
    """Groups whose entries sit at (k + 1/2) * scale, or one ulp either side."""
    out = []
    for _ in range(count):
        a = np.float32(rng.uniform(0.5, 2.0) * 2.0 ** rng.integers(-20, 20))
        scale = np.float32(np.float64(a) / 7.0)
        v = np.zeros(64, np.float32)
        v[0] = a * (1 if rng.random() < 0.5 else -1)
        for i in range(1, 64):
            k = int(rng.integers(0, 7))
            t = np.float32(np.float64(k + 0.5) * np.float64(scale))
            t = [np.nextafter(t, np.float32(-np.inf)), t, np.nextafter(t, np.float32(np.inf))][
                int(rng.integers(0, 3))]
            if abs(t) > a:
                t = a
            v[i] = t * (1 if rng.random() < 0.5 else -1)
        out.append(v)
    return out


def _check_int4(v):
    q, scale, c = O.quant_group_int4(v, codes=True)
    qe, se = E.quant_group_int4_exact(v)
    assert Fraction(float(scale)) == se
    assert q.tolist() == qe
    assert c.tolist() == [(8 if np.signbit(x) else 0) | abs(k) for x, k in zip(v, qe)]
    # invariant: dequantization error at most scale/2, exactly
    for x, c in zip(v, q):
        assert abs(Fraction(float(x)) - c * se) <= se / 2
    assert np.all(np.abs(q) <= 7)


def test_int4_exact_random():
    rng = np.random.default_rng(11)
    for _ in range(150):
        v = (rng.standard_normal(64) * 2.0 ** rng.integers(-30, 30)).astype(np.float32)
        _check_int4(v)


def test_int4_exact_near_ties():
    rng = np.random.default_rng(12)
    for v in _near_tie_groups(rng, 250):
        _check_int4(v)


def test_int4_exact_subnormal_and_extremes():
    rng = np.random.default_rng(13)
    tiny = np.float32(2.0 ** -149)
    cases = [
        np.full(64, tiny, np.float32),
        (rng.integers(-300, 300, 64) * tiny).astype(np.float32),
        (rng.standard_normal(64) * 1e38).astype(np.float32),
        np.array([np.float32(3.4e38)] + [np.float32(-1e-45)] * 63, np.float32),
        np.array([-0.0] * 64, np.float32),
    ]
    for v in cases:
        _check_int4(v)


def test_int4_tie_trap_is_not_reciprocal_multiply():
    """Multiplying by fl32(7/absmax) differs from the exact rule (G4)."""
    v = np.zeros(64, np.float32)
    v[:2] = [1.0, 0.5]
    q, scale = O.quant_group_int4(v)
    naive = np.rint(np.float32(0.5) * np.float32(np.float32(7) / np.float32(1.0)))
    assert naive == 4 and q[1] == 3
    # the naive code breaks the error bound, the exact one keeps it
    assert abs(Fraction(0.5) - 4 * Fraction(float(scale))) > Fraction(float(scale)) / 2


def test_nibble_round_trip():
    rng = np.random.default_rng(14)
    c = rng.integers(0, 16, 4096).astype(np.uint8)
    packed = O.pack_nibbles(c)
    assert packed[0] == (int(c[0]) | (int(c[1]) << 4))
    assert np.array_equal(O.unpack_nibbles(packed), c)
    want = np.array([E.int4_code(int(x)) for x in c], np.int8)
    assert np.array_equal(O.unpack_int4(packed), want)
    assert [O.int4_value(x) for x in range(16)] == [0, 1, 2, 3, 4, 5, 6, 7, 0, -1, -2, -3, -4, -5, -6, -7]


# ------------------------------------------------- exact brute force, MXFP4

def test_mxfp4_exhaustive_grid_and_midpoints():
    """Every grid point, every midpoint and their fp32 neighbours, at several
    block exponents, against the exact rational conversion."""
    pts = set()
    for g in E.E2M1:
        pts.add(float(g))
    for a, b in zip(E.E2M1[:-1], E.E2M1[1:]):
        pts.add(float((a + b) / 2))
    pts.update([6.5, 7.0, 7.75, 7.999999])
    base = sorted(pts)
    for X in (-127, -100, -10, -3, 0, 1, 5, 100, 125):
        vals = []
        for t in base:
            f = np.float32(np.ldexp(t, X))
            vals += [np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf))]
        vals = np.array([v for v in vals if np.isfinite(v)], np.float32)
        for i in range(0, len(vals), 31):
            blk = np.zeros(32, np.float32)
            chunk = vals[i:i + 31]
            blk[: chunk.size] = chunk
            blk[31] = np.float32(np.ldexp(7.0, X)) if np.isfinite(np.ldexp(7.0, X)) else 0
            sign = np.where(np.random.default_rng(i + X + 200).random(32) < 0.5, -1, 1)
            blk = (blk * sign).astype(np.float32)
            codes, e = O.quant_block_mxfp4(blk)
            ce, ee = E.quant_block_mxfp4_exact(blk)
            assert e == ee
            assert codes.tolist() == ce


def test_mxfp4_random_blocks():
    rng = np.random.default_rng(15)
    for _ in range(200):
        blk = (rng.standard_t(4, 32) * 2.0 ** rng.integers(-40, 40)).astype(np.float32)
        codes, e = O.quant_block_mxfp4(blk)
        ce, ee = E.quant_block_mxfp4_exact(blk)
        assert e == ee and codes.tolist() == ce


def test_mxfp4_zero_and_negative_zero():
    blk = np.zeros(32, np.float32)
    blk[1] = -0.0
    codes, e = O.quant_block_mxfp4(blk)
    assert e == 0 and codes[0] == 0 and codes[1] == 8


def test_mxfp4_decode_tables():
    assert [O.e2m1_value(c) for c in range(8)] == [0, .5, 1, 1.5, 2, 3, 4, 6]
    assert [O.e2m1_value(c | 8) for c in range(8)] == [-0.0, -.5, -1, -1.5, -2, -3, -4, -6]
    assert O.e8m0_value(127) == 1.0 and O.e8m0_value(0) == 2.0 ** -127
    assert np.isnan(O.e8m0_value(255))
