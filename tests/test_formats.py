"""Pins for the oracle's number formats (CPU).

Each check compares ``oracle.formats`` with something it does not share code
with: a nearest-value search over all candidates, the OCP E4M3 code table,
exact rational arithmetic, or the math library's exp.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import exact
from oracle import formats as fm

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16

def _bf16_nearest(x32):
    """Nearest bf16 by comparing the two truncation neighbours in float64; ties to even."""
    u = x32.view(np.uint32)
    lo = (u >> 16).astype(np.uint32)
    hi = lo + 1
    vlo = (lo << 16).view(np.float32).astype(np.float64)
    vhi = (hi << 16).view(np.float32).astype(np.float64)
    x = x32.astype(np.float64)
    dlo = np.abs(x - vlo)
    dhi = np.abs(vhi - x)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (lo % 2 == 1))
    return np.where(pick_hi, hi, lo).astype(np.uint16)


def test_bf16_all_upper_patterns():
    hi = np.arange(1 << 16, dtype=np.uint32)
    for low in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234):
        u = (hi << 16) | low
        x = u.view(np.float32)
        ok = np.isfinite(x) & (np.abs(x) < 3.3e38)
        got = fm.bf16_bits(x[ok])
        want = _bf16_nearest(x[ok])
        assert np.array_equal(got, want), hex(low)


def test_bf16_specials():
    x = np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, 3.4028235e38], dtype=np.float32)
    b = fm.bf16_bits(x)
    assert b[0] == 0x7F80 and b[1] == 0xFF80
    assert np.isnan(fm.bf16_to_f32(b[2:3]))[0]
    assert b[3] == 0x0000 and b[4] == 0x8000
    assert b[5] == 0x7F80            # rounds up past the largest bf16 to infinity


def test_bf16_worked_value():
    g = json.load(open(os.path.join(GOLD, "bf16_boundary_worked_example.json")))
    assert fm.bf16_bits(np.array([g["q"]], np.float32))[0] == int(g["expected_bf16_bits_of_1_001"], 16)


# ---------------------------------------------------------------- E4M3FN

def test_e4m3_golden_codes():
    g = json.load(open(os.path.join(GOLD, "e4m3fn_codes.json")))
    for c, v in g["codes"].items():
        got = fm.e4m3_decode(np.array([int(c, 16)]))[0]
        assert got == v and np.signbit(got) == np.signbit(v), c
    for c in g["nan_codes"]:
        assert np.isnan(fm.e4m3_decode(np.array([int(c, 16)]))[0])


def test_e4m3_decode_table_structure():
    v = fm.e4m3_decode(np.arange(256))
    fin = np.isfinite(v)
    assert fin.sum() == 254
    pos = v[:128][fin[:128]]
    assert np.all(np.diff(pos) > 0)          # codes 0..126 increase strictly
    assert pos.max() == 448.0
    assert np.array_equal(v[128:][fin[128:]], -v[:128][fin[:128]])


def test_e4m3_encode_roundtrip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(fm.e4m3_encode(fm.e4m3_decode(codes)), codes.astype(np.uint8))


def _e4m3_nearest(x):
    codes = np.array([c for c in range(128) if c != 0x7F])
    vals = fm.e4m3_decode(codes)
    out = []
    for xv in x:
        d = np.abs(vals - abs(xv))
        best = np.flatnonzero(d == d.min())
        c = codes[best[0]] if best.size == 1 else [cc for cc in codes[best] if cc % 2 == 0][0]
        out.append(c | (0x80 if np.signbit(xv) else 0))
    return np.array(out, dtype=np.uint8)


def test_e4m3_encode_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.uniform(-448, 448, 3000),
        rng.uniform(-0.02, 0.02, 2000),                      # subnormal range
        np.exp2(rng.uniform(-12, 8.8, 2000)) * rng.choice([-1, 1], 2000),
    ]).astype(np.float32).astype(np.float64)
    # exact midpoints between neighbouring codes
    vals = fm.e4m3_decode(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([x, mids, -mids])
    assert np.array_equal(fm.e4m3_encode(x), _e4m3_nearest(x))


def test_e4m3_rejects_saturation():
    with pytest.raises(ValueError):
        fm.e4m3_encode(np.array([449.0]))


# ---------------------------------------------------------------- UE8M0

def _smallest_e(amax):
    if amax == 0:
        return 0
    e = -200
    while not (Fraction(amax) <= 448 * Fraction(2) ** e):
        e += 1
    return max(-127, min(127, e))


def test_ue8m0_rule_brute_force():
    rng = np.random.default_rng(1)
    a = np.concatenate([
        np.exp2(rng.uniform(-30, 30, 3000)),
        448.0 * np.exp2(rng.integers(-20, 20, 200)),            # exactly on the boundary
        np.nextafter(448.0 * np.exp2(rng.integers(-20, 20, 200)), np.inf),
        [0.0, 1e-45, 3.0e38],
    ]).astype(np.float32).astype(np.float64)
    got = fm.ue8m0_exponent(a)
    want = np.array([_smallest_e(v) for v in a])
    assert np.array_equal(got, want)


def test_fp8_quantize_never_saturates_and_is_close():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((50, 128)) * np.exp2(rng.uniform(-20, 20, (50, 1)))).astype(np.float32)
    for block in (128, 32):
        codes, sc = fm.quantize_fp8_blocks(x, block)
        assert not np.any(np.isnan(fm.e4m3_decode(codes)))
        deq = fm.dequantize_fp8_blocks(codes, sc, block)
        xb = x.astype(np.float64).reshape(50, -1, block)
        amax = np.abs(xb).max(-1, keepdims=True)
        # payload error is at most half a quantum: 2^-4 relative in the normal range,
        # and the block scale puts amax in (224, 448]
        err = np.abs(deq.reshape(xb.shape) - xb)
        assert np.all(err <= np.maximum(np.abs(xb) * 2.0 ** -4, amax / 448 * 2.0 ** -10) + 0)


# ---------------------------------------------------------------- fma32

def test_fma32_matches_exact_rational():
    rng = np.random.default_rng(3)
    n = 3000
    a = (rng.standard_normal(n) * np.exp2(rng.integers(-10, 10, n))).astype(np.float32)
    b = (rng.standard_normal(n) * np.exp2(rng.integers(-10, 10, n))).astype(np.float32)
    c = (rng.standard_normal(n) * np.exp2(rng.integers(-10, 10, n))).astype(np.float32)
    got = fm.fma32(a, b, c)
    want = np.array([exact.fma32_exact(x, y, z) for x, y, z in zip(a, b, c)], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_fma32_double_rounding_cases():
    # a*b + c lies within 2^-70 of an fp32 midpoint whose even neighbour is on the
    # wrong side: rounding to float64 first lands exactly on the midpoint, and a
    # second, independent rounding to fp32 would pick the even (wrong) neighbour.
    a = np.float32(2.0 ** -12 * (1 + 2.0 ** -23))
    b = np.float32(2.0 ** -12 * (1 - 2.0 ** -23))
    c = np.float32(1 + 2.0 ** -23)
    want = np.float32(1 + 2.0 ** -23)
    for bb in (b, -b):           # exact sums 1 + 3*2^-24 - 2^-70 and 1 + 2^-24 + 2^-70
        got = fm.fma32(np.array([a]), np.array([bb]), np.array([c]))[0]
        assert got == want == np.float32(exact.fma32_exact(a, bb, c))
        naive = np.float32(np.float64(a) * np.float64(bb) + np.float64(c))
        assert naive != want


# ---------------------------------------------------------------- pinned exp

def test_pexp_constants():
    assert fm.LOG2E_F32 == np.float32(1 / math.log(2))
    assert abs(float(fm.LN2_HI_F32) + float(fm.LN2_LO_F32) - math.log(2)) < 6e-14
    assert np.float32(fm.LN2_HI_F32).view(np.uint32) & 0x1FF == 0     # n*ln2_hi exact for |n| < 2^9
    for k in range(8):
        assert fm.EXP_POLY_F32[k] == np.float32(1 / math.factorial(k))


def test_pexp_accuracy_and_specials():
    z = np.concatenate([-np.exp2(np.linspace(-30, 6.7, 20000)), [0.0, -0.0, -103.9, -104.0, -104.5, -1e30]]).astype(np.float32)
    p = fm.pexp(z)
    assert p[-6] == 1.0 and p[-5] == 1.0
    assert p[-2] == 0.0 and p[-1] == 0.0
    ref = np.array([math.exp(float(v)) for v in z])
    normal = ref > 1.2e-38
    ulp = np.spacing(np.abs(ref[normal]).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(p[normal] - ref[normal]) <= 2 * ulp)
    # subnormal results: within one subnormal quantum
    assert np.all(np.abs(p[~normal] - ref[~normal]) <= 2.0 ** -149 * 2)
    order = np.argsort(z)
    assert np.all(np.diff(p[order].astype(np.float64)) >= 0)
