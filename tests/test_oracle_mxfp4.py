"""Pins of the oracle's MXFP4 cache functions (OCP Microscaling v1.0: FP4 E2M1 elements in
blocks of 32 sharing an E8M0 power-of-two scale), against the format's own definition: its
value table, an exact-rational brute force of round-to-nearest-even with saturation, torch's
E8M0 decoding, closed forms of the shared exponent, and the error bound of a quantised row."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

# E2M1 magnitudes as the format lists them (codes 0..7): subnormal 0 and 0.5, then 1, 1.5,
# 2, 3, 4, 6 (exponents 0..2 with one mantissa bit)
TABLE = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
         Fraction(4), Fraction(6)]


def test_e2m1_values_match_the_format_table():
    v = oracle.fp4_e2m1_value(np.arange(16))
    for c in range(8):
        assert v[c] == float(TABLE[c])
        assert v[c + 8] == -float(TABLE[c])  # bit 3 is the sign
    assert np.signbit(v[8])                  # code 8 is -0


def _nearest_even(x):
    """Brute force over the table with exact rationals: the nearest magnitude to
    min(|x|, 6), ties to the even code; sign in bit 3 unless the magnitude code is 0."""
    a = min(abs(Fraction(x)), TABLE[7])
    best = None
    for c, t in enumerate(TABLE):
        d = abs(a - t)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    c = best[1]
    return c | (8 if x < 0 and c != 0 else 0)


def test_encode_is_round_to_nearest_even_by_brute_force():
    grid = [k / 64 for k in range(-8 * 64, 8 * 64 + 1)]
    rng = np.random.default_rng(3)
    rand = list(rng.uniform(-9, 9, 2000)) + list(rng.standard_normal(500) * 0.3)
    xs = np.array(grid + rand)
    got = oracle.fp4_e2m1_encode(xs)
    want = np.array([_nearest_even(float(x)) for x in xs], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_encode_midpoints_and_saturation():
    # each midpoint between neighbours goes to the even code (mantissa bit 0)
    mids = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for x, c in mids.items():
        assert oracle.fp4_e2m1_encode(x) == c, x
        assert oracle.fp4_e2m1_encode(-x) == (c | 8 if c else 0), -x
    for x in (6.0, 6.5, 7.999, 1e6):
        assert oracle.fp4_e2m1_encode(x) == 7 and oracle.fp4_e2m1_encode(-x) == 15
    assert oracle.fp4_e2m1_encode(-0.2) == 0  # rounds to zero: stored as +0
    with pytest.raises(ValueError):
        oracle.fp4_e2m1_encode(np.nan)


def test_encode_round_trips_every_value():
    codes = np.array([c for c in range(16) if c != 8])
    assert np.array_equal(oracle.fp4_e2m1_encode(oracle.fp4_e2m1_value(codes)), codes)


def test_e8m0_matches_torch():
    codes = np.arange(255, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(oracle.e8m0_value(codes), want)
    assert np.isnan(oracle.e8m0_value(255))


def test_shared_exponent_closed_forms():
    # X puts the block maximum in [4, 8) * 2^X: its top element lands on 4 or 6 (or clips)
    for k in range(-20, 21):
        for m in (1.0, 1.25, 1.5, 1.999):
            amax = m * 2.0 ** k
            X = oracle.mx_scale_exponent(amax)
            assert X == k - 2 and 4.0 <= amax / 2.0 ** X < 8.0, (amax, X)
    assert oracle.mx_scale_exponent(0.0) == 0
    assert oracle.mx_scale_exponent(2.0 ** -140) == -127   # E8M0's smallest scale
    assert oracle.mx_scale_exponent(1.5 * 2.0 ** 127) == 125
    assert oracle.mx_scale_exponent(2.0 ** 200) == 127


def test_quantised_row_error_bound():
    rng = np.random.default_rng(5)
    for trial in range(50):
        c = rng.standard_normal(512) * np.exp2(rng.integers(-10, 10))
        codes, sc = oracle.quantise_mxfp4_row(c)
        assert codes.shape == (512,) and sc.shape == (16,)
        v = oracle.fp4_e2m1_value(codes) * np.repeat(oracle.e8m0_value(sc), 32)
        for k in range(16):
            blk, q = c[32 * k:32 * k + 32], v[32 * k:32 * k + 32]
            s = 2.0 ** (int(sc[k]) - 127)
            a = np.abs(blk) / s
            # inside E2M1's range the error is at most half the spacing at that magnitude
            # (0.25 below 2, 0.5 in [2, 4), 1 in [4, 6]); above 6 the value saturates
            half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0)) * s
            inside = a <= 6
            assert np.all(np.abs(q - blk)[inside] <= half[inside])
            assert np.all(np.abs(q)[~inside] == 6 * s)
            assert 4 <= np.max(a) < 8


def test_pack_nibble_order_and_round_trip():
    assert oracle.pack_fp4([0x1, 0x2])[0] == 0x21  # element 0 in the low nibble
    rng = np.random.default_rng(7)
    c = rng.integers(0, 16, (3, 64)).astype(np.uint8)
    assert np.array_equal(oracle.unpack_fp4(oracle.pack_fp4(c)), c)


def test_dequant_cache_values_and_nan_scale():
    rng = np.random.default_rng(11)
    P, d_c, d_R = 2, 64, 8
    codes = rng.integers(0, 16, (P, 64, d_c)).astype(np.uint8)
    kr = rng.integers(0, 1 << 15, (P, 64, d_R)).astype(np.uint16)
    kv4 = np.concatenate([oracle.pack_fp4(codes), kr.view(np.uint8).reshape(P, 64, 2 * d_R)],
                         axis=2)
    sc = rng.integers(120, 135, (P, 64, d_c // 32)).astype(np.uint8)
    sc[1, 5, 1] = 255  # a NaN scale: its block reads NaN, nothing else does
    out = oracle.dequant_mxfp4_cache(kv4, sc, d_c)
    vals = (out[:, :, :d_c].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for p in range(P):
        for t in range(64):
            for c in range(d_c):
                s = sc[p, t, c // 32]
                want = float(TABLE[codes[p, t, c] & 7]) * (-1 if codes[p, t, c] & 8 else 1)
                if s == 255:
                    assert np.isnan(vals[p, t, c])
                else:
                    assert vals[p, t, c] == want * 2.0 ** (int(s) - 127)
    assert np.isnan(vals).sum() == 32
    assert np.array_equal(out[:, :, d_c:], kr)
