"""Pins of the oracle's FP8 cache functions (CPU only).

fp8_e4m3_value is pinned to the format's definition by hand-worked bytes and to torch's own
float8_e4m3fn conversion over all 256 bytes (an independent library routine); the
dequantisation to a value-for-value bf16 cache by hand-worked rows, and the generator's FP8
cache by its round trip back to the bf16 values it was drawn from."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W


# byte -> value from the E4M3 definition: sign, 4-bit exponent (bias 7), 3-bit mantissa,
# subnormals m/8 * 2^-6, S.1111.111 NaN
HAND = {
    0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
    0x38: 1.0, 0x39: 1.125, 0x3C: 1.5, 0x40: 2.0, 0x77: 1.875 * 2.0 ** 7, 0x78: 256.0,
    0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9),
}


def test_fp8_hand_values():
    for code, want in HAND.items():
        assert oracle.fp8_e4m3_value(code) == want, hex(code)
    assert math.copysign(1.0, float(oracle.fp8_e4m3_value(0x80))) == -1.0  # negative zero
    assert np.isnan(oracle.fp8_e4m3_value(0x7F)) and np.isnan(oracle.fp8_e4m3_value(0xFF))
    # 0x7F/0xFF are the only NaNs: there is no infinity
    v = oracle.fp8_e4m3_value(np.arange(256))
    assert set(np.flatnonzero(np.isnan(v)).tolist()) == {0x7F, 0xFF}
    assert np.all(np.isfinite(v[~np.isnan(v)]))


def test_fp8_matches_torch_all_bytes():
    codes = np.arange(256)
    v = oracle.fp8_e4m3_value(codes)
    t = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(v), np.isnan(t))
    assert np.array_equal(v[~np.isnan(v)], t[~np.isnan(t)])


def test_fp8_monotone_positive_half():
    # the positive finite codes 0x00..0x7E are increasing (a plausible exponent or mantissa
    # slip breaks this)
    v = oracle.fp8_e4m3_value(np.arange(0x7F))
    assert np.all(np.diff(v) > 0)


def test_dequant_hand_rows():
    d_c, d_R = 4, 2
    kv8 = np.zeros((1, 64, d_c + 2 * d_R), dtype=np.uint8)
    kv8[0, 0, :d_c] = [0x38, 0xB8, 0x01, 0x7E]     # 1, -1, 2^-9, 448
    kv8[0, 0, d_c:] = [0x80, 0x3F, 0x00, 0xC0]     # k_R bf16 1.0, -2.0 (little endian)
    scales = np.ones((1, 64), dtype=np.float32)
    scales[0, 0] = 0.25
    out = oracle.dequant_fp8_cache(kv8, scales, d_c)
    assert out.shape == (1, 64, d_c + d_R)
    assert out[0, 0].tolist() == [0x3E80, 0xBE80, 0x3A00, 0x42E0, 0x3F80, 0xC000]
    assert np.all(out[0, 1:] == 0)
    # a scale outside the contract is refused, not reinterpreted
    for bad in (0.3, 1.99, 0.0, -0.25, 3.0):
        scales[0, 0] = bad
        with pytest.raises(ValueError):
            oracle.dequant_fp8_cache(kv8, scales, d_c)


def test_scale_contract():
    # positive normal powers of two (2^-126 .. 2^127) and NaN (unused slots) are accepted
    good = np.array([1.0, 0.25, 2.0 ** -126, 2.0 ** 127, 2.0 ** -20, np.nan])
    got = oracle.check_scales(good)
    assert got[:-1].tolist() == good[:-1].tolist() and np.isnan(got[-1])
    # anything else is refused: mantissa bits, zero, negative, subnormal, infinity
    for bad in (0.3, 1.5, 3.0, 2.0 ** 20 * 1.7, 0.0, -1.0, -2.0, 2.0 ** -127, 2.0 ** -140,
                np.inf):
        with pytest.raises(ValueError):
            oracle.check_scales(np.array([1.0, bad]))


def test_fp8_cache_round_trip():
    # the generator's FP8 cache dequantises back to the drawn c_KV rounded to 4 significant
    # bits (RNE), within the e4m3 relative step, with k_R untouched
    inp = W.make_inputs(3, 2, 8, 64, 8, 16, [5, 64, 70], seed=11)
    kv8, sc = W.fp8_cache(inp, seed=3)
    deq = oracle.dequant_fp8_cache(kv8.numpy(), sc.numpy(), 64)
    ref = W.u16(inp["kv_pages"])
    assert np.array_equal(deq[:, :, 64:], ref[:, :, 64:])
    a, b = oracle._f64(deq[:, :, :64]), oracle._f64(ref[:, :, :64])
    scale = sc.numpy().astype(np.float64)[:, :, None]
    # |error| <= half a step of the code: 2^-4 relative for normals, 2^-10 * scale absolute
    assert np.all(np.abs(a - b) <= np.maximum(np.abs(b) * 2.0 ** -4, 2.0 ** -10 * scale))
    assert np.mean(a == b) < 1.0  # quantisation really happened


# ---- the FP8 writer (quantise_fp8_row): round to nearest even E4M3 under a power-of-two
# scale chosen from the row's largest magnitude

def test_encode_round_trips_every_finite_code():
    v = oracle.fp8_e4m3_value(np.arange(256))
    fin = ~np.isnan(v)
    codes = np.arange(256)[fin]
    enc = oracle.fp8_e4m3_encode(v[fin]).astype(np.int64)
    # -0 (0x80) encodes as +0; every other finite code comes back as itself
    assert np.all((enc == codes) | ((codes == 0x80) & (enc == 0)))


def test_encode_rounds_to_nearest_ties_to_even():
    vals = oracle.fp8_e4m3_value(np.arange(127))
    mid = (vals[:-1] + vals[1:]) / 2
    e = oracle.fp8_e4m3_encode(mid).astype(np.int64)
    assert np.all(e % 2 == 0)                           # a tie takes the even code
    assert np.all((e == np.arange(126)) | (e == np.arange(1, 127)))
    gap = vals[1:] - vals[:-1]
    below = oracle.fp8_e4m3_encode(mid - gap / 8).astype(np.int64)
    above = oracle.fp8_e4m3_encode(mid + gap / 8).astype(np.int64)
    assert np.array_equal(below, np.arange(126)) and np.array_equal(above, np.arange(1, 127))
    neg = oracle.fp8_e4m3_encode(-vals[1:]).astype(np.int64)
    assert np.array_equal(neg, np.arange(1, 127) | 0x80)
    with pytest.raises(ValueError):
        oracle.fp8_e4m3_encode(np.array([448.5]))


def test_scale_exponent_is_the_smallest_that_fits():
    for e in (-20, -8, 0, 3, 40):
        edge = 448.0 * 2.0 ** e
        assert oracle.fp8_scale_exponent(edge) == e
        assert oracle.fp8_scale_exponent(edge * (1 + 2.0 ** -40)) == e + 1
        assert oracle.fp8_scale_exponent(edge / 2 * (1 + 2.0 ** -40)) == e
        assert oracle.fp8_scale_exponent(edge / 2) == e - 1
    assert oracle.fp8_scale_exponent(0.0) == 0
    assert oracle.fp8_scale_exponent(1e-300) == -126 and oracle.fp8_scale_exponent(1e300) == 127


def test_quantised_row_error_bound():
    rng = np.random.default_rng(7)
    for scale in (1e-3, 1.0, 50.0):
        c = rng.standard_normal(512) * scale
        codes, s = oracle.quantise_fp8_row(c)
        assert s == 2.0 ** np.round(np.log2(s))          # a power of two
        amax = np.max(np.abs(c))
        assert 224 * s < amax <= 448 * s                  # the smallest that fits
        back = oracle.fp8_e4m3_value(codes) * s
        normal = np.abs(c) >= 2.0 ** -6 * s
        # half an E4M3 ulp: 2^-4 relative for normals, 2^-10 * s for subnormals
        assert np.all(np.abs(back - c)[normal] <= 2.0 ** -4 * np.abs(c)[normal])
        assert np.all(np.abs(back - c)[~normal] <= 2.0 ** -10 * s)
    codes, s = oracle.quantise_fp8_row(np.zeros(64))
    assert s == 1.0 and np.all(codes == 0)



def test_encode_agrees_with_torch_float8_cast():
    # torch's float32 -> float8_e4m3fn cast rounds to nearest even as well; on fp32 values
    # within the format's range (normals, subnormals, ties) both give the same byte
    import torch
    rng = np.random.default_rng(11)
    mags = np.concatenate([rng.uniform(0, 448, 4000), rng.uniform(0, 2.0 ** -6, 2000),
                           oracle.fp8_e4m3_value(np.arange(127))])
    v = (mags * rng.choice([-1.0, 1.0], mags.size)).astype(np.float32)
    vals = oracle.fp8_e4m3_value(np.arange(127))
    ties = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)     # exact in fp32
    v = np.concatenate([v, ties, -ties])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.fp8_e4m3_encode(v.astype(np.float64))
    # torch keeps the sign of a value that rounds to zero (0x80); the encoder writes 0x00
    same = (got == ref) | ((got == 0) & (ref == 0x80))
    assert np.all(same), v[~same][:5]
