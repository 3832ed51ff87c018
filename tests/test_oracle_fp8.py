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
