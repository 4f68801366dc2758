"""Pins of the FP8 (OCP E4M3) oracle: codes and values against torch's float8_e4m3fn (an
independent implementation of the same format), closed forms of the format, the
power-of-two scale identity, the round-trip error bound and the append."""

import numpy as np
import pytest
import torch

from oracle import fp8

ALL = np.arange(256, dtype=np.uint8)


def torch_values(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_codes(x32):
    return torch.from_numpy(np.asarray(x32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def check_decode_matches_torch():
    got, want = fp8.e4m3_decode(ALL), torch_values(ALL)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def check_encode_matches_torch():
    # every fp16 value in range, and every midpoint between neighbouring codes (ties)
    h = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float32)
    h = h[np.isfinite(h) & (np.abs(h) <= 448)]
    pos = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[1:] + pos[:-1]) / 2)  # exact in fp32
    rng = np.random.default_rng(0)
    rnd = (rng.standard_normal(200000) * np.exp2(rng.integers(-12, 9, 200000))).astype(np.float32)
    rnd = rnd[np.abs(rnd) <= 448]
    for x in (h, mids, -mids, rnd):
        assert np.array_equal(fp8.e4m3_encode(x), torch_codes(x))


def check_closed_forms():
    enc = lambda v: int(fp8.e4m3_encode(np.float32(v)))
    assert enc(1.0) == 0x38 and enc(-1.0) == 0xB8
    assert enc(448.0) == 0x7E and enc(-448.0) == 0xFE
    assert enc(449.0) == 0x7E and enc(1e6) == 0x7E and enc(np.inf) == 0x7E and enc(-1e30) == 0xFE
    assert enc(np.nan) & 0x7F == 0x7F
    assert enc(2.0 ** -9) == 0x01 and enc(2.0 ** -10) == 0x00 and enc(3 * 2.0 ** -10) == 0x02
    assert enc(2.0 ** -6) == 0x08  # smallest normal
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    assert fp8.e4m3_decode(0x7E) == 448.0 and fp8.e4m3_decode(0x01) == 2.0 ** -9
    assert np.isnan(fp8.e4m3_decode(0x7F)) and np.isnan(fp8.e4m3_decode(0xFF))


def check_scaled_quantize():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(50000).astype(np.float16)
    for k in (-3, 0, 2):  # power-of-two scales are exact: quantize(x, 2^k) = encode(x / 2^k)
        s = 2.0 ** k
        assert np.array_equal(fp8.quantize(x, s), fp8.e4m3_encode(x.astype(np.float32) / np.float32(s)))
    s = 0.037
    q = fp8.quantize(x, s)
    back = fp8.e4m3_decode(q) * np.float32(s)
    xs = x.astype(np.float64)
    normal = np.abs(xs) / s >= 2.0 ** -6
    # round to nearest with 3 mantissa bits: relative error at most 2^-4 (plus the fp32 product)
    assert np.all(np.abs(back[normal] - xs[normal]) <= (2.0 ** -4 + 2.0 ** -20) * np.abs(xs[normal]))
    assert np.all(np.abs(back[~normal] - xs[~normal]) <= 2.0 ** -10 * s * 1.0001)


def check_append():
    rng = np.random.default_rng(2)
    pool = np.full((6, 16, 2, 2, 8), 0x7F, np.uint8)
    key = rng.standard_normal((5, 2, 8)).astype(np.float16)
    val = rng.standard_normal((5, 2, 8)).astype(np.float16)
    slots = np.array([3, 17, -1, 95, 40])
    got = fp8.kv_append_fp8(pool, key, val, slots, 0.5, 0.25)
    want = pool.copy()
    keep = slots >= 0
    s = slots[keep]
    want[s // 16, s % 16, 0] = fp8.quantize(key[keep], 0.5)
    want[s // 16, s % 16, 1] = fp8.quantize(val[keep], 0.25)
    assert np.array_equal(got, want)


def test_decode_matches_torch():
    check_decode_matches_torch()


def test_encode_matches_torch():
    check_encode_matches_torch()


def test_closed_forms():
    check_closed_forms()


def test_scaled_quantize():
    check_scaled_quantize()


def test_append():
    check_append()


def test_dequantized_pool_is_code_times_scale():
    rng = np.random.default_rng(3)
    pool = rng.integers(0, 256, (3, 16, 2, 2, 8)).astype(np.uint8)
    d = fp8.dequantize_pool(pool, 0.5, 3.0)
    assert np.array_equal(d[:, :, 0], fp8.e4m3_decode(pool[:, :, 0]) * 0.5, equal_nan=True)
    assert np.array_equal(d[:, :, 1], fp8.e4m3_decode(pool[:, :, 1]) * 3.0, equal_nan=True)


# planted mistakes: each must fail a pin

def test_pins_catch_ties_away_from_zero(monkeypatch):
    def enc(x):
        x = np.asarray(x, np.float32).astype(np.float64)
        a = np.minimum(np.abs(x), 448.0)
        pos = fp8._POS
        i = np.clip(np.searchsorted(pos, a), 1, 0x7E)
        code = np.where(a - pos[i - 1] < pos[i] - a, i - 1, i)  # ties upward
        return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)
    monkeypatch.setattr(fp8, "e4m3_encode", enc)
    with pytest.raises(AssertionError):
        check_encode_matches_torch()


def test_pins_catch_bias_eight(monkeypatch):
    orig = fp8.e4m3_decode
    monkeypatch.setattr(fp8, "e4m3_decode", lambda c: orig(c) / 2.0)  # the fnuz exponent bias
    with pytest.raises(AssertionError):
        check_decode_matches_torch()


def test_pins_catch_no_saturation(monkeypatch):
    orig = fp8.e4m3_encode
    monkeypatch.setattr(fp8, "e4m3_encode",
                        lambda x: np.where(np.abs(np.asarray(x, np.float32)) > 448, 0x7F, orig(x)).astype(np.uint8))
    with pytest.raises(AssertionError):
        check_closed_forms()


def test_pins_catch_scale_multiplied(monkeypatch):
    monkeypatch.setattr(fp8, "quantize", lambda x, s: fp8.e4m3_encode(np.asarray(x, np.float32) * np.float32(s)))
    with pytest.raises(AssertionError):
        check_scaled_quantize()
