"""Pins for the read-copy oracle (CPU only): the E4M3 format's defining values (OCP
8-bit floating point specification: largest finite 448, smallest normal 2**-6,
smallest subnormal 2**-9, no infinities), round to nearest with ties to even, and
the error bounds of every copy."""

import numpy as np

from oracle import readcopy as rc


def test_e4m3_defining_values():
    assert rc.e4m3_value(0x7E) == 448.0
    assert rc.e4m3_value(0x08) == 2.0 ** -6
    assert rc.e4m3_value(0x01) == 2.0 ** -9
    assert rc.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert rc.e4m3_value(0x38) == 1.0
    assert rc.e4m3_value(0x3C) == 1.5
    assert rc.e4m3_value(0xB8) == -1.0
    assert np.isnan(rc.e4m3_value(0x7F)) and np.isnan(rc.e4m3_value(0xFF))
    assert rc.e4m3_value(0x00) == 0.0 and np.signbit(rc.e4m3_value(0x80))
    pos = np.array([rc.e4m3_value(c) for c in range(0x7F)])
    assert pos.size == 127 and np.all(np.diff(pos) > 0)


def test_e4m3_round_trip_and_ties_to_even():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = rc.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(rc.e4m3_encode(vals), codes)
    cases = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02,
             0.0146484375: 0x08, 1.0625 + 2.0 ** -20: 0x39, 500.0: 0x7E, -460.0: 0xFE, -0.0: 0x80,
             240.0: 0x77, 232.0: 0x76}
    for v, c in cases.items():
        assert int(rc.e4m3_encode(np.float32(v))) == c, v


def test_e4m3_matches_exponent_mantissa_rounding():
    # independent form: scale |x| to the binade's grid (3 mantissa bits, subnormal step
    # 2**-9), round half to even with numpy, saturate at 448
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-12, 7, 20000))).astype(np.float32)
    a = np.abs(x.astype(np.float64))
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
    step = np.ldexp(1.0, (e - 3).astype(int))
    ref = np.minimum(np.round(a / step) * step, 448.0) * np.where(np.signbit(x), -1.0, 1.0)
    got = rc.e4m3_decode(rc.e4m3_encode(x))
    assert np.array_equal(got, ref)


def test_fp8_copy_rows():
    rng = np.random.default_rng(4)
    h = (0.1 * rng.standard_normal((3, 8, 32))).astype(np.float32)
    h[1, 2] = 0.0
    h[2, 5, :] *= np.float32(1e-4)
    h[2, 5, 7] = np.float32(3.0)          # one large entry: the rest go subnormal
    codes, scale = rc.fp8_copy(h)
    assert scale[1, 2] == 0 and not codes[1, 2].any()
    amax = np.max(np.abs(h), axis=-1)
    np.testing.assert_array_equal(scale, (amax / np.float32(448)).astype(np.float32))
    # the largest element of a row takes code 448 (up to the last bit of the product)
    idx = np.argmax(np.abs(h), axis=-1)
    top = np.take_along_axis(codes, idx[..., None], -1)[..., 0] & 0x7F
    assert np.all((top == 0x7E) | (scale == 0))
    err = np.abs(rc.fp8_values(codes, scale) - h)
    bound = rc.copy_error_bound(h, "fp8", scale) * (1 + 1e-6)
    assert np.all(err <= bound)
    assert np.max(err / np.where(bound > 0, bound, 1)) > 0.5       # the bound is not slack


def test_bf16_and_f16_copies():
    assert rc.f16_copy(np.float32(1 + 2.0 ** -11)) == 1.0
    assert rc.f16_copy(np.float32(1 + 3 * 2.0 ** -11)) == 1 + 2.0 ** -9
    assert rc.bf16_copy(np.array([1 + 2.0 ** -8], np.float32))[0] == 1.0
    assert rc.bf16_copy(np.array([1 + 3 * 2.0 ** -8], np.float32))[0] == 1 + 2.0 ** -6
    rng = np.random.default_rng(5)
    h = (0.1 * rng.standard_normal(50000) * np.exp(rng.uniform(-10, 3, 50000))).astype(np.float32)
    for kind, fn in (("bf16", rc.bf16_copy), ("f16", rc.f16_copy)):
        err = np.abs(fn(h) - h)
        bound = rc.copy_error_bound(h, kind)
        assert np.all(err <= bound) and np.max(err / bound) > 0.5, kind



def test_e4m3_matches_torch_cast():
    # independent pin: torch's CPU cast to float8_e4m3fn rounds to nearest, ties to even;
    # it turns values past the largest finite into NaN instead of saturating, so the
    # inputs stay within +-448
    import pytest
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(40000) * np.exp(rng.uniform(-14, 6, 40000))).astype(np.float32)
    x = np.concatenate([x[np.abs(x) <= 448], np.float32([0.0, -0.0, 448.0, -448.0, 2.0 ** -10])])
    lib8 = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(rc.e4m3_encode(x), lib8)


def test_bf16_and_f16_copies_match_bitwise_rounding():
    # independent forms: bf16 keeps the upper 16 bits of the fp32 word after adding
    # 0x7FFF plus the kept part's lowest bit (round to nearest, ties to even); fp16 rounds
    # |x| to its binade's grid (10 mantissa bits, subnormal step 2**-24) half to even
    rng = np.random.default_rng(7)
    y = (rng.standard_normal(40000) * np.exp(rng.uniform(-20, 20, 40000))).astype(np.float32)
    y = np.concatenate([y, np.float32([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -0.0, 2.0 ** -130])])
    u = y.view(np.uint32).astype(np.uint64)
    bf = (((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)).view(np.float32)
    assert np.array_equal(np.asarray(rc.bf16_copy(y), np.float32), bf)
    z = y[np.abs(y) < 65504].astype(np.float64)
    e = np.maximum(np.floor(np.log2(np.where(z != 0, np.abs(z), 1.0))), -14)
    step = np.ldexp(1.0, (e - 10).astype(int))
    f16 = np.round(z / step) * step
    assert np.array_equal(np.asarray(rc.f16_copy(z.astype(np.float32)), np.float64), f16)
