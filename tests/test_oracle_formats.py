"""Pins of the oracle's number formats against things other than itself:
numpy's binary32 bit layout, torch's float8_e4m3fn and bfloat16 conversions
(library routines), brute-force searches and the error bounds of
round-to-nearest."""

import math

import numpy as np
import torch

import oracle as O


def _torch_bf16_bits(v32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(v32.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_decode_all_patterns():
    # Every bf16 pattern is the top half of a binary32 pattern.
    for b in range(0, 1 << 16, 7):
        f32 = np.array([b << 16], np.uint32).view(np.float32)[0]
        got = O.bf16_to_double(b)
        if math.isnan(f32):
            assert math.isnan(got)
        else:
            assert got == float(f32) and math.copysign(1, got) == math.copysign(1, f32)


def test_bf16_rne_matches_torch_on_binary32_values():
    rng = np.random.default_rng(1)
    raw = rng.integers(0, 1 << 32, 20000, dtype=np.uint64).astype(np.uint32)
    # exact ties (low half 0x8000) of both parities, plus small subnormals
    ties = (rng.integers(0, 1 << 16, 2000).astype(np.uint32) << 16) | 0x8000
    pats = np.concatenate([raw, ties, np.arange(1, 300, dtype=np.uint32)])
    vals = pats.view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) < 3e38)]
    want = _torch_bf16_bits(vals)
    got = np.array([O.bf16_rne(float(v)) for v in vals], np.uint16)
    np.testing.assert_array_equal(got, want)


def test_bf16_rne_is_nearest_for_doubles():
    # Doubles off the binary32 grid: the result must be a nearest bf16 value
    # and, on an exact tie, the even one.
    rng = np.random.default_rng(2)
    vals = rng.standard_normal(5000) * np.exp2(rng.integers(-30, 30, 5000))
    n_truncation_would_fail = 0
    for v in vals:
        b = O.bf16_rne(v)
        r = O.bf16_to_double(b)
        lo = O.bf16_to_double(b - 1) if (b & 0x7FFF) else -r
        hi = O.bf16_to_double(b + 1)
        assert abs(v - r) <= abs(v - lo) and abs(v - r) <= abs(v - hi)
        trunc = O.bf16_to_double(
            int(np.array([v], np.float64).astype(np.float32).view(np.uint32)[0] >> 16))
        n_truncation_would_fail += abs(v - trunc) > abs(v - r)
    assert n_truncation_would_fail > 100  # the check has teeth


def test_e4m3_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = O.e4m3_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c], c
    assert O.e4m3_decode(0x7E) == 448.0 and O.e4m3_decode(0x01) == 2.0 ** -9


def test_e4m3_encode_roundtrip_all_finite_codes():
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert O.e4m3_encode(O.e4m3_decode(c)) == c, hex(c)


def test_e4m3_encode_midpoints_round_to_even():
    for c in range(0, 0x7E):
        a, b = O.e4m3_decode(c), O.e4m3_decode(c + 1)
        mid = (a + b) / 2
        even = c if c % 2 == 0 else c + 1
        assert O.e4m3_encode(mid) == even, hex(c)
        assert O.e4m3_encode(math.nextafter(mid, 0)) == c
        assert O.e4m3_encode(math.nextafter(mid, 1e9)) == c + 1
        assert O.e4m3_encode(-mid) == 0x80 | even


def test_e4m3_encode_matches_torch_on_random_values():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-12, 9, 20000)))
    v = v.astype(np.float32)
    v = v[np.abs(v) < 464]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.e4m3_encode(float(x)) for x in v], np.uint8)
    np.testing.assert_array_equal(got, ref)


def test_e4m3_encode_saturates_and_keeps_sign():
    assert O.e4m3_encode(448.0) == 0x7E
    assert O.e4m3_encode(463.9) == 0x7E
    assert O.e4m3_encode(1e9) == 0x7E
    assert O.e4m3_encode(-1e9) == 0xFE
    assert O.e4m3_encode(-1e-30) == 0x80
    assert O.e4m3_encode(0.0) == 0x00


def _brute_exponent(a):
    for e in range(-127, 128):
        if a <= 448.0 * 2.0 ** e:
            return e
    return 127


def test_ue8m0_exponent_brute_force():
    rng = np.random.default_rng(4)
    vals = list(np.exp2(rng.uniform(-140, 40, 4000)))
    for k in range(-135, 30):
        edge = 448.0 * 2.0 ** k
        vals += [edge, math.nextafter(edge, 0), math.nextafter(edge, 1e300),
                 224.0 * 2.0 ** k, math.nextafter(224.0 * 2.0 ** k, 1e300)]
    for a in vals:
        assert O.ue8m0_exponent(a) == _brute_exponent(a), a
    assert O.ue8m0_exponent(0.0) == -127
    assert O.ue8m0_exponent(1e-300) == -127    # clamped
    assert O.ue8m0_exponent(1e300) == 127      # clamped


def test_ue8m0_exponent_brackets_amax():
    # For an unclamped exponent, 224 * 2^e < amax <= 448 * 2^e, so the block's
    # largest scaled magnitude lands in (224, 448].
    rng = np.random.default_rng(5)
    for a in np.exp2(rng.uniform(-100, 20, 2000)):
        e = O.ue8m0_exponent(a)
        assert 224.0 * 2.0 ** e < a <= 448.0 * 2.0 ** e
