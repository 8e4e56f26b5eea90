"""Pins of the oracle's fp16 codec (numpy float16 as the library reference)
and of the general packed operator: agreement with the guarded form, and
constant-row closed forms for interleaved / NeoX, partial rotary, head widths
64/128/256 and fp16 (normalised value exactly w, rotation = complex
multiplication of the pair)."""

import numpy as np
import pytest

import oracle as O


def test_fp16_decode_all_patterns():
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    for b in range(0, 1 << 16, 3):
        got = O.fp16_to_double(b)
        if np.isnan(ref[b]):
            assert np.isnan(got)
        else:
            assert got == ref[b], b


def test_fp16_rne_matches_numpy():
    rng = np.random.default_rng(80)
    vals = list(rng.standard_normal(6000) * np.exp2(rng.integers(-28, 17, 6000)))
    # exact ties between neighbours, in the normal and subnormal ranges
    for b in rng.integers(1, 0x7BFF, 1500):
        lo, hi = O.fp16_to_double(int(b)), O.fp16_to_double(int(b) + 1)
        vals += [(lo + hi) / 2, -(lo + hi) / 2]
    vals += [65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -25, 2.0 ** -26, 0.0]
    for v in vals:
        assert O.fp16_rne(v) == int(np.array([v]).astype(np.float16).view(np.uint16)[0]), v


def _bf16(x):
    return np.array([O.bf16_rne(float(v)) for v in np.ravel(x)],
                    np.uint16).reshape(np.shape(x))


def _fp16(x):
    return np.array([O.fp16_rne(float(v)) for v in np.ravel(x)],
                    np.uint16).reshape(np.shape(x))


def test_general_form_equals_guarded_form():
    rng = np.random.default_rng(81)
    T, hq, hk, hv, D = 9, 4, 2, 3, 128
    qkv = _bf16(rng.standard_normal((T, (hq + hk + hv) * D)))
    qw, kw = _bf16(rng.uniform(0.5, 1.5, D)), _bf16(rng.uniform(0.5, 1.5, D))
    cs = rng.uniform(-1, 1, (20, D)).astype(np.float32)
    pos = rng.integers(0, 20, T).astype(np.int64)
    a, b = qkv.copy(), qkv.copy()
    O.qk_norm_rope_packed(a, hq, hk, hv, D, 1e-6, qw, kw, cs, pos)
    O.qk_norm_rope_packed_ex(b, hq, hk, hv, D, D, 1, 0, 1e-6, qw, kw, cs, pos)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("D,R,neox,fp16", [
    (128, 128, 0, 0), (128, 64, 1, 0), (128, 64, 0, 0), (64, 64, 1, 0),
    (64, 32, 0, 0), (256, 256, 1, 0), (256, 128, 1, 0), (128, 128, 1, 1),
    (128, 32, 0, 1), (256, 64, 0, 1), (128, 0, 1, 0)])
def test_constant_rows_closed_form(D, R, neox, fp16):
    # eps = 0 and constant rows make the normalised value exactly w_d; the
    # rotation is then the complex product of each pair with (c_i + i s_i),
    # rounded once; dims >= R keep bf16/fp16(w_d)
    rng = np.random.default_rng(82 + D + R)
    enc, dec = (_fp16, O.fp16_to_double) if fp16 else (_bf16, O.bf16_to_double)
    hq, hk, hv, T = 2, 1, 1, 3
    qw, kw = enc(rng.uniform(0.5, 1.5, D)), enc(rng.uniform(0.5, 1.5, D))
    cs = rng.uniform(-1, 1, (7, max(R, 2))).astype(np.float32)[:, :R].copy()
    pos = np.array([6, 0, 3], np.int64)
    one = O.fp16_rne(1.0) if fp16 else O.bf16_rne(1.0)
    qkv = np.full((T, (hq + hk + hv) * D), one, np.uint16)
    qkv[:, (hq + hk) * D:] = enc(rng.standard_normal((T, hv * D)))
    out = qkv.copy()
    O.qk_norm_rope_packed_ex(out, hq, hk, hv, D, R, neox, fp16, 0.0, qw, kw,
                             cs if R else np.zeros((7, 0), np.float32), pos)
    np.testing.assert_array_equal(out[:, (hq + hk) * D:], qkv[:, (hq + hk) * D:])
    half = R // 2
    for t in range(T):
        for h in range(hq + hk):
            w = np.array([dec(int(v)) for v in (qw if h < hq else kw)])
            head = out[t, h * D:(h + 1) * D]
            np.testing.assert_array_equal(head[R:], enc(w[R:]))
            if R == 0:
                continue
            c = cs[pos[t], :half].astype(np.float64)
            s = cs[pos[t], half:].astype(np.float64)
            if neox:
                z = (w[:half] + 1j * w[half:R]) * (c + 1j * s)
                np.testing.assert_array_equal(head[:half], enc(z.real))
                np.testing.assert_array_equal(head[half:R], enc(z.imag))
            else:
                z = (w[0:R:2] + 1j * w[1:R:2]) * (c + 1j * s)
                np.testing.assert_array_equal(head[0:R:2], enc(z.real))
                np.testing.assert_array_equal(head[1:R:2], enc(z.imag))
