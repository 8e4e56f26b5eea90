"""Pins of the oracle's cache read side (gather + dequantise) against the
hand-derived worked example, torch's float8_e4m3fn decoding, and the
quantisation error bound of a round trip through the fused prologue."""

import numpy as np
import torch

import oracle as O
from fp8_kv_cache_slot_amd import inputs as I
from tests import golden_case


def _val(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def test_golden_round_trip_returns_the_weights():
    # In the worked example the normalised KV values are exactly +-kv_weight
    # and every one of them is representable as E4M3 * 2^e, so dequantising
    # the written rows gives the weights back bit for bit (negated for the
    # token whose row was -1), and the rotary part is the stored bf16.
    g = golden_case.load()
    x = golden_case.inputs(g)
    O.qnorm_rope_kv_quant_insert(x["q"], x["kv"], x["q_weight"], x["kv_weight"],
                                 x["cos_sin_cache"], x["positions"],
                                 x["slot_mapping"], x["kv_cache"], x["kv_scale"],
                                 x["eps"])
    out = O.kv_cache_gather_dequant(x["kv_cache"], x["kv_scale"],
                                    np.array([5, 2, -1, 64], np.int64))
    np.testing.assert_array_equal(out[0], x["kv_weight"])
    np.testing.assert_array_equal(out[1, :448], x["kv_weight"][:448] | 0x8000)
    e = g["expected"]["rope_bf16_token1"]
    assert np.all(out[1, 448::2] == e["even"]) and np.all(out[1, 449::2] == e["odd"])
    assert np.all(out[2] == 0) and np.all(out[3] == 0)


def test_dequant_matches_torch_float8_decode():
    rng = np.random.default_rng(30)
    pages = 2
    cache = rng.integers(0, 256, (pages, 64, 576), dtype=np.uint8)
    cache[..., :448][(cache[..., :448] & 0x7F) == 0x7F] = 0x7E   # no NaN codes
    scale = rng.integers(127 - 30, 127 + 10, (pages, 64, 8), dtype=np.uint8)
    slots = rng.permutation(pages * 64)[:50].astype(np.int64)
    out = O.kv_cache_gather_dequant(cache, scale, slots)
    rows = cache.reshape(-1, 576)[slots]
    codes = torch.from_numpy(rows[:, :448].copy()).view(torch.float8_e4m3fn)
    dec = codes.to(torch.float64).numpy()
    e = scale.reshape(-1, 8)[slots][:, :7].astype(np.float64) - 127
    want = dec * np.exp2(np.repeat(e, 64, axis=1))
    np.testing.assert_array_equal(_val(out[:, :448]), want)   # exact in bf16
    np.testing.assert_array_equal(out[:, 448:], rows[:, 448:].copy().view(np.uint16))


def test_round_trip_error_bound():
    # dequantise(quantise(y)) is within half an E4M3 step of the unrounded y
    # (relative 2^-4 for normal codes, 2^(e-10) absolute in the subnormal
    # range), and the rotary part within half a bf16 step.
    w = I.custom_dsv4(40, 2, seed=31)
    x = {k: (I.bits(v).copy() if isinstance(v, torch.Tensor) else v)
         for k, v in I.make_dsv4(w, "cpu").items()}
    O.qnorm_rope_kv_quant_insert(x["q"], x["kv"], x["q_weight"], x["kv_weight"],
                                 x["cos_sin_cache"], x["positions"],
                                 x["slot_mapping"], x["kv_cache"], x["kv_scale"],
                                 x["eps"])
    v = x["slot_mapping"] >= 0
    y = O.kv_normalised(x["kv"][v].copy(), x["kv_weight"], x["cos_sin_cache"],
                        x["positions"][v].copy(), x["eps"])
    out = _val(O.kv_cache_gather_dequant(x["kv_cache"], x["kv_scale"],
                                         x["slot_mapping"][v]))
    e = x["kv_scale"].reshape(-1, 8)[x["slot_mapping"][v]][:, :7].astype(np.float64) - 127
    e = np.repeat(e, 64, axis=1)
    yq = y[:, :448]
    bound = np.maximum(np.abs(yq) * 2.0 ** -4, np.exp2(e - 10))
    assert np.all(np.abs(out[:, :448] - yq) <= bound * (1 + 1e-12))
    yr = y[:, 448:]
    assert np.all(np.abs(out[:, 448:] - yr) <= np.abs(yr) * 2.0 ** -8 + 1e-300)
