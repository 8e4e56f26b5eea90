"""Pins of the oracle's scalar-scale cache convention: the hand-derived worked
example (with a saturating block), torch's float8_e4m3fn conversion of
y / s, and q identical to the blockwise operator's."""

import numpy as np
import torch

import oracle as O
from fp8_kv_cache_slot_amd import inputs as I
from tests import golden_case


def test_worked_example_with_scale_2_to_minus_8():
    # normalised values are exactly +-kv_weight (constant rows, eps = 0); with
    # s = 2^-8 the codes are E4M3(w * 256): 1 -> 256 (0x78), 1.5 -> 384
    # (0x7C), 0.5 -> 128 (0x70), 1.75 -> 448 (0x7E), 0.75 -> 192 (0x74),
    # 2^-17 -> 2^-9 (0x01), 2^-7 -> 2 (0x40), and 3 -> 768, which saturates to
    # 448 (0x7E)
    g = golden_case.load()
    x = golden_case.inputs(g)
    exp = golden_case.expected(g)
    q = x["q"].copy()
    cache = x["kv_cache"].copy()
    O.qnorm_rope_kv_quant_insert_scalar(q, x["kv"], x["q_weight"], x["kv_weight"],
                                        x["cos_sin_cache"], x["positions"],
                                        x["slot_mapping"], cache, 2.0 ** -8, x["eps"])
    np.testing.assert_array_equal(q, exp["q"])
    want = np.concatenate([np.full(64, 0x78), np.full(64, 0x7C), np.full(64, 0x70),
                           np.full(64, 0x7E), np.tile([0x78, 0x74], 32),
                           np.full(64, 0x40), np.full(64, 0x7E)]).astype(np.uint8)
    want[64 * 4 + 63] = 0x01
    rows = cache.reshape(-1, 576)
    np.testing.assert_array_equal(rows[5, :448], want)
    np.testing.assert_array_equal(rows[2, :448], want | 0x80)
    # the rotary bytes are the blockwise operator's
    np.testing.assert_array_equal(rows[[5, 2], 448:],
                                  exp["kv_cache"].reshape(-1, 576)[[5, 2], 448:])
    untouched = np.ones(64, bool)
    untouched[[5, 2]] = False
    assert np.all(rows[untouched] == I.CACHE_CANARY)


def test_codes_match_torch_float8_of_y_over_s():
    w = I.custom_dsv4(24, 2, seed=90)
    x = {k: (I.bits(v).copy() if isinstance(v, torch.Tensor) else v)
         for k, v in I.make_dsv4(w, "cpu").items()}
    s = 0.0173
    q = x["q"].copy()
    cache = x["kv_cache"].copy()
    O.qnorm_rope_kv_quant_insert_scalar(q, x["kv"], x["q_weight"], x["kv_weight"],
                                        x["cos_sin_cache"], x["positions"],
                                        x["slot_mapping"], cache, s, x["eps"])
    v = x["slot_mapping"] >= 0
    y = O.kv_normalised(x["kv"][v].copy(), x["kv_weight"], x["cos_sin_cache"],
                        x["positions"][v].copy(), x["eps"])
    # the code is decided in fp32: fp32(y) / fp32(s) in IEEE float32 (numpy),
    # saturated at the E4M3 range and converted by torch's float8_e4m3fn
    scaled = y[:, :448].astype(np.float32) / np.float32(s)
    ref = torch.from_numpy(np.clip(scaled, np.float32(-448), np.float32(448))) \
        .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = cache.reshape(-1, 576)[x["slot_mapping"][v]][:, :448]
    np.testing.assert_array_equal(got, ref)
    # q is the blockwise operator's q
    q2 = x["q"].copy()
    O.qnorm_rope_kv_quant_insert(q2, x["kv"], x["q_weight"], x["kv_weight"],
                                 x["cos_sin_cache"], x["positions"],
                                 x["slot_mapping"], x["kv_cache"].copy(),
                                 x["kv_scale"].copy(), x["eps"])
    np.testing.assert_array_equal(q, q2)


def test_read_side_round_trip_of_the_worked_example():
    # dequantising the scalar-scale rows of the worked example with the same
    # s = 2^-8 returns the weights exactly, except the saturated block, which
    # comes back as 448 * 2^-8 = 1.75
    g = golden_case.load()
    x = golden_case.inputs(g)
    cache = x["kv_cache"].copy()
    O.qnorm_rope_kv_quant_insert_scalar(x["q"].copy(), x["kv"], x["q_weight"],
                                        x["kv_weight"], x["cos_sin_cache"],
                                        x["positions"], x["slot_mapping"], cache,
                                        2.0 ** -8, x["eps"])
    out = O.kv_cache_gather_dequant_scalar(cache, 2.0 ** -8,
                                           np.array([5, -1], np.int64))
    want = x["kv_weight"].copy()
    want[384:448] = O.bf16_rne(1.75)
    np.testing.assert_array_equal(out[0], want)
    assert np.all(out[1] == 0)
