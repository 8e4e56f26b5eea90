"""Pins of the oracle at the bottom of the exponent range against the
hand-derived worked example ``golden/dsv4_low_exponent_rows.json``: the UE8M0
exponent clamped to -127 (from -128, -133, -134 and -141), the unclamped
boundary 448 * 2^-127, fp32-subnormal normalised values, E4M3 codes of
subnormal-scaled values, bf16 subnormal outputs of the rotation, and the read
sides' dequantisation back into the subnormal range."""

import numpy as np

import oracle as O
from tests import golden_low_case as G


def _inputs():
    g = G.load()
    return g, G.inputs(g)


def test_fixture_values_match_their_patterns():
    g = G.load()
    w = G.weight_patterns(g)     # asserts value == pattern for every entry
    assert w.shape == (512,)
    assert G.scalar_scale(g) == np.float32(2.0 ** -126)
    # the derivation's boundary claims, in exact arithmetic
    assert G.parse_value("1.75*2^-119") == 448 * 2.0 ** -127
    assert G.parse_value("1.75*2^-120") == 448 * 2.0 ** -128
    assert G.parse_value("1.7578125*2^-119") > 448 * 2.0 ** -127


def test_normalised_values_are_the_weights():
    # eps = 0 and rows of +-1: y_d = x_d * w_d exactly, down to 2^-133
    g, x = _inputs()
    y = O.kv_normalised(x["kv"], x["kv_weight"], x["cos_sin_cache"],
                        x["positions"], 0.0)
    w = np.array([O.bf16_to_double(b) for b in x["kv_weight"]])
    for t, tok in enumerate(g["tokens"]):
        np.testing.assert_array_equal(y[t, :448], tok["value"] * w[:448])
    assert w[64] == 2.0 ** -133 and w[64] > 0


def test_exponent_rule_at_the_clamp():
    for amax, e in [(2.0 ** -126, -127), (2.0 ** -133, -127),
                    (448 * 2.0 ** -127, -127), (448 * 2.0 ** -128, -127),
                    (1.7578125 * 2.0 ** -119, -126), (0.0, -127),
                    (1.5 * 2.0 ** -125, -127), (2.0 ** -149, -127)]:
        assert O.ue8m0_exponent(amax) == e, amax


def test_blockwise_write_side():
    g, x = _inputs()
    exp = G.expected(g)
    q, cache, scale = x["q"].copy(), x["kv_cache"].copy(), x["kv_scale"].copy()
    O.qnorm_rope_kv_quant_insert(q, x["kv"], x["q_weight"], x["kv_weight"],
                                 x["cos_sin_cache"], x["positions"],
                                 x["slot_mapping"], cache, scale, x["eps"])
    np.testing.assert_array_equal(q, exp["q"])
    np.testing.assert_array_equal(scale, exp["kv_scale"])
    np.testing.assert_array_equal(cache, exp["kv_cache"])


def test_scalar_scale_write_side():
    g, x = _inputs()
    exp = G.expected(g, scalar=True)
    q, cache = x["q"].copy(), x["kv_cache"].copy()
    O.qnorm_rope_kv_quant_insert_scalar(q, x["kv"], x["q_weight"], x["kv_weight"],
                                        x["cos_sin_cache"], x["positions"],
                                        x["slot_mapping"], cache,
                                        float(G.scalar_scale(g)), x["eps"])
    np.testing.assert_array_equal(q, exp["q"])
    np.testing.assert_array_equal(cache, exp["kv_cache"])


def test_read_sides_return_the_subnormal_values():
    g, x = _inputs()
    slots = G.written_slots(g)
    want = G.expected_read(g)
    blk = G.expected(g)
    np.testing.assert_array_equal(
        O.kv_cache_gather_dequant(blk["kv_cache"], blk["kv_scale"], slots), want)
    sc = G.expected(g, scalar=True)
    np.testing.assert_array_equal(
        O.kv_cache_gather_dequant_scalar(sc["kv_cache"], float(G.scalar_scale(g)),
                                         slots), want)
    # through a block table: one sequence of the whole page
    out = np.zeros((64, 512), np.uint16)
    O.kv_cache_gather_dequant_paged(blk["kv_cache"], blk["kv_scale"],
                                    np.zeros((1, 1), np.int32),
                                    np.array([64], np.int32),
                                    np.zeros(1, np.int64), out)
    np.testing.assert_array_equal(out[slots], want)
    out2 = np.zeros((64, 512), np.uint16)
    O.kv_cache_gather_dequant_paged_scalar(sc["kv_cache"], float(G.scalar_scale(g)),
                                           np.zeros((1, 1), np.int32),
                                           np.array([64], np.int32),
                                           np.zeros(1, np.int64), out2)
    np.testing.assert_array_equal(out2[slots], want)
