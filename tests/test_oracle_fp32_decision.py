"""Pins of the oracle's quantiser decisions: the UE8M0 block exponent and the
E4M3 codes are taken on fp32 values, the precision the operator computes in.
The expected bytes are derived by hand in tests/fp32_decision_case.py; a
decision taken in double gives different exponent and code bytes there."""

import numpy as np

import oracle as O
from tests import fp32_decision_case as C


def test_the_case_straddles_a_boundary_in_double_only():
    x = C.inputs()
    y = O.kv_normalised(x["kv"], x["kv_weight"], x["cos_sin_cache"],
                        x["positions"], C.EPS)[0]
    # double: just above 1.75 = 448 * 2^-8 and 1.8125; fp32: exactly on them
    assert y[0] > 1.75 and y[64] > 1.8125
    assert np.float32(y[0]) == 1.75 and np.float32(y[64]) == 1.8125
    assert O.ue8m0_exponent(float(y[0])) == -7        # the double decision
    assert O.ue8m0_exponent(float(np.float32(y[0]))) == -8


def test_blockwise_bytes_decided_in_fp32():
    x = C.inputs()
    q, cache, scale = x["q"].copy(), x["kv_cache"].copy(), x["kv_scale"].copy()
    O.qnorm_rope_kv_quant_insert(q, x["kv"], x["q_weight"], x["kv_weight"],
                                 x["cos_sin_cache"], x["positions"],
                                 x["slot_mapping"], cache, scale, C.EPS)
    row, sc = cache.reshape(-1, 576)[5], scale.reshape(-1, 8)[5]
    assert list(sc[:7]) == C.SCALE_BYTES
    assert list(sc[:7]) != C.DOUBLE_SCALE_BYTES
    assert sc[7] == 0x5A
    assert list(row[:448]) == C.CODES
    assert np.all(row[448:].view(np.uint16) == C.ROPE_BF16)
    others = np.delete(cache.reshape(-1, 576), 5, axis=0)
    assert np.all(others == 0xA5)
    # q: bf16(1 + 2^-28) = 1.0, bf16(0.5 (1 + 2^-28)) = 0.5
    assert np.all(q[0, 0, :448] == 0x3F80) and np.all(q[0, 0, 448:] == 0x3F00)


def test_scalar_scale_code_decided_in_fp32():
    x = C.inputs()
    cache = x["kv_cache"].copy()
    O.qnorm_rope_kv_quant_insert_scalar(x["q"].copy(), x["kv"], x["q_weight"],
                                        x["kv_weight"], x["cos_sin_cache"],
                                        x["positions"], x["slot_mapping"], cache,
                                        1.0, C.EPS)
    row = cache.reshape(-1, 576)[5]
    assert list(row[:448]) == C.SCALAR_CODES
    assert np.all(row[448:].view(np.uint16) == C.ROPE_BF16)


def test_decision_reach_counts_the_hand_derived_case():
    # The counting helper used for the full-size record: in this row the
    # exponent of block 0 and all 64 codes of block 1 depend on the precision
    # of the decision; nothing else does.  A row of exact fp32 values changes
    # nothing.
    from tests import decision_reach as R

    x = C.inputs()
    y = O.kv_normalised(x["kv"], x["kv_weight"], x["cos_sin_cache"],
                        x["positions"], C.EPS)
    assert R.decision_differences(y) == (1, 64)
    assert R.decision_differences(np.float32(y).astype(np.float64)) == (0, 0)
    # its rounding agrees with the oracle's encoder on every E4M3 midpoint and
    # its neighbours
    vals = np.array([O.e4m3_decode(c) for c in range(0x7F)])
    mids = (vals[1:] + vals[:-1]) / 2
    probe = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9)])
    want = np.array([O.e4m3_decode(O.e4m3_encode(v)) for v in probe])
    np.testing.assert_array_equal(R._e4m3_round(probe), want)
    amax = np.array([0.0, 2.0 ** -140, 448 * 2.0 ** -8, np.nextafter(448 * 2.0 ** -8, 1)])
    assert R._exponent(amax).tolist() == [O.ue8m0_exponent(a) for a in amax]
