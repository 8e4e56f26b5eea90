"""Pins of the oracle's packed-QKV Q/K RMSNorm + NeoX RoPE against closed
forms, numpy complex multiplication and invariants."""

import numpy as np

import oracle as O
from fp8_kv_cache_slot_amd import inputs as I


def _bf16(x):
    return np.array([O.bf16_rne(float(v)) for v in np.ravel(x)],
                    np.uint16).reshape(np.shape(x))


def _val(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _run(qkv, Hq, Hk, Hv, D, eps, qw, kw, cs, pos):
    out = qkv.copy()
    O.qk_norm_rope_packed(out, Hq, Hk, Hv, D, eps, qw, kw, cs, pos)
    return out


def test_constant_rows_neox_complex_multiplication_and_weights():
    # eps = 0, constant rows: the normalised value is exactly w_d.  Each head
    # must then be bf16((w_i + i w_{i+64}) (c_i + i s_i)) on pairs (i, i+64),
    # with q_weight on Q heads and k_weight on K heads (each element with its
    # own weight, the paired-weight rule); V is untouched.
    rng = np.random.default_rng(20)
    Hq, Hk, Hv, D = 3, 2, 2, 128
    qw = _bf16(rng.uniform(0.5, 1.5, D))
    kw = _bf16(rng.uniform(0.5, 1.5, D))
    cs = rng.uniform(-1, 1, (6, D)).astype(np.float32)
    T = 4
    qkv = np.full((T, (Hq + Hk + Hv) * D), O.bf16_rne(-2.0), np.uint16)
    qkv[:, (Hq + Hk) * D:] = _bf16(rng.standard_normal((T, Hv * D)))
    pos = np.array([5, 0, 2, 2], np.int64)
    out = _run(qkv, Hq, Hk, Hv, D, 0.0, qw, kw, cs, pos)
    np.testing.assert_array_equal(out[:, (Hq + Hk) * D:], qkv[:, (Hq + Hk) * D:])
    for t in range(T):
        c = cs[pos[t], :64].astype(np.float64)
        s = cs[pos[t], 64:].astype(np.float64)
        for h in range(Hq + Hk):
            w = _val(qw if h < Hq else kw)
            z = (-w[:64] - 1j * w[64:]) * (c + 1j * s)
            head = out[t, h * D:(h + 1) * D]
            np.testing.assert_array_equal(head[:64], _bf16(z.real))
            np.testing.assert_array_equal(head[64:], _bf16(z.imag))


def test_identity_rotation_and_norm_preservation():
    # A true cos/sin table with unit weights and eps = 0: rotation keeps each
    # pair's norm, so every head's sum of squares stays 128 (up to the bf16
    # rounding of the outputs); position 0 is the identity.
    w = I.PACKED_WORKLOADS["packed_t17"]
    x = I.make_packed(w, "cpu")
    qkv = I.bits(x["qkv"])
    cs = I.bits(x["cos_sin_cache"])
    pos = I.bits(x["position_ids"]).copy()
    one = np.full(128, O.bf16_rne(1.0), np.uint16)
    out = _run(qkv, 16, 8, 8, 128, 0.0, one, one, cs, pos)
    heads = _val(out[:, :24 * 128]).reshape(17, 24, 128)
    ss = (heads ** 2).sum(-1)
    assert np.all(np.abs(ss - 128) <= 128 * 2 ** -7)
    pos0 = np.zeros_like(pos)
    a = _run(qkv, 16, 8, 8, 128, 0.0, one, one, cs, pos0)
    # with rotation off, output / input is one positive constant per head
    ratio = _val(a[:, :24 * 128]).reshape(17, 24, 128) / \
        _val(qkv[:, :24 * 128]).reshape(17, 24, 128)
    assert np.all(np.abs(ratio / ratio[..., :1] - 1) <= 2 ** -7)


def test_zero_k_heads_and_slices():
    w = I.PACKED_WORKLOADS["packed_t17"]
    x = I.make_packed(w, "cpu")
    qkv = I.bits(x["qkv"])[:, : (16 + 8) * 128].copy()   # Hq=16, Hk=0, Hv=8
    cs = I.bits(x["cos_sin_cache"])
    pos = I.bits(x["position_ids"]).copy()
    qw, kw = I.bits(x["q_weight"]), I.bits(x["k_weight"])
    whole = _run(qkv, 16, 0, 8, 128, 1e-6, qw, kw, cs, pos)
    np.testing.assert_array_equal(whole[:, 16 * 128:], qkv[:, 16 * 128:])
    # per-token independence
    parts = [_run(qkv[s:e].copy(), 16, 0, 8, 128, 1e-6, qw, kw, cs, pos[s:e].copy())
             for s, e in [(0, 1), (1, 9), (9, 17)]]
    np.testing.assert_array_equal(np.concatenate(parts), whole)
    # the K weight is unused when there are no K heads
    other = _run(qkv, 16, 0, 8, 128, 1e-6, qw, qw, cs, pos)
    np.testing.assert_array_equal(other, whole)
