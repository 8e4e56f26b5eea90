"""Pins of the oracle's separate stages of the packed Q/K operator (RmsNorm of
a group of heads into its own output, then NeoX RoPE of it in place), the
launches InfiniOps PR #1019 "Benchmark / Performance Impact" compares the
fused call with: a closed form, equality with the fused packed oracle where
the rotation is the identity, numpy complex multiplication, and agreement of
the composed stages with the fused oracle up to the extra bf16 rounding
between them."""

import numpy as np
import torch

import oracle as O
from fp8_kv_cache_slot_amd import inputs as I

HQ, HK, HV, D = 16, 8, 8, 128


def _bf16(x):
    return np.array([O.bf16_rne(float(v)) for v in np.ravel(x)],
                    np.uint16).reshape(np.shape(x))


def _val(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _packed(T, seed, hq=HQ, hk=HK, hv=HV):
    x = I.make_packed(I.PackedWorkload("p", T, hq, hk, hv, seed=seed), "cpu")
    return {k: (I.bits(v).copy() if isinstance(v, torch.Tensor) else v)
            for k, v in x.items()}


def test_rms_norm_heads_closed_form():
    rng = np.random.default_rng(60)
    w = _bf16(rng.uniform(0.5, 1.5, D))
    x = np.full((3, (HQ + HK + HV) * D), O.bf16_rne(0.5), np.uint16)
    out = O.rms_norm_heads(x, HQ, HK, D, w, 0.25)
    want = _bf16(_val(w) * (0.5 / np.sqrt(0.25 + 0.25)))
    assert out.shape == (3, HK, D)
    for t in range(3):
        for h in range(HK):
            np.testing.assert_array_equal(out[t, h], want)


def test_rms_norm_heads_equals_fused_without_rotation():
    # position 0 rotates by the identity, so the fused packed output of each
    # Q and K head is exactly its normalised head; the stage reads heads out
    # of the packed row at the right offset, with the right weight
    x = _packed(7, seed=61)
    x["position_ids"][:] = 0
    fused = x["qkv"].copy()
    O.qk_norm_rope_packed(fused, HQ, HK, HV, D, x["eps"], x["q_weight"],
                          x["k_weight"], x["cos_sin_cache"], x["position_ids"])
    q = O.rms_norm_heads(x["qkv"], 0, HQ, D, x["q_weight"], x["eps"])
    k = O.rms_norm_heads(x["qkv"], HQ, HK, D, x["k_weight"], x["eps"])
    np.testing.assert_array_equal(q.reshape(7, -1), fused[:, :HQ * D])
    np.testing.assert_array_equal(k.reshape(7, -1), fused[:, HQ * D:(HQ + HK) * D])


def test_rope_neox_heads_complex_multiplication():
    rng = np.random.default_rng(62)
    T, H = 5, 3
    x = _bf16(rng.standard_normal((T, H, D)) * 3)
    cs = rng.uniform(-1, 1, (9, D)).astype(np.float32)
    pos = rng.integers(0, 9, T).astype(np.int64)
    out = x.copy()
    O.rope_neox_heads(out, cs, pos)
    v = _val(x)
    for t in range(T):
        z = (v[t, :, :D // 2] + 1j * v[t, :, D // 2:]) * (
            cs[pos[t], :D // 2].astype(np.float64)
            + 1j * cs[pos[t], D // 2:].astype(np.float64))
        np.testing.assert_array_equal(out[t, :, :D // 2], _bf16(z.real))
        np.testing.assert_array_equal(out[t, :, D // 2:], _bf16(z.imag))


def test_stages_compose_to_the_fused_operator():
    # norm -> rope equals the fused packed oracle up to the one extra bf16
    # rounding of both pair inputs between the stages
    T = 40
    x = _packed(T, seed=63)
    fused = x["qkv"].copy()
    O.qk_norm_rope_packed(fused, HQ, HK, HV, D, x["eps"], x["q_weight"],
                          x["k_weight"], x["cos_sin_cache"], x["position_ids"])
    q = O.rms_norm_heads(x["qkv"], 0, HQ, D, x["q_weight"], x["eps"])
    k = O.rms_norm_heads(x["qkv"], HQ, HK, D, x["k_weight"], x["eps"])
    O.rope_neox_heads(q, x["cos_sin_cache"], x["position_ids"])
    O.rope_neox_heads(k, x["cos_sin_cache"], x["position_ids"])
    got = np.concatenate([q.reshape(T, -1), k.reshape(T, -1)], axis=1)
    ref = fused[:, :(HQ + HK) * D]
    g = _val(got).reshape(T, HQ + HK, D)
    f = _val(ref).reshape(T, HQ + HK, D)
    a, b = f[..., :D // 2], f[..., D // 2:]
    norm = np.concatenate([np.sqrt(a * a + b * b)] * 2, axis=-1)
    assert np.all(np.abs(g - f) <= norm * 2.0 ** -7)
    assert np.mean(got != ref) < 0.5   # mostly the same bits
    assert np.mean(got != ref) > 0.0   # but the extra rounding shows
