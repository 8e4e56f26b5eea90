"""Pins of the oracle's fused DeepSeek-V4 prologue against closed forms, the
hand-derived worked example, numpy complex multiplication, invariants of
RMSNorm and of the quantiser, and brute force on small inputs."""

import numpy as np
import torch

import oracle as O
from fp8_kv_cache_slot_amd import inputs as I
from tests import golden_case


def _bf16(x):
    return np.array([O.bf16_rne(float(v)) for v in np.ravel(x)],
                    np.uint16).reshape(np.shape(x))


def _val(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _run(x):
    y = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in x.items()}
    O.qnorm_rope_kv_quant_insert(
        y["q"], y["kv"], y["q_weight"], y["kv_weight"], y["cos_sin_cache"],
        y["positions"], y["slot_mapping"], y["kv_cache"], y["kv_scale"],
        y["eps"])
    return y


def _host(w):
    d = I.make_dsv4(w, "cpu")
    return {k: (I.bits(v) if isinstance(v, torch.Tensor) else v)
            for k, v in d.items()}


def _constant_case(T, H, c, eps, positions, cs, q_w, kv_w, slots, pages=1):
    return dict(
        q=np.full((T, H, 512), O.bf16_rne(c), np.uint16),
        kv=np.full((T, 512), O.bf16_rne(c), np.uint16),
        q_weight=q_w, kv_weight=kv_w, cos_sin_cache=cs,
        positions=np.array(positions, np.int64),
        slot_mapping=np.array(slots, np.int64),
        kv_cache=np.full((pages, 64, 576), I.CACHE_CANARY, np.uint8),
        kv_scale=np.full((pages, 64, 8), I.SCALE_CANARY, np.uint8), eps=eps)


def test_golden_worked_example():
    g = golden_case.load()
    out = _run(golden_case.inputs(g))
    exp = golden_case.expected(g)
    np.testing.assert_array_equal(out["q"], exp["q"])
    np.testing.assert_array_equal(out["kv_scale"], exp["kv_scale"])
    np.testing.assert_array_equal(out["kv_cache"], exp["kv_cache"])


def test_rmsnorm_constant_row_closed_form():
    # x = c everywhere: y_d = c / sqrt(c^2 + eps) * w_d.  With c = 0.5 and
    # eps = 0.25 the eps term is half the denominator, so dropping it, moving
    # it outside the root or using a sum instead of a mean all fail.
    rng = np.random.default_rng(10)
    w = _bf16(rng.uniform(0.5, 1.5, 512))
    cs = np.zeros((1, 64), np.float32)
    cs[0, :32] = 1.0
    x = _constant_case(2, 3, 0.5, 0.25, [0, 0], cs, w, w, [0, 1])
    out = _run(x)
    want = _bf16(_val(w) * (0.5 / np.sqrt(0.25 + 0.25)))
    for t in range(2):
        for h in range(3):
            np.testing.assert_array_equal(out["q"][t, h], want)
    # rotary part of the cache is the same bf16 value
    rope = out["kv_cache"][0, 0, 448:].view(np.uint16)
    np.testing.assert_array_equal(rope, want[448:])


def test_rope_equals_complex_multiplication():
    # eps = 0 and a constant row make the normalised value exactly w_d, so
    # the rotary dims must be bf16((w_a + i w_b)(c_i + i s_i)) with pair i on
    # dims (448 + 2i, 449 + 2i), each element with its own weight.  The table
    # row is arbitrary (the operator takes it as input), which exposes any
    # swap of cos/sin, of the pair order or of the index.
    rng = np.random.default_rng(11)
    qw = _bf16(rng.uniform(0.5, 1.5, 512))
    kw = _bf16(rng.uniform(0.5, 1.5, 512))
    cs = rng.uniform(-1, 1, (5, 64)).astype(np.float32)
    pos = [3, 1, 4]
    x = _constant_case(3, 2, 1.0, 0.0, pos, cs, qw, kw, [7, 0, 63])
    out = _run(x)
    for wbits, get in [(qw, lambda t: out["q"][t, 1]),
                       (kw, lambda t: out["kv_cache"][0, [7, 0, 63][t], 448:]
                        .view(np.uint16))]:
        w = _val(wbits)
        for t, p in enumerate(pos):
            z = (w[448::2] + 1j * w[449::2]) * (
                cs[p, :32].astype(np.float64) + 1j * cs[p, 32:].astype(np.float64))
            got = get(t)
            if got.shape[0] == 512:
                np.testing.assert_array_equal(got[:448], _bf16(w[:448]))
                got = got[448:]
            np.testing.assert_array_equal(got[0::2], _bf16(z.real))
            np.testing.assert_array_equal(got[1::2], _bf16(z.imag))


def test_position_zero_identity_and_scale_invariance():
    # Row 0 of a true cos/sin table is (1.., 0..): rotation is the identity, so
    # the output with position 0 on rows whose rotary dims are swapped within
    # each pair is the pair-swapped output.  And RMSNorm with eps = 0 ignores a
    # power-of-two scale of the input exactly.
    w = I.custom_dsv4(4, 3, seed=12)
    x = _host(w)
    x["positions"][:] = 0
    x["eps"] = 0.0
    a = _run(x)
    y = dict(x)
    y["q"] = _bf16(_val(x["q"]) * 8.0)
    y["kv"] = _bf16(_val(x["kv"]) * 8.0)
    b = _run(y)
    for k in ("q", "kv_cache", "kv_scale"):
        np.testing.assert_array_equal(a[k], b[k])
    z = dict(x)
    qs = x["q"].copy()
    qs[..., 448::2], qs[..., 449::2] = x["q"][..., 449::2], x["q"][..., 448::2]
    z["q"] = qs
    z["q_weight"] = x["q_weight"].copy()
    z["q_weight"][448::2], z["q_weight"][449::2] = (x["q_weight"][449::2],
                                                    x["q_weight"][448::2])
    c = _run(z)
    np.testing.assert_array_equal(c["q"][..., 448::2], a["q"][..., 449::2])
    np.testing.assert_array_equal(c["q"][..., :448], a["q"][..., :448])


def test_rmsnorm_uses_all_512_dims():
    # Rotary dims 30x larger than the rest: with eps = 0, w = 1 and position
    # 0, sum of squared outputs is 512 up to bf16 rounding (<= 2^-8 relative
    # per square), whereas a mean over 448 dims would give about 4x that.
    rng = np.random.default_rng(13)
    xv = rng.standard_normal((2, 1, 512))
    xv[..., 448:] *= 30
    one = np.full(512, O.bf16_rne(1.0), np.uint16)
    cs = np.zeros((1, 64), np.float32)
    cs[0, :32] = 1
    x = dict(q=_bf16(xv), kv=_bf16(xv[:, 0]), q_weight=one, kv_weight=one,
             cos_sin_cache=cs, positions=np.zeros(2, np.int64),
             slot_mapping=np.array([0, -1], np.int64),
             kv_cache=np.zeros((1, 64, 576), np.uint8),
             kv_scale=np.zeros((1, 64, 8), np.uint8), eps=0.0)
    out = _run(x)
    ss = (_val(out["q"]) ** 2).sum(axis=-1)
    assert np.all(np.abs(ss - 512) <= 512 * 2 ** -7)
    # and the output direction is the input's: y_d / x_d is one constant
    ratio = _val(out["q"]) / _val(x["q"])
    assert np.all(np.abs(ratio / ratio[..., :1] - 1) <= 2 ** -7)


def test_quantised_block_matches_q_path():
    # Give the KV row the same values and weight as one Q head.  The q output
    # is bf16(y) and the cache holds E4M3(y 2^-e) 2^e; the two must agree to
    # within both roundings, the block's largest dequantised magnitude must sit
    # in [224, 448] 2^e, and the rotary dims in the cache equal the q output.
    w = I.custom_dsv4(16, 1, seed=14)
    x = _host(w)
    x["kv_weight"] = x["q_weight"].copy()
    x["kv"] = x["q"][:, 0].copy()
    x["slot_mapping"] = np.arange(16, dtype=np.int64)
    out = _run(x)
    for t in range(16):
        yq = _val(out["q"][t, 0])
        row = out["kv_cache"].reshape(-1, 576)[t]
        np.testing.assert_array_equal(row[448:].view(np.uint16), out["q"][t, 0, 448:])
        for b in range(7):
            e = int(out["kv_scale"].reshape(-1, 8)[t, b]) - 127
            deq = np.array([O.e4m3_decode(c) for c in row[64 * b:64 * b + 64]]) * 2.0 ** e
            yb = yq[64 * b:64 * b + 64]
            # E4M3 relative step is 2^-3 (half: 2^-4); subnormal step 2^-9 2^e
            bound = np.maximum(np.abs(yb) * 2 ** -4, 2.0 ** (e - 10)) * 1.01 + np.abs(yb) * 2 ** -8
            assert np.all(np.abs(deq - yb) <= bound), (t, b)
            m = np.abs(deq).max()
            assert 224 * 2.0 ** e <= m <= 448 * 2.0 ** e
            assert abs(O.ue8m0_exponent(np.abs(yb).max()) - e) <= 1


def test_scatter_brute_force_and_untouched_bytes():
    # Written rows are exactly {slot_t : 0 <= slot_t < pages*64}, each equal to
    # that token processed alone; every other byte, and byte 7 of every scale
    # row, keeps its canary.  Negative and too-large slots are skipped, while q
    # is still rewritten for those tokens.
    w = I.custom_dsv4(40, 2, seed=15, num_pages=2)
    x = _host(w)
    x["slot_mapping"][3] = -1
    x["slot_mapping"][5] = -7
    x["slot_mapping"][8] = 128          # = pages * 64: out of range
    out = _run(x)
    cache = out["kv_cache"].reshape(-1, 576)
    scale = out["kv_scale"].reshape(-1, 8)
    written = set()
    for t in range(40):
        s = int(x["slot_mapping"][t])
        one = {k: (v[t:t + 1].copy() if isinstance(v, np.ndarray) and k in
                   ("q", "kv", "positions", "slot_mapping") else v)
               for k, v in x.items()}
        one["slot_mapping"] = np.array([0], np.int64)
        one["kv_cache"] = np.full((1, 64, 576), 0, np.uint8)
        one["kv_scale"] = np.full((1, 64, 8), 0, np.uint8)
        single = _run(one)
        np.testing.assert_array_equal(out["q"][t], single["q"][0])
        if 0 <= s < 128:
            written.add(s)
            np.testing.assert_array_equal(cache[s], single["kv_cache"][0, 0])
            np.testing.assert_array_equal(scale[s, :7], single["kv_scale"][0, 0, :7])
    assert written == {int(s) for s in x["slot_mapping"] if 0 <= s < 128}
    for s in range(128):
        assert scale[s, 7] == I.SCALE_CANARY
        if s not in written:
            assert np.all(cache[s] == I.CACHE_CANARY)
            assert np.all(scale[s] == I.SCALE_CANARY)


def test_token_slices_equal_whole():
    w = I.custom_dsv4(37, 3, seed=16)
    x = _host(w)
    whole = _run(x)
    cache, scale = x["kv_cache"].copy(), x["kv_scale"].copy()
    qs = []
    for s, e in [(0, 5), (5, 6), (6, 30), (30, 37)]:
        part = dict(x)
        for k in ("q", "kv", "positions", "slot_mapping"):
            part[k] = x[k][s:e].copy()
        part["kv_cache"], part["kv_scale"] = cache, scale
        O.qnorm_rope_kv_quant_insert(
            part["q"], part["kv"], part["q_weight"], part["kv_weight"],
            part["cos_sin_cache"], part["positions"], part["slot_mapping"],
            cache, scale, part["eps"])
        qs.append(part["q"])
    np.testing.assert_array_equal(np.concatenate(qs), whole["q"])
    np.testing.assert_array_equal(cache, whole["kv_cache"])
    np.testing.assert_array_equal(scale, whole["kv_scale"])


def test_zero_input():
    one = np.full(512, O.bf16_rne(1.0), np.uint16)
    cs = I.cos_sin_cache(8, 64).numpy()
    x = dict(q=np.zeros((2, 2, 512), np.uint16), kv=np.zeros((2, 512), np.uint16),
             q_weight=one, kv_weight=one, cos_sin_cache=cs,
             positions=np.array([0, 5], np.int64),
             slot_mapping=np.array([1, 0], np.int64),
             kv_cache=np.full((1, 64, 576), 0xA5, np.uint8),
             kv_scale=np.full((1, 64, 8), 0xEE, np.uint8), eps=1e-6)
    out = _run(x)
    # rotation of a zero pair may give a signed zero; values must be zero
    assert np.all(_val(out["q"]) == 0)
    assert np.all(out["kv_cache"][0, :2, :448] == 0)
    assert np.all(_val(out["kv_cache"][0, :2, 448:].copy().view(np.uint16)) == 0)
    assert np.all(out["kv_scale"][0, :2, :7] == 0)        # e = -127
    assert np.all(out["kv_scale"][0, :2, 7] == 0xEE)


def test_cos_sin_generator_row_zero():
    cs = I.cos_sin_cache(16, 64).numpy()
    assert np.all(cs[0, :32] == 1.0) and np.all(cs[0, 32:] == 0.0)
    np.testing.assert_allclose(cs[:, :32] ** 2 + cs[:, 32:] ** 2, 1.0, atol=1e-6)


def test_kv_normalised_is_the_unrounded_kv_row():
    # The unrounded KV values the bound checks compare against: rounding them
    # as the operator does must give the fused oracle's stored bytes exactly
    # (bf16 rotary dims; the exponent of each block's maximum and the E4M3
    # codes of y 2^-e, both taken on the fp32 values of y), and with a
    # constant row and eps = 0 the non-rotary dims are exactly kv_weight.
    x = _host(I.custom_dsv4(12, 3, seed=77))
    y = O.kv_normalised(x["kv"].copy(), x["kv_weight"], x["cos_sin_cache"],
                        x["positions"], x["eps"])
    out = _run(x)
    rows = out["kv_cache"].reshape(-1, 576)
    scales = out["kv_scale"].reshape(-1, 8)
    for t, s in enumerate(x["slot_mapping"]):
        if not 0 <= s < rows.shape[0]:
            continue
        rot = _bf16(y[t, 448:])
        np.testing.assert_array_equal(rows[s, 448:].view(np.uint16), rot)
        for b in range(7):
            blk = y[t, 64 * b:64 * b + 64].astype(np.float32).astype(np.float64)
            e = O.ue8m0_exponent(float(np.abs(blk).max()))
            assert scales[s, b] == e + 127
            codes = [O.e4m3_encode(float(v) * 2.0 ** -e) for v in blk]
            np.testing.assert_array_equal(rows[s, 64 * b:64 * b + 64], codes)
    rng = np.random.default_rng(78)
    kw = _bf16(rng.uniform(0.5, 1.5, 512))
    kv = np.full((2, 512), O.bf16_rne(0.75), np.uint16)
    cs = rng.uniform(-1, 1, (4, 64)).astype(np.float32)
    yc = O.kv_normalised(kv, kw, cs, np.array([3, 1], np.int64), 0.0)
    np.testing.assert_array_equal(yc[:, :448], np.broadcast_to(_val(kw[:448]), (2, 448)))
    # with a large eps the closed form c / sqrt(c^2 + eps) * w (eps inside the
    # root, mean over all 512 dims) separates a dropped or misplaced eps
    for eps in (0.25, 4.0):
        ye = O.kv_normalised(kv, kw, cs, np.array([3, 1], np.int64), eps)
        want = 0.75 / np.sqrt(0.75 ** 2 + eps) * _val(kw[:448])
        np.testing.assert_allclose(ye[:, :448], np.broadcast_to(want, (2, 448)),
                                   rtol=1e-14, atol=0)
