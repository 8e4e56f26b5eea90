"""The GPU parity comparison, exercised on the CPU: the oracle compared with
itself passes, and copies of its output with planted mistakes fail."""

import numpy as np
import pytest
import torch

import oracle as O
from fp8_kv_cache_slot_amd import inputs as I
from tests import parity as P


def _case():
    w = I.custom_dsv4(24, 3, seed=77)
    x = I.make_dsv4(w, "cpu")
    h = {k: (I.bits(v).copy() if isinstance(v, torch.Tensor) else v)
         for k, v in x.items()}
    ref = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in h.items()}
    O.qnorm_rope_kv_quant_insert(ref["q"], ref["kv"], ref["q_weight"],
                                 ref["kv_weight"], ref["cos_sin_cache"],
                                 ref["positions"], ref["slot_mapping"],
                                 ref["kv_cache"], ref["kv_scale"], ref["eps"])
    v = P.valid_slots(h["slot_mapping"], w.num_pages * 64)
    y = O.kv_normalised(h["kv"][v].copy(), h["kv_weight"], h["cos_sin_cache"],
                        h["positions"][v].copy(), h["eps"])
    return h, ref, h["slot_mapping"][v], y


def _check(ref, got_cache, got_scale, slots, y):
    return P.check_cache(got_cache, got_scale, ref["kv_cache"], ref["kv_scale"],
                         slots, y, I.CACHE_CANARY, I.SCALE_CANARY, "t")


def test_oracle_against_itself():
    h, ref, slots, y = _case()
    P.check_bf16(ref["q"], ref["q"])
    st = _check(ref, ref["kv_cache"], ref["kv_scale"], slots, y)
    assert st["code_diff"] == 0 and st["band_blocks"] == 0
    P.check_untouched(ref["kv_cache"], ref["kv_scale"], slots, I.CACHE_CANARY,
                      I.SCALE_CANARY)


def test_one_step_code_difference_is_accepted():
    h, ref, slots, y = _case()
    c = ref["kv_cache"].copy().reshape(-1, 576)
    c[slots[0], 5] = (c[slots[0], 5] & 0x80) | ((c[slots[0], 5] & 0x7F) + 1)
    assert _check(ref, c, ref["kv_scale"], slots, y)["code_diff"] == 1


@pytest.mark.parametrize("mistake", ["code+2", "exponent", "rope", "q", "canary",
                                     "reserved", "many_codes"])
def test_planted_mistakes_fail(mistake):
    h, ref, slots, y = _case()
    c = ref["kv_cache"].copy().reshape(-1, 576)
    s = ref["kv_scale"].copy().reshape(-1, 8)
    q = ref["q"].copy()
    s0 = slots[0]
    if mistake == "code+2":
        c[s0, 7] = (c[s0, 7] & 0x80) | ((c[s0, 7] & 0x7F) + 2)
    elif mistake == "exponent":
        s[s0, 3] += 1
    elif mistake == "rope":
        c[s0, 449] ^= 0x40           # high byte of a rotary bf16
    elif mistake == "q":
        q[0, 0, 10] ^= 0x4000
    elif mistake == "canary":
        free = sorted(set(range(c.shape[0])) - set(slots.tolist()))[0]
        c[free, 0] = 0
    elif mistake == "reserved":
        s[s0, 7] = 0
    elif mistake == "many_codes":
        m = c[slots, :448]
        c[slots, :448] = np.where((m & 0x7F) < 0x7E, m + 1, m)
    with pytest.raises(AssertionError):
        P.check_bf16(q, ref["q"])
        _check(ref, c.reshape(ref["kv_cache"].shape), s.reshape(ref["kv_scale"].shape),
               slots, y)
        P.check_untouched(c, s, slots, I.CACHE_CANARY, I.SCALE_CANARY)


def test_bf16_truncation_is_caught_by_mismatch_rate():
    # a kernel that truncated instead of rounding would stay within the
    # tolerance but flip about half of the values
    h, ref, slots, y = _case()
    val = P.bf16_val(ref["q"])
    lo = (val.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    up = lo + 1
    flip = np.random.default_rng(0).random(lo.shape) < 0.3
    with pytest.raises(AssertionError):
        P.check_bf16(np.where(flip, up, lo), ref["q"])


def test_bf16_rule_statistics_and_nan():
    # 1.0, 2^-10, -1.0, 0, 2.0
    ref = np.array([0x3F80, 0x3A80, 0xBF80, 0x0000, 0x4000] * 400, np.uint16)
    got = ref.copy()
    got[0] = 0x3F81          # one step up at 1.0
    got[6] = 0x3A82          # two steps up at 2^-10, inside the absolute 1e-3
    st = {}
    frac = P.check_bf16(got, ref, "t", stats=st)
    # the step count covers |ref| >= 2^-7 only; the absolute difference all
    assert st == {"n": 2000, "diff": 2, "max_steps": 1, "max_abs": 2.0 ** -7}
    assert frac == 2 / 2000
    st = {}
    small = np.full(2000, 0x3A80, np.uint16)     # 2^-10: the absolute term governs
    off = small.copy()
    off[5] = 0x3A82
    P.check_bf16(off, small, "t", stats=st)
    assert st == {"n": 2000, "diff": 1, "max_steps": 0, "max_abs": 2.0 ** -16}
    assert P.bf16_ordered(np.array([0x8000, 0x0000, 0x8001, 0x0001])).tolist() == [0, 0, -1, 1]
    nan_ref = ref.copy()
    nan_ref[3] = 0x7FC0
    with pytest.raises(AssertionError):
        P.check_bf16(nan_ref, nan_ref, "t")   # equal NaNs are never within tolerance
    nan_got = ref.copy()
    nan_got[3] = 0xFFC0
    with pytest.raises(AssertionError):
        P.check_bf16(nan_got, ref, "t")


def test_mismatch_cap_on_small_arrays():
    # A last-bit flip within the tolerance is what fp32 arithmetic against a
    # double oracle produces near a rounding midpoint: one among 640 values
    # (ten cache rows of rotary dims) passes, as do two; a systematic error on
    # a small array (a third of its values flipped) still fails, and so does a
    # 0.2% rate on a large one.
    rng = np.random.default_rng(5)

    def bf16(v):
        return I.bits(torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)).copy()

    ref = bf16(rng.normal(size=640) + 3.0)
    for flips in (1, 2):
        got = ref.copy()
        got[rng.choice(640, flips, replace=False)] ^= 1
        P.check_bf16(got, ref, "small")
    got = ref.copy()
    got[::3] ^= 1
    with pytest.raises(AssertionError):
        P.check_bf16(got, ref, "small, systematic")
    big = bf16(rng.normal(size=100000) + 3.0)
    got = big.copy()
    got[::500] ^= 1
    with pytest.raises(AssertionError):
        P.check_bf16(got, big, "large, 0.2%")
    codes = rng.integers(0, 0x70, 448).astype(np.uint8)
    g = codes.copy()
    g[[3, 200]] += 1
    P.check_codes(g, codes, "two codes one step apart")
    g[::4] = codes[::4] + 1
    with pytest.raises(AssertionError):
        P.check_codes(g, codes, "a quarter of the codes")
