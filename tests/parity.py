"""Comparison of the GPU library's outputs with the CPU oracle's.

Acceptance rules (floating point decided per element; integer and byte results
bit-exact):
  * bf16 outputs (q, the rotary part of the cache, packed Q/K):
        |got - ref| <= 2^-7 |ref| + 1e-3
    and at most ``MAX_MISMATCH`` of the elements may differ in their bits at
    all (``MIN_MISMATCH`` elements are allowed whatever the size) (fp32 kernel
    arithmetic vs double oracle only flips a rounding when the value sits next
    to a bf16 midpoint; a wrong rounding mode would flip ~50%).
  * E4M3 codes: at most one step apart on the signed integer line
    (sign-magnitude, +0 == -0), and at most ``MAX_MISMATCH`` differ
    (``MIN_MISMATCH`` whatever the size).
  * UE8M0 exponent bytes: bit-exact, except in a block whose oracle maximum A
    lies within 2^-18 of an exponent boundary (A / (448 2^e) > 1 - 2^-18 or
    < (1 + 2^-18) / 2): there the two exponents may differ by one and the
    block's codes are checked by dequantised value against the oracle's
    unrounded values instead.  Both sides decide exponents and codes on fp32
    values; the allowance covers the kernel's own fp32 rounding error, which
    can move a maximum that sits within a few fp32 steps of a boundary.
  * Everything the operator must not write: bit-exact (canary bytes, byte 7
    of every scale row, the V section of packed qkv).
"""

from __future__ import annotations

import numpy as np

import oracle as O

MAX_MISMATCH = 1e-3
# The cap is a fraction meant to catch a systematic error (a wrong rounding
# mode flips about half of the values).  Below 1 / MAX_MISMATCH values it would
# refuse a single value whose last bit flipped within the tolerance, so an
# array of any size may hold MIN_MISMATCH differing values.
MIN_MISMATCH = 2
BAND = 2.0 ** -18


def within_cap(n_diff, n):
    """Whether n_diff differing values of n stay under the mismatch cap."""
    return n_diff <= max(MAX_MISMATCH * n, MIN_MISMATCH)

_E4M3 = np.array([O.e4m3_decode(c) for c in range(256)], np.float64)


def bf16_val(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(
        np.float32).astype(np.float64)


def bf16_ordered(bits):
    """bf16 patterns on the signed integer line (sign-magnitude, +0 == -0),
    so that the difference of two is their distance in bf16 steps."""
    b = np.asarray(bits, np.uint16).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_bf16(got, ref, what="", stats=None):
    """Apply the bf16 rule; returns the fraction of values whose bits differ.
    Only the differing values need the tolerance test: an equal pair is
    within it unless it is a NaN, which never is.  With ``stats`` (a dict),
    adds to it the values compared ("n"), the values differing ("diff"), the
    largest distance in bf16 steps where |ref| >= 2^-7, so that the relative
    term governs ("max_steps"), and the largest absolute difference of any
    value ("max_abs"; near zero, where the absolute term governs, a result of
    a cancelling rotation may even differ in sign)."""
    got = np.asarray(got, np.uint16)
    ref = np.asarray(ref, np.uint16)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    gr, rr = got.reshape(-1), ref.reshape(-1)
    nan = (rr & 0x7FFF) > 0x7F80
    if nan.any():
        i = np.flatnonzero(nan)[:5]
        raise AssertionError(f"{what}: NaN in the reference at {i}")
    idx = np.flatnonzero(gr != rr)
    g, r = bf16_val(gr[idx]), bf16_val(rr[idx])
    bad = ~(np.abs(g - r) <= 2.0 ** -7 * np.abs(r) + 1e-3)
    if bad.any():
        i = idx[np.flatnonzero(bad)[:5]]
        raise AssertionError(
            f"{what}: {bad.sum()} bf16 values out of tolerance, e.g. at {i}: "
            f"got {bf16_val(gr[i])} ref {bf16_val(rr[i])}")
    frac = idx.size / gr.size if gr.size else 0.0
    if stats is not None:
        big = np.abs(r) >= 2.0 ** -7
        steps = np.abs(bf16_ordered(gr[idx][big]) - bf16_ordered(rr[idx][big]))
        stats["n"] = stats.get("n", 0) + gr.size
        stats["diff"] = stats.get("diff", 0) + idx.size
        stats["max_steps"] = max(stats.get("max_steps", 0), int(steps.max(initial=0)))
        stats["max_abs"] = max(stats.get("max_abs", 0.0),
                               float(np.abs(g - r).max(initial=0.0)))
    assert within_cap(idx.size, gr.size), (
        f"{what}: {idx.size} of {gr.size} bf16 values ({frac:.2e}) differ in bits")
    return frac


def fp16_val(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def check_fp16(got, ref, what=""):
    """fp16 outputs: |got - ref| <= 2^-10 |ref| + 1e-4 (one fp16 step) and at
    most MAX_MISMATCH of the values differing in their bits."""
    got = np.asarray(got, np.uint16)
    ref = np.asarray(ref, np.uint16)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    g, r = fp16_val(got), fp16_val(ref)
    bad = ~(np.abs(g - r) <= 2.0 ** -10 * np.abs(r) + 1e-4)
    if bad.any():
        i = np.flatnonzero(bad.ravel())[:5]
        raise AssertionError(
            f"{what}: {bad.sum()} fp16 values out of tolerance, e.g. at {i}: "
            f"got {g.ravel()[i]} ref {r.ravel()[i]}")
    n_diff = int(np.count_nonzero(got != ref))
    frac = n_diff / got.size if got.size else 0.0
    assert within_cap(n_diff, got.size), (
        f"{what}: {n_diff} of {got.size} fp16 values ({frac:.2e}) differ in bits")
    return frac


def _signed_code(c):
    c = np.asarray(c, np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def check_cache(got_cache, got_scale, ref_cache, ref_scale, slots, y_ref,
                canary_cache, canary_scale, what=""):
    """Compare the rows of ``slots`` (the valid slots of the tokens whose
    unrounded oracle KV values are ``y_ref[i]``) and return a dict of
    statistics.  Rows outside ``slots`` are not looked at here."""
    gc = got_cache.reshape(-1, 576)
    gs = got_scale.reshape(-1, 8)
    rc = ref_cache.reshape(-1, 576)
    rs = ref_scale.reshape(-1, 8)
    stats = dict(rows=len(slots), code_diff=0, band_blocks=0, rope_frac=0.0)
    if len(slots) == 0:
        return stats
    slots = np.asarray(slots, np.int64)
    g_rows, r_rows = gc[slots], rc[slots]
    g_sc, r_sc = gs[slots], rs[slots]
    assert np.all(g_sc[:, 7] == canary_scale), f"{what}: reserved scale byte written"
    # rotary dims as bf16
    stats["rope_frac"] = check_bf16(
        g_rows[:, 448:].copy().view(np.uint16), r_rows[:, 448:].copy().view(np.uint16),
        what + " rope bf16")
    # exponents
    e_g = g_sc[:, :7].astype(np.int32) - 127
    e_r = r_sc[:, :7].astype(np.int32) - 127
    y = np.asarray(y_ref)[:, :448].reshape(len(slots), 7, 64)
    amax = np.abs(y).max(axis=2)
    rho = amax / (448.0 * np.exp2(e_r.astype(np.float64)))
    in_band = (rho > 1 - BAND) | (rho < 0.5 * (1 + BAND))
    diff_e = e_g != e_r
    bad_e = diff_e & ~(in_band & (np.abs(e_g - e_r) == 1))
    assert not bad_e.any(), (
        f"{what}: {bad_e.sum()} exponent bytes differ outside the boundary band; "
        f"first at {np.argwhere(bad_e)[:3].tolist()}")
    stats["band_blocks"] = int(diff_e.sum())
    # codes
    codes_g = g_rows[:, :448].reshape(len(slots), 7, 64)
    codes_r = r_rows[:, :448].reshape(len(slots), 7, 64)
    same_e = ~diff_e
    d = np.abs(_signed_code(codes_g) - _signed_code(codes_r))
    bad_c = (d > 1) & same_e[:, :, None]
    assert not bad_c.any(), (
        f"{what}: {bad_c.sum()} codes more than one E4M3 step apart; first at "
        f"{np.argwhere(bad_c)[:3].tolist()}")
    n_same = int(same_e.sum()) * 64
    n_diff = int(((d != 0) & same_e[:, :, None]).sum())
    stats["code_diff"] = n_diff
    assert within_cap(n_diff, n_same), f"{what}: {n_diff}/{n_same} codes differ"
    # blocks in the band: dequantised values against the unrounded oracle
    for (i, b) in np.argwhere(diff_e):
        deq = _E4M3[codes_g[i, b]] * 2.0 ** e_g[i, b]
        yy = y[i, b]
        tol = np.maximum(np.abs(yy) * 2.0 ** -4, 2.0 ** (e_g[i, b] - 10)) * 1.05 + 1e-30
        assert np.all(np.abs(deq - yy) <= tol), f"{what}: band block {i},{b}"
    return stats


def check_codes(got, ref, what=""):
    """E4M3 codes without exponents (the scalar-scale convention): at most one
    step apart on the signed line and at most MAX_MISMATCH differing."""
    d = np.abs(_signed_code(got) - _signed_code(ref))
    assert d.max(initial=0) <= 1, f"{what}: codes more than one step apart"
    n_diff = int(np.count_nonzero(d))
    frac = n_diff / d.size if d.size else 0.0
    assert within_cap(n_diff, d.size), f"{what}: {n_diff} of {d.size} codes differ"
    return frac


def check_untouched(got_cache, got_scale, written_slots, canary_cache,
                    canary_scale, what=""):
    gc = got_cache.reshape(-1, 576)
    gs = got_scale.reshape(-1, 8)
    mask = np.ones(gc.shape[0], bool)
    mask[np.asarray(list(written_slots), np.int64)] = False
    assert np.all(gc[mask] == canary_cache), f"{what}: untouched cache row written"
    assert np.all(gs[mask] == canary_scale), f"{what}: untouched scale row written"
    assert np.all(gs[:, 7] == canary_scale), f"{what}: reserved scale byte written"


def valid_slots(slot_mapping, num_slots):
    sm = np.asarray(slot_mapping, np.int64)
    return (sm >= 0) & (sm < num_slots)
