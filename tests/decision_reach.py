"""How often the precision of the quantiser's decisions matters.

The oracle takes the FP8 quantiser's two integer decisions, the UE8M0 block
exponent and the E4M3 code, on each unrounded normalised KV value rounded to
fp32, the precision the operator computes in.  This module counts, over
unrounded rows from the oracle (``oracle.kv_normalised``), the blocks whose
exponent would change if the decisions were taken on the double values
instead, and the codes that would change in the other blocks.  It is a
measurement for the record, not a parity rule; ``tests/fp32_decision_case.py``
gives a hand-derived row where both counts are known.

Decisions (vectorised; the same rules as the oracle states them):
  exponent: smallest e with amax <= 448 * 2^e, amax = 0 -> -127, clamped to
            [-127, 127];
  code:     the E4M3 value nearest to y * 2^-e, ties to even, saturating at
            448 (spacing 2^(floor(log2 |v|) - 3), and 2^-9 below 2^-6).
"""

import numpy as np

BLOCKS, BLOCK = 7, 64


def _exponent(amax):
    m, k = np.frexp(amax)
    e = k - 9 + (m > 0.875)
    e = np.where(amax == 0, -127, e)
    return np.clip(e, -127, 127)


def _e4m3_round(v):
    a = np.abs(v)
    _, k = np.frexp(a)
    lsb = np.maximum(k - 1, -6) - 3
    r = np.rint(np.ldexp(a, -lsb))     # rint: nearest, ties to even
    r = np.minimum(np.ldexp(r, lsb), 448.0)
    return np.copysign(r, v)


def decision_differences(y):
    """y: float64 [n, >=448] unrounded KV rows.  Returns (blocks whose
    exponent differs, codes that differ in blocks whose exponent agrees)
    between deciding on fp32(y) and on y."""
    y = np.asarray(y, np.float64)[:, :BLOCKS * BLOCK].reshape(-1, BLOCKS, BLOCK)
    yf = y.astype(np.float32).astype(np.float64)
    e_d = _exponent(np.abs(y).max(axis=2))
    e_f = _exponent(np.abs(yf).max(axis=2))
    same = e_d == e_f
    s = np.ldexp(1.0, -e_f)[..., None]
    codes = (_e4m3_round(y * s) != _e4m3_round(yf * s)) & same[..., None]
    return int((~same).sum()), int(codes.sum())
