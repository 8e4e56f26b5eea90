"""Builds the inputs and expected outputs of the hand-derived worked example at
the bottom of the exponent range, ``golden/dsv4_low_exponent_rows.json``
(constant rows of +-1, eps = 0, weights at and below 2^-126).  Test helper
only: every number comes from the fixture, never from either implementation.
Each weight is stated both as a value ("1.75*2^-119") and as a bf16 pattern;
``weight_patterns`` checks that the two agree."""

import json
import os

import numpy as np

from fp8_kv_cache_slot_amd import inputs as I

HERE = os.path.dirname(os.path.abspath(__file__))
PATH = os.path.join(HERE, "golden", "dsv4_low_exponent_rows.json")


def load():
    with open(PATH) as f:
        return json.load(f)


def parse_value(text):
    """'0', '2^-126' or 'm*2^k' -> float (exact)."""
    text = text.strip()
    if text == "0":
        return 0.0
    mant, _, power = text.rpartition("2^")
    m = float(mant.rstrip("*")) if mant else 1.0
    return float(np.ldexp(m, int(power)))


def _bf16_value(bits):
    return float(np.array([bits << 16], np.uint32).view(np.float32)[0])


def _fill(spec, n, key=None):
    """A block of n elements from an {'all'} or {'even','odd','last'} spec;
    ``key`` picks a field of each entry (e.g. 'bf16')."""
    def get(e):
        return e if key is None else e[key]
    out = np.empty(n, dtype=object)
    if "all" in spec:
        out[:] = get(spec["all"])
    else:
        out[0::2] = get(spec["even"])
        out[1::2] = get(spec["odd"])
        if "last" in spec:
            out[-1] = get(spec["last"])
    return out


def weight_patterns(g):
    """The 512 bf16 weight patterns, after checking that every stated value
    is the value of its pattern."""
    wb = g["weights"]
    for name, spec in wb.items():
        if name == "note":
            continue
        for entry in spec.values():
            assert _bf16_value(entry["bf16"]) == parse_value(entry["value"]), (name, entry)
    parts = [_fill(wb[f"block{b}"], 64, "bf16") for b in range(7)]
    parts.append(_fill(wb["rope"], 64, "bf16"))
    return np.concatenate(parts).astype(np.uint16)


def _bf16_bits(x):
    b = int(np.array([x], np.float32).view(np.uint32)[0])
    assert b & 0xFFFF == 0, x
    return b >> 16


def scalar_scale(g):
    s = g["scalar_scale"]
    v = np.array([s["float32_bits"]], np.uint32).view(np.float32)[0]
    assert float(v) == parse_value(s["value"])
    return np.float32(v)


def inputs(g):
    """Host (numpy) inputs: bf16 as uint16 bit patterns."""
    toks = g["tokens"]
    T, H = len(toks), g["num_heads"]
    w = weight_patterns(g)
    q = np.stack([np.full((H, 512), _bf16_bits(t["value"]), np.uint16) for t in toks])
    kv = np.stack([np.full(512, _bf16_bits(t["value"]), np.uint16) for t in toks])
    rows = g["cos_sin_rows"]
    cs = np.zeros((len(rows), 64), np.float32)
    for p, r in rows.items():
        cs[int(p), :32] = r["cos"]
        cs[int(p), 32:] = r["sin"]
    pages = g["num_pages"]
    return dict(q=q, kv=kv, q_weight=w.copy(), kv_weight=w.copy(),
                cos_sin_cache=cs,
                positions=np.array([t["position"] for t in toks], np.int64),
                slot_mapping=np.array([t["slot"] for t in toks], np.int64),
                kv_cache=np.full((pages, 64, 576), I.CACHE_CANARY, np.uint8),
                kv_scale=np.full((pages, 64, 8), I.SCALE_CANARY, np.uint8),
                eps=g["eps"])


def _rope(g, tok):
    sign = "positive" if tok["value"] > 0 else "negative"
    spec = g["expected"]["rope_bf16"][f"position{tok['position']}_{sign}"]
    return _fill(spec, 64).astype(np.uint16)


def _codes(g, key, tok):
    c = np.concatenate([_fill(g["expected"][key][f"block{b}"], 64)
                        for b in range(7)]).astype(np.uint8)
    return c if tok["value"] > 0 else (c | 0x80)


def expected(g, scalar=False):
    """Expected q, kv_cache and (blockwise convention) kv_scale after the
    call; ``scalar`` gives the scalar-scale convention's cache instead."""
    x = inputs(g)
    w = x["kv_weight"]
    q = np.empty_like(x["q"])
    cache = x["kv_cache"].copy().reshape(-1, 576)
    scale = x["kv_scale"].copy().reshape(-1, 8)
    key = "scalar_codes_positive" if scalar else "codes_positive"
    for t, tok in enumerate(g["tokens"]):
        sign = 0 if tok["value"] > 0 else 0x8000
        q[t, :, :448] = w[:448] | sign
        q[t, :, 448:] = _rope(g, tok)
        s = tok["slot"]
        if s < 0:
            continue
        cache[s, :448] = _codes(g, key, tok)
        cache[s, 448:] = _rope(g, tok).view(np.uint8)  # little-endian host
        scale[s, :7] = g["expected"]["scale_bytes"]["values"]
    out = dict(q=q, kv_cache=cache.reshape(x["kv_cache"].shape))
    if not scalar:
        out["kv_scale"] = scale.reshape(x["kv_scale"].shape)
    return out


def written_slots(g):
    return np.array([t["slot"] for t in g["tokens"] if t["slot"] >= 0], np.int64)


def expected_read(g):
    """Dequantised bf16 rows of the written slots, in ``written_slots``
    order (the same for both cache conventions)."""
    deq = np.concatenate([_fill(g["expected"]["dequant"][f"block{b}"], 64)
                          for b in range(7)]).astype(np.uint16)
    rows = []
    for tok in g["tokens"]:
        if tok["slot"] < 0:
            continue
        sign = 0 if tok["value"] > 0 else 0x8000
        rows.append(np.concatenate([deq | sign, _rope(g, tok)]))
    return np.stack(rows)
