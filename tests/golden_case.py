"""Builds the inputs and expected outputs of the hand-derived worked example in
``golden/dsv4_constant_rows.json`` (constant rows, eps = 0).  Test helper only:
numbers come from the fixture, never from either implementation."""

import json
import os

import numpy as np
import torch

from fp8_kv_cache_slot_amd import inputs as I

HERE = os.path.dirname(os.path.abspath(__file__))
PATH = os.path.join(HERE, "golden", "dsv4_constant_rows.json")


def load():
    with open(PATH) as f:
        return json.load(f)


def _bf16_bits(x):
    return int(torch.tensor([x], dtype=torch.float32).to(torch.bfloat16)
               .view(torch.int16).item()) & 0xFFFF


def _fill(spec, n):
    out = np.empty(n, dtype=np.float64)
    if "all" in spec:
        out[:] = spec["all"]
    else:
        out[0::2] = spec["even"]
        out[1::2] = spec["odd"]
        if "last" in spec:
            out[-1] = spec["last"]
    return out


def inputs(g):
    """Host (numpy) inputs: bf16 as uint16 bit patterns."""
    T = len(g["tokens"])
    H = g["num_heads"]
    w = []
    for b in range(7):
        w.append(_fill(g["kv_weight_blocks"][f"block{b}"], 64))
    w.append(_fill(g["kv_weight_blocks"]["rope"], 64))
    kv_weight = np.array([_bf16_bits(v) for v in np.concatenate(w)], np.uint16)
    q_weight = np.full(512, _bf16_bits(g["q_weight"]), np.uint16)
    q = np.full((T, H, 512), _bf16_bits(g["q_value"]), np.uint16)
    kv = np.stack([np.full(512, _bf16_bits(t["kv_value"]), np.uint16)
                   for t in g["tokens"]])
    rows = g["cos_sin_rows"]
    cs = np.zeros((len(rows), 64), np.float32)
    for p, r in rows.items():
        cs[int(p), :32] = r["cos"]
        cs[int(p), 32:] = r["sin"]
    positions = np.array([t["position"] for t in g["tokens"]], np.int64)
    slots = np.array([t["slot"] for t in g["tokens"]], np.int64)
    pages = g["num_pages"]
    cache = np.full((pages, 64, 576), I.CACHE_CANARY, np.uint8)
    scale = np.full((pages, 64, 8), I.SCALE_CANARY, np.uint8)
    return dict(q=q, kv=kv, q_weight=q_weight, kv_weight=kv_weight,
                cos_sin_cache=cs, positions=positions, slot_mapping=slots,
                kv_cache=cache, kv_scale=scale, eps=g["eps"])


def expected(g):
    """Expected q, kv_cache and kv_scale after the call."""
    e = g["expected"]
    x = inputs(g)
    T, H = x["q"].shape[:2]
    q = np.empty_like(x["q"])
    for t, tok in enumerate(g["tokens"]):
        if tok["position"] == 0:
            q[t] = e["q_token_position0"]["all"]
        else:
            s = e["q_token_position1"]
            q[t, :, :448] = s["dims_0_447"]
            q[t, :, 448::2] = s["rope_even"]
            q[t, :, 449::2] = s["rope_odd"]
    cache = x["kv_cache"].copy().reshape(-1, 576)
    scale = x["kv_scale"].copy().reshape(-1, 8)
    codes0 = np.concatenate(
        [_fill(e["codes_token0"][f"block{b}"], 64) for b in range(7)]
    ).astype(np.uint8)
    for t, tok in enumerate(g["tokens"]):
        s = tok["slot"]
        if s < 0:
            continue
        codes = codes0 if tok["kv_value"] > 0 else (codes0 | 0x80)
        cache[s, :448] = codes
        rope = _fill(e["rope_bf16_token0" if tok["position"] == 0
                       else "rope_bf16_token1"], 64).astype(np.uint16)
        cache[s, 448:] = rope.view(np.uint8)  # little-endian host
        scale[s, :7] = e["scale_bytes"]["values"]
    return dict(q=q, kv_cache=cache.reshape(x["kv_cache"].shape),
                kv_scale=scale.reshape(x["kv_scale"].shape))
