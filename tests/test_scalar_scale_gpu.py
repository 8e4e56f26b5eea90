"""Parity of the scalar-scale cache convention (write and read side) with the
oracle.  Needs an MI355X."""

import numpy as np
import pytest
import torch

import fp8_kv_cache_slot_amd as K
import oracle as O
from fp8_kv_cache_slot_amd import inputs as I
from tests import golden_case
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SMALL, TILED = 2 ** 63 - 1, 0
# The scalar-scale prologue is built in two shapes: one head per one-wave
# block (the small-batch shape and the default tiled shape) and 4 waves x 2
# heads, reached by selecting that tiling.
TILED_4X2 = (TILED, (4, 2))


@pytest.fixture(autouse=True)
def _restore():
    yield
    K.set_dispatch_threshold(-1)
    K.set_tiling(0, 0)


def _run(x, s, thr):
    tiling = (0, 0)
    if isinstance(thr, tuple):
        thr, tiling = thr
    K.set_tiling(*tiling)
    K.set_dispatch_threshold(thr)
    q, cache = x["q"].clone(), x["kv_cache"].clone()
    scale = torch.tensor([s], dtype=torch.float32, device=DEV)
    K.qnorm_rope_kv_quant_insert_scalar_scale(
        q, x["kv"], x["q_weight"], x["kv_weight"], x["cos_sin_cache"],
        x["positions"], x["slot_mapping"], cache, scale, x["eps"])
    torch.cuda.synchronize()
    return q, cache


def _oracle(h, s):
    q, cache = h["q"].copy(), h["kv_cache"].copy()
    O.qnorm_rope_kv_quant_insert_scalar(q, h["kv"], h["q_weight"], h["kv_weight"],
                                        h["cos_sin_cache"], h["positions"],
                                        h["slot_mapping"], cache, s, h["eps"])
    return q, cache


@pytest.mark.parametrize("thr", [SMALL, TILED, TILED_4X2],
                         ids=["small", "tiled", "tiled-4x2"])
def test_worked_example(thr):
    g = golden_case.load()
    h = golden_case.inputs(g)
    x = {k: (I.from_bits(v, DEV) if isinstance(v, np.ndarray) else v)
         for k, v in h.items()}
    q, cache = _run(x, 2.0 ** -8, thr)
    rq, rc = _oracle(h, 2.0 ** -8)
    np.testing.assert_array_equal(I.bits(q), rq)
    np.testing.assert_array_equal(I.bits(cache), rc)


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
@pytest.mark.parametrize("s", [0.0173, 2.0 ** -6])
def test_workloads(name, s):
    w = I.DSV4_WORKLOADS[name]
    x = I.make_dsv4(w, DEV)
    paths = ([("small", SMALL), ("tiled", TILED), ("tiled-4x2", TILED_4X2)]
             if name != "prefill" else [("default", -1)])
    if name == "prefill":
        # sampled tokens at full size
        toks = np.array(sorted(set(range(64)) | set(range(w.num_tokens - 64, w.num_tokens)) |
                               set(np.random.default_rng(5).choice(w.num_tokens, 128, replace=False).tolist())))
    else:
        toks = np.arange(w.num_tokens)
    ti = torch.from_numpy(toks).to(DEV)
    h = dict(q=I.bits(x["q"][ti]).copy(), kv=I.bits(x["kv"][ti]).copy(),
             q_weight=I.bits(x["q_weight"]), kv_weight=I.bits(x["kv_weight"]),
             cos_sin_cache=I.bits(x["cos_sin_cache"]),
             positions=I.bits(x["positions"][ti]).copy(),
             slot_mapping=I.bits(x["slot_mapping"][ti]).copy(),
             kv_cache=np.full((w.num_pages, 64, 576), I.CACHE_CANARY, np.uint8),
             eps=x["eps"])
    rq, rc = _oracle(h, s)
    num_slots = w.num_pages * 64
    v = P.valid_slots(h["slot_mapping"], num_slots)
    slots = h["slot_mapping"][v]
    for label, thr in paths:
        q, cache = _run(x, s, thr)
        P.check_bf16(I.bits(q[ti]), rq, f"{name}/{label} q")
        gc = I.bits(cache).reshape(-1, 576)
        P.check_codes(gc[slots, :448], rc.reshape(-1, 576)[slots, :448],
                      f"{name}/{label} codes")
        P.check_bf16(gc[slots, 448:].copy().view(np.uint16),
                     rc.reshape(-1, 576)[slots, 448:].copy().view(np.uint16),
                     f"{name}/{label} rope")
        if name != "prefill":
            mask = np.ones(num_slots, bool)
            mask[slots] = False
            assert np.all(gc[mask] == I.CACHE_CANARY)


@pytest.mark.parametrize("heads", [3, 7])
def test_ragged_heads(heads):
    # in the 4 x 2 shape the last wave of each token holds one head (of two)
    w = I.custom_dsv4(29, heads, seed=3200 + heads, max_position=8192)
    x = I.make_dsv4(w, DEV)
    h = {k: (I.bits(v).copy() if isinstance(v, torch.Tensor) else v)
         for k, v in x.items()}
    s = 0.0173
    rq, rc = _oracle(h, s)
    v = P.valid_slots(h["slot_mapping"], w.num_pages * 64)
    slots = h["slot_mapping"][v]
    for label, thr in [("small", SMALL), ("tiled", TILED), ("tiled-4x2", TILED_4X2)]:
        q, cache = _run(x, s, thr)
        P.check_bf16(I.bits(q), rq, f"H={heads} {label} q")
        gc = I.bits(cache).reshape(-1, 576)
        rcc = rc.reshape(-1, 576)
        P.check_codes(gc[slots, :448], rcc[slots, :448], f"H={heads} {label} codes")
        mask = np.ones(gc.shape[0], bool)
        mask[slots] = False
        assert np.all(gc[mask] == I.CACHE_CANARY)


@pytest.mark.parametrize("s", [0.0173, 3.5, 2.0 ** -10])
def test_read_side(s):
    rng = np.random.default_rng(int(s * 1000) + 7)
    cache = rng.integers(0, 256, (16, 64, 576), dtype=np.uint8)
    codes = cache[..., :448]
    codes[(codes & 0x7F) == 0x7F] ^= 0x01
    slots = rng.integers(-3, 16 * 64 + 3, 700).astype(np.int64)
    out = K.kv_cache_gather_dequant_scalar_scale(
        torch.from_numpy(cache).to(DEV), torch.tensor([s], device=DEV),
        torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    ref = O.kv_cache_gather_dequant_scalar(cache, s, slots)
    got = I.bits(out)
    # the rotary part is copied bytes (random here, NaN patterns included)
    np.testing.assert_array_equal(got[:, 448:], ref[:, 448:])
    # fp32 product then bf16 against one rounding from double
    P.check_bf16(got[:, :448], ref[:, :448], "scalar read side")


def test_read_side_many_rows_per_wave():
    # as the blockwise test: 600,001 rows, the last group partial
    rng = np.random.default_rng(46)
    cache = rng.integers(0, 256, (4, 64, 576), dtype=np.uint8)
    codes = cache[..., :448]
    codes[(codes & 0x7F) == 0x7F] ^= 0x01
    slots = rng.integers(-3, 4 * 64 + 3, 600_001).astype(np.int64)
    s = 0.0173
    table = O.kv_cache_gather_dequant_scalar(cache, s, np.arange(256, dtype=np.int64))
    table = np.concatenate([table, np.zeros((1, 512), table.dtype)])
    idx = np.where((slots >= 0) & (slots < 256), slots, 256)
    out = K.kv_cache_gather_dequant_scalar_scale(
        torch.from_numpy(cache).to(DEV), torch.tensor([s], device=DEV),
        torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    got = I.bits(out)
    # every row is one of the 257 table rows: compare the distinct ones to
    # the oracle within the bf16 bound, and every row bit-exactly to its
    # table row as the kernel produced it for the first occurrence
    first = {}
    for k, v in enumerate(idx[:20000]):
        first.setdefault(int(v), k)
    rows = np.array(sorted(first.values()))
    np.testing.assert_array_equal(got[rows][:, 448:], table[idx[rows]][:, 448:])
    P.check_bf16(got[rows][:, :448], table[idx[rows]][:, :448], "scalar read side rows")
    kernel_table = np.zeros((257, 512), got.dtype)
    kernel_table[idx[rows]] = got[rows]
    assert len(first) == 257
    np.testing.assert_array_equal(got, kernel_table[idx])


def test_zero_pages():
    w = I.custom_dsv4(9, 3, seed=99)
    x = I.make_dsv4(w, DEV)
    x["kv_cache"] = torch.empty((0, 64, 576), dtype=torch.uint8, device=DEV)
    q, _ = _run(x, 0.5, TILED)
    h = {k: (I.bits(v).copy() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    rq, _ = _oracle(h, 0.5)
    P.check_bf16(I.bits(q), rq, "zero pages q")
    out = K.kv_cache_gather_dequant_scalar_scale(
        x["kv_cache"], torch.tensor([0.5], device=DEV),
        torch.tensor([0, -1, 3], device=DEV))
    torch.cuda.synchronize()
    assert bool((out == 0).all())
