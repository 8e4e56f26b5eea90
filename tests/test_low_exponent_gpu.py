"""The hand-derived worked example at the bottom of the exponent range
(``golden/dsv4_low_exponent_rows.json``) on the GPU, bit for bit: the UE8M0
exponent clamped to -127, the unclamped boundary 448 * 2^-127, fp32-subnormal
normalised values, scaled codes and rotated rotary dims, bf16 subnormal q and
cache outputs, and their dequantisation back into the subnormal range by both
read sides.  Through both dispatch sides, a multi-wave tiling, both cache
conventions and the separate-launch stages.  Needs an MI355X."""

import numpy as np
import pytest
import torch

import fp8_kv_cache_slot_amd as K
from fp8_kv_cache_slot_amd import inputs as I
from tests import golden_low_case as G

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SMALL = 2 ** 63 - 1   # every call to the small-batch kernel
TILED = 0             # every call to the tiled kernel
PATHS = [("small", SMALL, None), ("tiled", TILED, None), ("tiled4x2", TILED, (4, 2))]


@pytest.fixture(autouse=True)
def _restore_knobs():
    yield
    K.set_dispatch_threshold(-1)
    K.set_tiling(0, 0)


def _device_inputs(g):
    return {k: (I.from_bits(v, DEV) if isinstance(v, np.ndarray) else v)
            for k, v in G.inputs(g).items()}


def _set_path(threshold, tiling):
    K.set_dispatch_threshold(threshold)
    if tiling:
        K.set_tiling(*tiling)


def _read_back(g, cache, scale=None, s=None):
    """Both read sides of the written slots: by slot list and through a block
    table of the whole page (only the written rows are compared)."""
    slots = G.written_slots(g)
    si = torch.from_numpy(slots).to(DEV)
    table = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    lens = torch.tensor([64], dtype=torch.int32, device=DEV)
    offs = torch.zeros(1, dtype=torch.int64, device=DEV)
    page = torch.zeros((64, 512), dtype=torch.bfloat16, device=DEV)
    if s is None:
        rows = K.kv_cache_gather_dequant(cache, scale, si)
        K.kv_cache_gather_dequant_paged(cache, scale, table, lens, offs, page)
    else:
        rows = K.kv_cache_gather_dequant_scalar_scale(cache, s, si)
        K.kv_cache_gather_dequant_paged_scalar_scale(cache, s, table, lens, offs, page)
    torch.cuda.synchronize()
    return I.bits(rows), I.bits(page)[slots]


@pytest.mark.parametrize("label,threshold,tiling", PATHS, ids=[p[0] for p in PATHS])
def test_blockwise_convention(label, threshold, tiling):
    g = G.load()
    x = _device_inputs(g)
    exp = G.expected(g)
    q, cache, scale = x["q"].clone(), x["kv_cache"].clone(), x["kv_scale"].clone()
    _set_path(threshold, tiling)
    K.qnorm_rope_kv_quant_insert(q, x["kv"], x["q_weight"], x["kv_weight"],
                                 x["cos_sin_cache"], x["positions"],
                                 x["slot_mapping"], cache, scale, x["eps"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(I.bits(q), exp["q"])
    np.testing.assert_array_equal(I.bits(scale), exp["kv_scale"])
    np.testing.assert_array_equal(I.bits(cache), exp["kv_cache"])
    want = G.expected_read(g)
    by_slot, by_table = _read_back(g, cache, scale=scale)
    np.testing.assert_array_equal(by_slot, want)
    np.testing.assert_array_equal(by_table, want)


@pytest.mark.parametrize("label,threshold,tiling", PATHS, ids=[p[0] for p in PATHS])
def test_scalar_scale_convention(label, threshold, tiling):
    g = G.load()
    x = _device_inputs(g)
    exp = G.expected(g, scalar=True)
    s = torch.tensor([G.scalar_scale(g)], dtype=torch.float32, device=DEV)
    q, cache = x["q"].clone(), x["kv_cache"].clone()
    _set_path(threshold, tiling)
    K.qnorm_rope_kv_quant_insert_scalar_scale(
        q, x["kv"], x["q_weight"], x["kv_weight"], x["cos_sin_cache"],
        x["positions"], x["slot_mapping"], cache, s, x["eps"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(I.bits(q), exp["q"])
    np.testing.assert_array_equal(I.bits(cache), exp["kv_cache"])
    want = G.expected_read(g)
    by_slot, by_table = _read_back(g, cache, s=s)
    np.testing.assert_array_equal(by_slot, want)
    np.testing.assert_array_equal(by_table, want)


def test_separate_launch_stages():
    # RMSNorm, RoPE and quantise+insert as separate launches: every
    # intermediate here is a bf16 value (x * w, and the rotated pairs), so the
    # extra bf16 rounding between stages changes nothing and the bytes are the
    # fused call's
    g = G.load()
    x = _device_inputs(g)
    exp = G.expected(g)
    q, cache, scale = x["q"].clone(), x["kv_cache"].clone(), x["kv_scale"].clone()
    K.unfused_prologue(q, x["kv"], x["q_weight"], x["kv_weight"],
                       x["cos_sin_cache"], x["positions"], x["slot_mapping"],
                       cache, scale, x["eps"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(I.bits(q), exp["q"])
    np.testing.assert_array_equal(I.bits(scale), exp["kv_scale"])
    np.testing.assert_array_equal(I.bits(cache), exp["kv_cache"])
