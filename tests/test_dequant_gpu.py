"""Parity of the cache read side (gather + dequantise) with the CPU oracle.
Cache bytes come from the oracle's own prologue or from a seeded random
generator, never from the GPU path.  Needs an MI355X."""

import numpy as np
import pytest
import torch

import fp8_kv_cache_slot_amd as K
import oracle as O
from fp8_kv_cache_slot_amd import inputs as I
from tests import golden_case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _val(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _random_cache(pages, seed, e_lo=127 - 40, e_hi=127 + 8):
    rng = np.random.default_rng(seed)
    cache = rng.integers(0, 256, (pages, 64, 576), dtype=np.uint8)
    codes = cache[..., :448]
    codes[(codes & 0x7F) == 0x7F] ^= 0x01     # the writer never stores NaN codes
    scale = rng.integers(e_lo, e_hi, (pages, 64, 8), dtype=np.uint8)
    return cache, scale


def _gpu(cache, scale, slots):
    out = K.kv_cache_gather_dequant(torch.from_numpy(cache).to(DEV),
                                    torch.from_numpy(scale).to(DEV),
                                    torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    return I.bits(out)


def test_golden_cache_round_trip():
    g = golden_case.load()
    x = golden_case.inputs(g)
    O.qnorm_rope_kv_quant_insert(x["q"], x["kv"], x["q_weight"], x["kv_weight"],
                                 x["cos_sin_cache"], x["positions"],
                                 x["slot_mapping"], x["kv_cache"], x["kv_scale"],
                                 x["eps"])
    slots = np.array([5, 2, -1, 64, 3], np.int64)
    got = _gpu(x["kv_cache"], x["kv_scale"], slots)
    np.testing.assert_array_equal(got, O.kv_cache_gather_dequant(
        x["kv_cache"], x["kv_scale"], slots))
    np.testing.assert_array_equal(got[0], x["kv_weight"])


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_oracle_written_cache(name):
    w = I.DSV4_WORKLOADS[name]
    x = {k: (I.bits(v).copy() if isinstance(v, torch.Tensor) else v)
         for k, v in I.make_dsv4(w, "cpu").items()}
    O.qnorm_rope_kv_quant_insert(x["q"], x["kv"], x["q_weight"], x["kv_weight"],
                                 x["cos_sin_cache"], x["positions"],
                                 x["slot_mapping"], x["kv_cache"], x["kv_scale"],
                                 x["eps"])
    rng = np.random.default_rng(w.seed)
    slots = np.concatenate([x["slot_mapping"],
                            rng.integers(-3, w.num_pages * 64 + 3, 37)]).astype(np.int64)
    got = _gpu(x["kv_cache"], x["kv_scale"], slots)
    np.testing.assert_array_equal(got, O.kv_cache_gather_dequant(
        x["kv_cache"], x["kv_scale"], slots))


@pytest.mark.parametrize("rows", [1, 7, 8, 9, 1000])
def test_random_cache_ragged_row_counts(rows):
    cache, scale = _random_cache(4, seed=40 + rows)
    rng = np.random.default_rng(rows)
    slots = rng.integers(-2, 4 * 64 + 2, rows).astype(np.int64)
    got = _gpu(cache, scale, slots)
    np.testing.assert_array_equal(got, O.kv_cache_gather_dequant(cache, scale, slots))


def test_full_size_permutation_of_long_cache():
    # every slot of a 2048-page cache, in a random order, compared in full
    cache, scale = _random_cache(2048, seed=41)
    slots = np.random.default_rng(42).permutation(2048 * 64).astype(np.int64)
    got = _gpu(cache, scale, slots)
    np.testing.assert_array_equal(got, O.kv_cache_gather_dequant(cache, scale, slots))


def test_many_rows_per_wave():
    # 600,001 rows from a 256-slot cache (slots repeat; some are invalid): a
    # grid of 150,001 blocks whose last group is partial (one row).  The
    # oracle decodes each distinct slot once; a repeated slot has the same row
    # by definition, an invalid one a zero row.
    cache, scale = _random_cache(4, seed=44)
    rng = np.random.default_rng(45)
    slots = rng.integers(-3, 4 * 64 + 3, 600_001).astype(np.int64)
    table = O.kv_cache_gather_dequant(cache, scale, np.arange(256, dtype=np.int64))
    table = np.concatenate([table, np.zeros((1, 512), table.dtype)])
    idx = np.where((slots >= 0) & (slots < 256), slots, 256)
    got = _gpu(cache, scale, slots)
    np.testing.assert_array_equal(got, table[idx])


def test_exponent_range_and_empty_inputs():
    # exponents over [-110, +100]: every product is a normal or zero bf16
    cache, scale = _random_cache(2, seed=43, e_lo=17, e_hi=228)
    slots = np.arange(128, dtype=np.int64)
    got = _gpu(cache, scale, slots)
    np.testing.assert_array_equal(got, O.kv_cache_gather_dequant(cache, scale, slots))
    # zero pages: every row is zero
    empty_c = torch.empty((0, 64, 576), dtype=torch.uint8, device=DEV)
    empty_s = torch.empty((0, 64, 8), dtype=torch.uint8, device=DEV)
    out = K.kv_cache_gather_dequant(empty_c, empty_s,
                                    torch.tensor([0, -1, 5], device=DEV))
    torch.cuda.synchronize()
    assert bool((out == 0).all())
    # zero rows: nothing happens
    out = K.kv_cache_gather_dequant(empty_c, empty_s,
                                    torch.empty(0, dtype=torch.int64, device=DEV))
    assert out.shape == (0, 512)


def test_gpu_round_trip_within_quantisation_error():
    # GPU prologue then GPU read side, against the oracle's unrounded values
    w = I.DSV4_WORKLOADS["decode"]
    x = I.make_dsv4(w, DEV)
    q, cache, scale = x["q"].clone(), x["kv_cache"].clone(), x["kv_scale"].clone()
    K.qnorm_rope_kv_quant_insert(q, x["kv"], x["q_weight"], x["kv_weight"],
                                 x["cos_sin_cache"], x["positions"],
                                 x["slot_mapping"], cache, scale, x["eps"])
    sm = x["slot_mapping"]
    valid = sm >= 0
    out = K.kv_cache_gather_dequant(cache, scale, sm[valid].contiguous())
    torch.cuda.synchronize()
    y = O.kv_normalised(I.bits(x["kv"][valid]), I.bits(x["kv_weight"]),
                        I.bits(x["cos_sin_cache"]), I.bits(x["positions"][valid]),
                        w.eps)
    got = _val(I.bits(out))
    e = I.bits(scale).reshape(-1, 8)[I.bits(sm[valid])][:, :7].astype(np.float64) - 127
    e = np.repeat(e, 64, axis=1)
    yq = y[:, :448]
    # half an E4M3 step, plus one step where the kernel's fp32 value and the
    # oracle's double value straddle a rounding boundary
    bound = np.maximum(np.abs(yq) * 2.0 ** -3, np.exp2(e - 9)) * 1.01
    assert np.all(np.abs(got[:, :448] - yq) <= bound)
    yr = y[:, 448:]
    assert np.all(np.abs(got[:, 448:] - yr) <= np.abs(yr) * 2.0 ** -7 + 1e-3)
