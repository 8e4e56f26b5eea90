"""Parity of the block-table read side with the CPU oracle: random caches
(never bytes the GPU wrote), random block tables with invalid page ids,
ragged and empty sequences, the length cap, output rows out of range and
untouched gaps, all bit-exact; plus the GPU writer / GPU reader round trip
against the GPU slot-list read.  Needs an MI355X."""

import numpy as np
import pytest
import torch

import fp8_kv_cache_slot_amd as K
import oracle as O
from fp8_kv_cache_slot_amd import inputs as I
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CANARY = 0x7777


def _random_cache(pages, seed):
    rng = np.random.default_rng(seed)
    cache = rng.integers(0, 256, (pages, 64, 576), dtype=np.uint8)
    codes = cache[..., :448]
    codes[(codes & 0x7F) == 0x7F] ^= 0x01     # the writer never stores NaN codes
    scale = rng.integers(127 - 40, 127 + 8, (pages, 64, 8), dtype=np.uint8)
    return cache, scale


def _both(cache, scale, table, lens, offs, N):
    ref = np.full((N, 512), CANARY, np.uint16)
    O.kv_cache_gather_dequant_paged(cache, scale, table, lens, offs, ref)
    out = torch.full((N, 512), CANARY, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    K.kv_cache_gather_dequant_paged(d(cache), d(scale), d(table.astype(np.int32)),
                                    d(lens.astype(np.int32)), d(offs.astype(np.int64)),
                                    out)
    torch.cuda.synchronize()
    return I.bits(out), ref


def test_edge_semantics():
    cache, scale = _random_cache(4, 700)
    table = np.array([[0, -1, 9], [3, 2, 1], [1, 2, 3], [2, 0, 0]], np.int32)
    lens = np.array([150, 0, 300, 5], np.int32)
    offs = np.array([10, 0, 170, 395], np.int64)
    got, ref = _both(cache, scale, table, lens, offs, 398)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("seed", [701, 702, 703])
def test_random_tables(seed):
    rng = np.random.default_rng(seed)
    pages = int(rng.integers(3, 40))
    cache, scale = _random_cache(pages, seed)
    S = int(rng.integers(1, 12))
    M = int(rng.integers(1, 6))
    table = rng.integers(-2, pages + 2, (S, M)).astype(np.int32)
    lens = rng.integers(-1, M * 64 + 20, S).astype(np.int32)
    # disjoint output ranges (a precondition), with gaps between them
    start = int(rng.integers(0, 5))
    offs = start + np.concatenate(
        [[0], np.cumsum(np.maximum(lens, 0) + rng.integers(0, 7, S))[:-1]])
    N = int(offs[-1] + max(lens[-1], 0) - rng.integers(0, 3))
    got, ref = _both(cache, scale, table, lens, offs.astype(np.int64), max(N, 1))
    np.testing.assert_array_equal(got, ref)


def test_full_size_page_permutation():
    # 32 sequences x 4096 tokens over all 2048 pages of a cache, pages in a
    # random order: every row of the 131072 compared with the oracle
    pages, S, L = 2048, 32, 4096
    cache, scale = _random_cache(pages, 704)
    perm = np.random.default_rng(705).permutation(pages).astype(np.int32)
    table = perm.reshape(S, pages // S)
    lens = np.full(S, L, np.int32)
    offs = (np.arange(S) * L).astype(np.int64)
    got, ref = _both(cache, scale, table, lens, offs, S * L)
    np.testing.assert_array_equal(got, ref)


def test_zero_pages_and_empty_calls():
    empty_c = torch.empty((0, 64, 576), dtype=torch.uint8, device=DEV)
    empty_s = torch.empty((0, 64, 8), dtype=torch.uint8, device=DEV)
    table = torch.tensor([[0, 1]], dtype=torch.int32, device=DEV)
    out = torch.full((80, 512), CANARY, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    K.kv_cache_gather_dequant_paged(empty_c, empty_s, table,
                                    torch.tensor([70], dtype=torch.int32, device=DEV),
                                    torch.tensor([5], dtype=torch.int64, device=DEV), out)
    torch.cuda.synchronize()
    b = I.bits(out)
    assert np.all(b[5:75] == 0) and np.all(b[:5] == CANARY) and np.all(b[75:] == CANARY)
    # no sequences: nothing happens
    K.kv_cache_gather_dequant_paged(empty_c, empty_s, table[:0],
                                    torch.empty(0, dtype=torch.int32, device=DEV),
                                    torch.empty(0, dtype=torch.int64, device=DEV), out)
    torch.cuda.synchronize()
    assert np.array_equal(I.bits(out), b)


def test_gpu_writer_gpu_reader_round_trip():
    # The GPU prologue writes sequences into pages taken from a shuffled free
    # list; reading them back through the block table equals the GPU
    # slot-list read of the writer's slots.
    rng = np.random.default_rng(706)
    lens = [70, 1, 128, 33, 0, 64, 200]
    M, pages = 4, 16
    free = iter(rng.permutation(pages).tolist())
    table = np.full((len(lens), M), -1, np.int32)
    slots = []
    for s, L in enumerate(lens):
        own = [next(free) for _ in range(-(-L // 64))]
        table[s, :len(own)] = own
        ranges = [np.arange(p * 64, p * 64 + 64) for p in own]
        slots.append(np.concatenate(ranges)[:L] if ranges else np.zeros(0, np.int64))
    sm = np.concatenate(slots).astype(np.int64)
    T = sm.shape[0]
    x = I.make_dsv4(I.custom_dsv4(T, 3, seed=707, num_pages=pages), DEV)
    x["slot_mapping"] = torch.from_numpy(sm).to(DEV)
    K.qnorm_rope_kv_quant_insert(x["q"], x["kv"], x["q_weight"], x["kv_weight"],
                                 x["cos_sin_cache"], x["positions"],
                                 x["slot_mapping"], x["kv_cache"], x["kv_scale"],
                                 x["eps"])
    flat = K.kv_cache_gather_dequant(x["kv_cache"], x["kv_scale"], x["slot_mapping"])
    out = torch.empty((T, 512), dtype=torch.bfloat16, device=DEV)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    K.kv_cache_gather_dequant_paged(x["kv_cache"], x["kv_scale"],
                                    torch.from_numpy(table).to(DEV),
                                    torch.tensor(lens, dtype=torch.int32, device=DEV),
                                    torch.from_numpy(offs).to(DEV), out)
    torch.cuda.synchronize()
    assert torch.equal(out, flat)


# ---------------------------------------------------------------------------
# the scalar-scale convention through block tables
# ---------------------------------------------------------------------------

def _both_scalar(cache, s, table, lens, offs, N):
    ref = np.full((N, 512), CANARY, np.uint16)
    O.kv_cache_gather_dequant_paged_scalar(cache, s, table, lens, offs, ref)
    out = torch.full((N, 512), CANARY, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    K.kv_cache_gather_dequant_paged_scalar_scale(
        d(cache), torch.tensor([s], dtype=torch.float32, device=DEV),
        d(table.astype(np.int32)), d(lens.astype(np.int32)),
        d(offs.astype(np.int64)), out)
    torch.cuda.synchronize()
    return I.bits(out), ref


def _check_scalar_rows(got, ref, what):
    # rows the oracle left alone (canary) and the rotary part: bit-exact; the
    # dequantised dims: fp32 product then bf16 against one rounding from double
    np.testing.assert_array_equal(got[:, 448:], ref[:, 448:], err_msg=what)
    untouched = np.all(ref == CANARY, axis=1)
    np.testing.assert_array_equal(got[untouched], ref[untouched], err_msg=what)
    P.check_bf16(got[~untouched, :448], ref[~untouched, :448], what)


def test_scalar_edge_semantics():
    cache, _ = _random_cache(4, 710)
    table = np.array([[0, -1, 9], [3, 2, 1], [1, 2, 3], [2, 0, 0]], np.int32)
    lens = np.array([150, 0, 300, 5], np.int32)
    offs = np.array([10, 0, 170, 395], np.int64)
    got, ref = _both_scalar(cache, 0.0173, table, lens, offs, 398)
    _check_scalar_rows(got, ref, "scalar edge semantics")


@pytest.mark.parametrize("seed", [711, 712, 713])
def test_scalar_random_tables(seed):
    rng = np.random.default_rng(seed)
    pages = int(rng.integers(3, 40))
    cache, _ = _random_cache(pages, seed)
    s = float(rng.choice([0.0173, 3.5, 2.0 ** -10]))
    S = int(rng.integers(1, 12))
    M = int(rng.integers(1, 6))
    table = rng.integers(-2, pages + 2, (S, M)).astype(np.int32)
    lens = rng.integers(-1, M * 64 + 20, S).astype(np.int32)
    start = int(rng.integers(0, 5))
    offs = start + np.concatenate(
        [[0], np.cumsum(np.maximum(lens, 0) + rng.integers(0, 7, S))[:-1]])
    N = int(offs[-1] + max(lens[-1], 0) - rng.integers(0, 3))
    got, ref = _both_scalar(cache, s, table, lens, offs.astype(np.int64), max(N, 1))
    _check_scalar_rows(got, ref, f"scalar random tables seed {seed} s={s}")


def test_scalar_full_size_equals_the_slot_list_read():
    # all 2048 pages in a random order: every row equals, bit for bit, the
    # GPU slot-list read of the slots the tables name (same arithmetic)
    pages, S, L = 2048, 32, 4096
    cache, _ = _random_cache(pages, 714)
    perm = np.random.default_rng(715).permutation(pages).astype(np.int32)
    table = perm.reshape(S, pages // S)
    sc = torch.tensor([0.0173], dtype=torch.float32, device=DEV)
    dc = torch.from_numpy(cache).to(DEV)
    out = torch.empty((S * L, 512), dtype=torch.bfloat16, device=DEV)
    K.kv_cache_gather_dequant_paged_scalar_scale(
        dc, sc, torch.from_numpy(table).to(DEV),
        torch.full((S,), L, dtype=torch.int32, device=DEV),
        torch.arange(S, dtype=torch.int64, device=DEV) * L, out)
    slots = (table.astype(np.int64)[:, :, None] * 64 + np.arange(64)).reshape(-1)
    flat = K.kv_cache_gather_dequant_scalar_scale(dc, sc, torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), flat.view(torch.int16))
    # and a sample of rows against the oracle
    rows = np.random.default_rng(716).choice(S * L, 512, replace=False)
    ref = O.kv_cache_gather_dequant_scalar(cache, 0.0173, slots[rows])
    got = I.bits(out)[rows]
    np.testing.assert_array_equal(got[:, 448:], ref[:, 448:])
    P.check_bf16(got[:, :448], ref[:, :448], "scalar full size sample")


def test_scalar_zero_pages():
    empty_c = torch.empty((0, 64, 576), dtype=torch.uint8, device=DEV)
    sc = torch.tensor([0.5], dtype=torch.float32, device=DEV)
    out = torch.full((80, 512), CANARY, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    K.kv_cache_gather_dequant_paged_scalar_scale(
        empty_c, sc, torch.tensor([[0, 1]], dtype=torch.int32, device=DEV),
        torch.tensor([70], dtype=torch.int32, device=DEV),
        torch.tensor([5], dtype=torch.int64, device=DEV), out)
    torch.cuda.synchronize()
    b = I.bits(out)
    assert np.all(b[5:75] == 0) and np.all(b[:5] == CANARY) and np.all(b[75:] == CANARY)
