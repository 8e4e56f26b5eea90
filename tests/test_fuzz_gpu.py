"""Seeded random cases against the oracle: each case draws its own sizes and
knobs (token and head counts, cache pages, skipped and out-of-range slots,
eps, the built tiling and the dispatch side for the fused prologue; head
width, rotary width, pairing, dtype and head mix for the packed forms; the
cache, slots, block tables and output layout for the read sides), so
combinations no hand-written case names get checked too.  Every case is
deterministic in its seed and small enough for the oracle to finish in well
under a second.  Needs an MI355X.  FP8KV_FUZZ_CASES sets the number of
cases of each kind (default 128)."""

import os

import numpy as np
import pytest
import torch

import fp8_kv_cache_slot_amd as K
import oracle as O
from fp8_kv_cache_slot_amd import inputs as I
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CASES = int(os.environ.get("FP8KV_FUZZ_CASES", "128"))
SHAPES = [(1, 1), (1, 2), (2, 1), (2, 2), (4, 1), (4, 2), (4, 4), (8, 1),
          (8, 2), (8, 4), (16, 1), (16, 2)]


@pytest.fixture(autouse=True)
def _restore_knobs():
    yield
    K.set_dispatch_threshold(-1)
    K.set_tiling(0, 0)


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("case", range(CASES))
def test_prologue_random_case(case):
    rng = np.random.default_rng(7000 + case)
    T = int(rng.integers(1, 300))
    H = int(rng.integers(1, 97))
    pages = int(np.ceil(T * rng.uniform(1.0, 3.0) / 64))
    skipped = int(rng.integers(0, T // 4 + 1))
    eps = float(rng.choice([1e-6, 1e-3, 0.5]))
    shape = SHAPES[int(rng.integers(len(SHAPES)))]
    threshold = int(rng.choice([0, 2 ** 63 - 1]))
    _say(f"case {case}: T={T} H={H} pages={pages} skipped={skipped} eps={eps} "
         f"tiling={shape} threshold={threshold}")
    w = I.custom_dsv4(T, H, 7100 + case, num_pages=pages,
                      outliers=bool(rng.integers(2)), max_position=2048,
                      skipped=skipped)
    x = I.make_dsv4(w, DEV)
    x["eps"] = eps
    # a few tokens point past the cache: they are skipped like slot -1
    n_out = int(rng.integers(0, 3))
    if n_out:
        idx = rng.choice(T, size=min(n_out, T), replace=False)
        x["slot_mapping"][torch.from_numpy(idx).to(DEV)] = pages * 64 + torch.arange(
            len(idx), device=DEV)
    h = {k: (I.bits(v).copy() if isinstance(v, torch.Tensor) else v)
         for k, v in x.items()}

    K.set_tiling(*shape)
    K.set_dispatch_threshold(threshold)
    q, cache, scale = x["q"].clone(), x["kv_cache"].clone(), x["kv_scale"].clone()
    K.qnorm_rope_kv_quant_insert(q, x["kv"], x["q_weight"], x["kv_weight"],
                                 x["cos_sin_cache"], x["positions"],
                                 x["slot_mapping"], cache, scale, eps)
    torch.cuda.synchronize()

    ref = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in h.items()}
    O.qnorm_rope_kv_quant_insert(ref["q"], ref["kv"], ref["q_weight"],
                                 ref["kv_weight"], ref["cos_sin_cache"],
                                 ref["positions"], ref["slot_mapping"],
                                 ref["kv_cache"], ref["kv_scale"], eps)
    what = f"case {case}"
    P.check_bf16(I.bits(q), ref["q"], what + " q")
    num_slots = pages * 64
    v = P.valid_slots(h["slot_mapping"], num_slots)
    slots = h["slot_mapping"][v]
    y = O.kv_normalised(h["kv"][v].copy(), h["kv_weight"], h["cos_sin_cache"],
                        h["positions"][v].copy(), eps)
    P.check_cache(I.bits(cache), I.bits(scale), ref["kv_cache"], ref["kv_scale"],
                  slots, y, I.CACHE_CANARY, I.SCALE_CANARY, what)
    P.check_untouched(I.bits(cache), I.bits(scale), slots, I.CACHE_CANARY,
                      I.SCALE_CANARY, what)


def _bits16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("case", range(CASES))
def test_packed_random_case(case):
    rng = np.random.default_rng(8000 + case)
    D = int(rng.choice([64, 128, 256]))
    R = int(rng.choice([r for r in range(0, D + 1, 16)]))
    neox = bool(rng.integers(2))
    dtype = torch.float16 if rng.integers(2) else torch.bfloat16
    hq, hk, hv = (int(v) for v in rng.integers(0, 21, 3))
    if hq + hk == 0:
        hq = 1
    T = int(rng.integers(1, 300))
    # one case in eight launches just over 8192 waves, where the variants
    # kernel leaves its block-sharing forms for one-wave blocks
    if rng.random() < 0.125:
        waves_per_token = max(1, -(-(hq + hk) // (3 * (512 // D))))
        T = -(-8193 // waves_per_token) + int(rng.integers(0, 64))
    guarded = dtype == torch.bfloat16 and D == 128 and R == 128 and neox
    _say(f"case {case}: T={T} heads={hq},{hk},{hv} D={D} R={R} neox={neox} "
         f"{dtype} guarded={guarded}")
    g = torch.Generator(device=DEV)
    g.manual_seed(8100 + case)
    qkv = torch.randn((T, (hq + hk + hv) * D), generator=g, device=DEV).to(dtype)
    qw = (torch.rand(D, generator=g, device=DEV) + 0.5).to(dtype)
    kw = (torch.rand(D, generator=g, device=DEV) + 0.5).to(dtype)
    max_pos = 1024
    cs = (I.cos_sin_cache(max_pos, R, device=DEV) if R else
          torch.zeros((max_pos, 0), dtype=torch.float32, device=DEV))
    pos = torch.randint(0, max_pos, (T,), generator=g, device=DEV)
    out = qkv.clone()
    if guarded and rng.integers(2):
        K.qk_norm_rope_packed(out, hq, hk, hv, D, 1e-6, qw, kw, cs, True, pos)
    else:
        K.qk_norm_rope_packed_ex(out, hq, hk, hv, D, 1e-6, qw, kw, cs, neox, pos,
                                 rotary_dim=R)
    torch.cuda.synchronize()
    ref = _bits16(qkv).copy()
    O.qk_norm_rope_packed_ex(ref, hq, hk, hv, D, R, int(neox),
                             int(dtype == torch.float16), 1e-6, _bits16(qw),
                             _bits16(kw), I.bits(cs).copy(), I.bits(pos))
    got = _bits16(out)
    n = (hq + hk) * D
    np.testing.assert_array_equal(got[:, n:], _bits16(qkv)[:, n:],
                                  err_msg=f"case {case}: V changed")
    chk = P.check_fp16 if dtype == torch.float16 else P.check_bf16
    chk(got[:, :n], ref[:, :n], f"case {case}")


@pytest.mark.parametrize("case", range(max(8, CASES // 2)))
def test_packed_guarded_random_case(case):
    # The guarded entry point (bf16, head_dim 128, full NeoX) on random head
    # mixes, up to 160 Q/K heads: a token spans up to 14 waves of 12 heads,
    # so up to two blocks, each reading the position and cos/sin row itself.
    # A few positions are out of range: those tokens are left as they were.
    rng = np.random.default_rng(8500 + case)
    hq, hk, hv = int(rng.integers(0, 121)), int(rng.integers(0, 41)), int(rng.integers(0, 17))
    if hq + hk == 0:
        hk = 1
    T = int(rng.integers(1, 3001))
    _say(f"guarded case {case}: T={T} heads={hq},{hk},{hv}")
    w = I.PackedWorkload("fuzz", T, hq, hk, hv, max_position=2048, seed=8600 + case)
    x = I.make_packed(w, DEV)
    bad = rng.choice(T, size=min(T, int(rng.integers(0, 4))), replace=False)
    pos = x["position_ids"].clone()
    for i, b in enumerate(bad):
        pos[int(b)] = [-1, 2048, 2 ** 40][i % 3]
    out = x["qkv"].clone()
    K.qk_norm_rope_packed(out, hq, hk, hv, 128, w.eps, x["q_weight"], x["k_weight"],
                          x["cos_sin_cache"], True, pos)
    torch.cuda.synchronize()
    n = (hq + hk) * 128
    got, src = I.bits(out), I.bits(x["qkv"])
    np.testing.assert_array_equal(got[:, n:], src[:, n:], err_msg=f"case {case}: V changed")
    keep = np.setdiff1d(np.arange(T), bad)
    np.testing.assert_array_equal(got[bad], src[bad], err_msg=f"case {case}: skipped token written")
    ref = src[keep].copy()
    O.qk_norm_rope_packed(ref, hq, hk, hv, 128, w.eps, I.bits(x["q_weight"]),
                          I.bits(x["k_weight"]), I.bits(x["cos_sin_cache"]),
                          I.bits(pos)[keep].copy())
    P.check_bf16(got[keep][:, :n], ref[:, :n], f"guarded case {case}")


@pytest.mark.parametrize("case", range(CASES))
def test_read_side_random_case(case):
    # The four read sides (slot list or block tables, blockwise or scalar
    # scale) on random caches of 0 to 39 pages: slots and page ids past either
    # end, sequences longer than their table row or of negative length,
    # disjoint output ranges with gaps and rows past the output.
    rng = np.random.default_rng(9000 + case)
    pages = int(rng.integers(0, 40))
    scalar = bool(rng.integers(2))
    paged = bool(rng.integers(2))
    s = float(rng.choice([2.0 ** -8, 0.37, 3.0, 2.0 ** 10]))
    cache = rng.integers(0, 256, (pages, 64, 576), dtype=np.uint8)
    codes = cache[..., :448]
    codes[(codes & 0x7F) == 0x7F] ^= 0x01     # the writer never stores NaN codes
    scale = rng.integers(127 - 60, 127 + 10, (pages, 64, 8), dtype=np.uint8)
    sc = torch.tensor([s], dtype=torch.float32, device=DEV)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)

    if not paged:
        rows = int(rng.integers(1, 3000))
        slots = rng.integers(-3, pages * 64 + 3, rows).astype(np.int64)
        _say(f"read case {case}: pages={pages} scalar={scalar} slot list of {rows}")
        if scalar:
            out = K.kv_cache_gather_dequant_scalar_scale(d(cache), sc, d(slots))
            ref = O.kv_cache_gather_dequant_scalar(cache, s, slots)
        else:
            out = K.kv_cache_gather_dequant(d(cache), d(scale), d(slots))
            ref = O.kv_cache_gather_dequant(cache, scale, slots)
    else:
        S, M = int(rng.integers(1, 12)), int(rng.integers(1, 6))
        table = rng.integers(-2, pages + 2, (S, M)).astype(np.int32)
        lens = rng.integers(-1, M * 64 + 20, S).astype(np.int32)
        gaps = np.maximum(lens, 0) + rng.integers(0, 7, S)
        offs = (int(rng.integers(0, 5)) +
                np.concatenate([[0], np.cumsum(gaps)[:-1]])).astype(np.int64)
        N = max(1, int(offs[-1]) + max(int(lens[-1]), 0) - int(rng.integers(0, 3)))
        _say(f"read case {case}: pages={pages} scalar={scalar} tables {S}x{M} N={N}")
        ref = np.full((N, 512), 0x7777, np.uint16)
        out = torch.full((N, 512), 0x7777, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        if scalar:
            K.kv_cache_gather_dequant_paged_scalar_scale(d(cache), sc, d(table), d(lens),
                                                         d(offs), out)
            O.kv_cache_gather_dequant_paged_scalar(cache, s, table, lens, offs, ref)
        else:
            K.kv_cache_gather_dequant_paged(d(cache), d(scale), d(table), d(lens),
                                            d(offs), out)
            O.kv_cache_gather_dequant_paged(cache, scale, table, lens, offs, ref)
    torch.cuda.synchronize()
    got = I.bits(out)
    if scalar:
        # rotary bytes are copied (random here, NaN patterns included); the
        # codes' fp32 product rounds to bf16 against one rounding from double
        np.testing.assert_array_equal(got[:, 448:], ref[:, 448:])
        P.check_bf16(got[:, :448], ref[:, :448], f"read case {case}")
    else:
        np.testing.assert_array_equal(got, ref, err_msg=f"read case {case}")
