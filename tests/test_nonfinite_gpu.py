"""A NaN or an infinity in q, kv or qkv stays in its own head: every other
head, token and cache row comes out as the oracle gives it for the same
inputs with that element finite, unwritten cache rows keep their canaries,
and V elements (never read) keep their bits whatever their values.  A kernel
whose reductions or partner exchanges reached across heads, or whose shared
per-block data mixed tokens, would spread the NaN.  The poisoned heads
themselves are unspecified and are not compared.  Needs an MI355X."""

import numpy as np
import pytest
import torch

import fp8_kv_cache_slot_amd as K
import oracle as O
from fp8_kv_cache_slot_amd import inputs as I
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SMALL, TILED = 2 ** 63 - 1, 0
NAN, INF = float("nan"), float("inf")


@pytest.fixture(autouse=True)
def _restore_knobs():
    yield
    K.set_dispatch_threshold(-1)
    K.set_tiling(0, 0)


def _host(x):
    return {k: (I.bits(v) if isinstance(v, torch.Tensor) else v)
            for k, v in x.items()}


# (token, head, dim, value): dims 449 and 500 sit in the rotary lanes
Q_POISON = [(5, 3, 17, NAN), (9, 0, 500, INF), (9, 6, 449, -INF), (20, 7, 0, NAN)]
# (token, dim, value)
KV_POISON = [(11, 200, NAN), (13, 460, -INF), (17, 0, INF)]


@pytest.mark.parametrize("threshold,tiling",
                         [(SMALL, (0, 0)), (TILED, (0, 0)), (TILED, (4, 2)),
                          (TILED, (8, 4))],
                         ids=["small", "tiled", "tiled-4x2", "tiled-8x4"])
def test_prologue(threshold, tiling):
    T, H = 24, 8
    x = I.make_dsv4(I.custom_dsv4(T, H, seed=4100, num_pages=1), DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(4101)
    x["slot_mapping"] = torch.randperm(64, generator=g, device=DEV)[:T].to(torch.int64)
    x["slot_mapping"][2] = -1
    h = _host(x)
    ref = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in h.items()}
    O.qnorm_rope_kv_quant_insert(ref["q"], ref["kv"], ref["q_weight"], ref["kv_weight"],
                                 ref["cos_sin_cache"], ref["positions"],
                                 ref["slot_mapping"], ref["kv_cache"], ref["kv_scale"],
                                 ref["eps"])

    q, kv = x["q"].clone(), x["kv"].clone()
    for t, hh, d, v in Q_POISON:
        q[t, hh, d] = v
    for t, d, v in KV_POISON:
        kv[t, d] = v
    cache, scale = x["kv_cache"].clone(), x["kv_scale"].clone()
    K.set_tiling(*tiling)
    K.set_dispatch_threshold(threshold)
    K.qnorm_rope_kv_quant_insert(q, kv, x["q_weight"], x["kv_weight"],
                                 x["cos_sin_cache"], x["positions"], x["slot_mapping"],
                                 cache, scale, x["eps"])
    torch.cuda.synchronize()

    qg, qr = I.bits(q).copy(), ref["q"].copy()
    for t, hh, _, _ in Q_POISON:
        qg[t, hh] = 0
        qr[t, hh] = 0
    P.check_bf16(qg, qr, "q heads other than the poisoned ones")

    v = P.valid_slots(h["slot_mapping"], 64)
    assert all(v[t] for t, _, _ in KV_POISON)
    keep = v.copy()
    keep[[t for t, _, _ in KV_POISON]] = False
    y = O.kv_normalised(h["kv"][keep].copy(), h["kv_weight"], h["cos_sin_cache"],
                        h["positions"][keep].copy(), h["eps"])
    cg, sg = I.bits(cache), I.bits(scale)
    P.check_cache(cg, sg, ref["kv_cache"], ref["kv_scale"], h["slot_mapping"][keep], y,
                  I.CACHE_CANARY, I.SCALE_CANARY, "rows of the finite KV heads")
    P.check_untouched(cg, sg, h["slot_mapping"][v], I.CACHE_CANARY, I.SCALE_CANARY,
                      "rows no token writes")


def _bits16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _packed_case(T, hq, hk, hv, D, R, neox, dtype, seed, poison, guarded):
    """poison: (token, head, dim, value) over all Hq + Hk + Hv heads."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    qkv = torch.randn((T, (hq + hk + hv) * D), generator=g, device=DEV).to(dtype)
    qw = (torch.rand(D, generator=g, device=DEV) + 0.5).to(dtype)
    kw = (torch.rand(D, generator=g, device=DEV) + 0.5).to(dtype)
    cs = I.cos_sin_cache(4096, R, device=DEV)
    pos = torch.randint(0, 4096, (T,), generator=g, device=DEV)
    ref = _bits16(qkv).copy()
    O.qk_norm_rope_packed_ex(ref, hq, hk, hv, D, R, int(neox), int(dtype == torch.float16),
                             1e-6, _bits16(qw), _bits16(kw), I.bits(cs).copy(), I.bits(pos))
    bad = qkv.clone()
    for t, hh, d, v in poison:
        bad[t, hh * D + d] = v
    given = _bits16(bad).copy()
    if guarded:
        K.qk_norm_rope_packed(bad, hq, hk, hv, D, 1e-6, qw, kw, cs, True, pos)
    else:
        K.qk_norm_rope_packed_ex(bad, hq, hk, hv, D, 1e-6, qw, kw, cs, neox, pos,
                                 rotary_dim=R)
    torch.cuda.synchronize()
    got = _bits16(bad).copy()
    n = (hq + hk) * D
    np.testing.assert_array_equal(got[:, n:], given[:, n:],
                                  err_msg="V changed (a NaN or infinity there included)")
    for t, hh, _, _ in poison:
        if hh < hq + hk:
            got[t, hh * D:(hh + 1) * D] = 0
            ref[t, hh * D:(hh + 1) * D] = 0
    chk = P.check_fp16 if dtype == torch.float16 else P.check_bf16
    chk(got[:, :n], ref[:, :n], "Q/K heads other than the poisoned ones")


# 16/8/8 heads: Q heads 0..15, K heads 16..23, V heads 24..31
POISON = [(4, 2, 10, NAN), (7, 21, 100, INF), (7, 21, 101, -INF), (12, 27, 5, NAN),
          (20, 0, 0, NAN), (21, 23, 3, INF)]


@pytest.mark.parametrize("T", [33, 8197])
def test_packed(T):
    _packed_case(T, 16, 8, 8, 128, 128, True, torch.bfloat16, 4200 + T, POISON, True)


# every block form of the variants kernel (16/8/8 heads: one wave per token at
# D=64, two at D=128, four at D=256): one-wave blocks (interleaved fp16, and
# any launch above 8192 waves), four one-wave tokens per block (NeoX), two per
# block (interleaved bf16), a token's waves in one block
VARIANTS = [(37, 64, 64, False, torch.float16), (8200, 64, 32, False, torch.bfloat16),
            (37, 64, 32, True, torch.bfloat16), (37, 64, 64, False, torch.bfloat16),
            (37, 128, 64, False, torch.bfloat16), (37, 256, 128, True, torch.bfloat16),
            (37, 256, 208, True, torch.float16)]


@pytest.mark.parametrize("T,D,R,neox,dtype", VARIANTS,
                         ids=[f"T{c[0]}-D{c[1]}-R{c[2]}-{'neox' if c[3] else 'inter'}-"
                              f"{'f16' if c[4] == torch.float16 else 'bf16'}"
                              for c in VARIANTS])
def test_packed_variants(T, D, R, neox, dtype):
    poison = [(t, hh, d * D // 128, v) for t, hh, d, v in POISON]
    _packed_case(T, 16, 8, 8, D, R, neox, dtype, 4300 + D + R, poison, False)
