"""Parity of the packed operator's separate stages (RMSNorm of a group of
heads into its own output, NeoX RoPE in place: the four-launch baseline of
InfiniOps PR #1019 "Benchmark / Performance Impact") with the oracle's stage
functions, each on its own input bytes, and of the four composed launches
stage by stage.  Needs an MI355X."""

import numpy as np
import pytest
import torch

import fp8_kv_cache_slot_amd as K
import oracle as O
from fp8_kv_cache_slot_amd import inputs as I
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D = 128


def _packed(T, hq, hk, hv, seed):
    return I.make_packed(I.PackedWorkload("p", T, hq, hk, hv, seed=seed), DEV)


@pytest.mark.parametrize("T,heads", [(1, (16, 8, 8)), (17, (16, 8, 8)),
                                     (333, (5, 3, 1)), (8192, (16, 8, 8)),
                                     (40, (1, 2, 0)), (9, (7, 0, 2))])
def test_rms_norm_heads(T, heads):
    hq, hk, hv = heads
    x = _packed(T, hq, hk, hv, seed=700 + T + hq)
    h = I.bits(x["qkv"])
    for first, n, w in ((0, hq, x["q_weight"]), (hq, hk, x["k_weight"])):
        out = torch.full((T, n, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        K.rms_norm_heads(x["qkv"], first, n, D, w, out, x["eps"])
        torch.cuda.synchronize()
        ref = O.rms_norm_heads(h, first, n, D, I.bits(w), x["eps"])
        P.check_bf16(I.bits(out), ref, f"rms_norm_heads T={T} heads {first}+{n}")
    # the input is only read
    assert np.array_equal(I.bits(x["qkv"]), h)


def test_rms_norm_heads_in_place():
    x = _packed(50, 6, 2, 0, seed=711)
    heads = x["qkv"].view(50, 8, D)
    a = torch.empty_like(heads)
    K.rms_norm_heads(x["qkv"], 0, 8, D, x["q_weight"], a, x["eps"])
    K.rms_norm_heads(x["qkv"], 0, 8, D, x["q_weight"], heads, x["eps"])
    torch.cuda.synchronize()
    assert torch.equal(a, heads)


@pytest.mark.parametrize("T,H", [(1, 1), (5, 3), (17, 16), (1000, 8), (4097, 5)])
def test_rope_neox_heads(T, H):
    g = torch.Generator(device=DEV)
    g.manual_seed(720 + T * H)
    x = (torch.randn((T, H, D), generator=g, device=DEV) * 2).to(torch.bfloat16)
    cs = I.cos_sin_cache(1000, D, device=DEV)
    pos = torch.randint(0, 1000, (T,), generator=g, device=DEV)
    got = x.clone()
    K.rope_neox_heads(got, cs, pos)
    torch.cuda.synchronize()
    ref = I.bits(x).copy()
    O.rope_neox_heads(ref, I.bits(cs), I.bits(pos))
    P.check_bf16(I.bits(got), ref, f"rope_neox_heads T={T} H={H}")
    # a token with an out-of-range position is left as it was
    pos[0] = 1000
    pos[-1] = -3
    got = x.clone()
    K.rope_neox_heads(got, cs, pos)
    torch.cuda.synchronize()
    assert torch.equal(got[0], x[0]) and torch.equal(got[-1], x[-1])


@pytest.mark.parametrize("name", ["packed_t17", "packed_t1024", "packed_t8192"])
def test_four_launches_stage_by_stage(name):
    # Each launch is compared with the oracle's stage on the same input bytes:
    # the norm on qkv, the rotation on the GPU's own normalised heads.  (The
    # GPU and oracle compositions cannot be compared element by element: where
    # the norm's bf16 result is one step from the oracle's, about 1e-5 of the
    # values, the rotation carries that step into its partner's output.)  The
    # composed binding gives the same bytes as the launches one by one.
    w = I.PACKED_WORKLOADS[name]
    x = I.make_packed(w, DEV)
    before = x["qkv"].clone()
    T, hq, hk = w.num_tokens, w.num_heads_q, w.num_heads_k
    h = I.bits(x["qkv"])
    cs, pos = I.bits(x["cos_sin_cache"]), I.bits(x["position_ids"])
    for first, n, wt, tag in ((0, hq, x["q_weight"], "q"), (hq, hk, x["k_weight"], "k")):
        normed = torch.empty((T, n, D), dtype=torch.bfloat16, device=DEV)
        K.rms_norm_heads(x["qkv"], first, n, D, wt, normed, w.eps)
        torch.cuda.synchronize()
        mid = I.bits(normed)
        P.check_bf16(mid, O.rms_norm_heads(h, first, n, D, I.bits(wt), w.eps),
                     f"{name} {tag} norm")
        K.rope_neox_heads(normed, x["cos_sin_cache"], x["position_ids"])
        torch.cuda.synchronize()
        ref = mid.copy()
        O.rope_neox_heads(ref, cs, pos)
        P.check_bf16(I.bits(normed), ref, f"{name} {tag} rope")
        if tag == "q":
            q_steps = normed
        else:
            k_steps = normed
    q, k = K.unfused_qk_norm_rope_packed(
        x["qkv"], hq, hk, w.num_heads_v, w.head_dim, w.eps, x["q_weight"],
        x["k_weight"], x["cos_sin_cache"], x["position_ids"])
    torch.cuda.synchronize()
    assert torch.equal(q, q_steps) and torch.equal(k, k_steps)
    assert torch.equal(x["qkv"], before)   # qkv is only read


def test_rejects():
    x = _packed(4, 2, 2, 0, seed=730)
    out = torch.empty((4, 2, D), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(K.Fp8kvError):   # eps must be finite and >= 0
        K.rms_norm_heads(x["qkv"], 0, 2, D, x["q_weight"], out, -1.0)
    L = K.lib()
    p = x["qkv"].data_ptr()
    # head_dim other than 128; a stride shorter than the heads; misaligned
    assert L.rms_norm_heads(p, 512, out.data_ptr(), x["q_weight"].data_ptr(), 4, 2,
                            64, 1e-6, None) == 3
    assert L.rms_norm_heads(p, 128, out.data_ptr(), x["q_weight"].data_ptr(), 4, 2,
                            128, 1e-6, None) == 2
    assert L.rms_norm_heads(p + 2, 512, out.data_ptr(), x["q_weight"].data_ptr(), 4,
                            2, 128, 1e-6, None) == 4
    assert L.rope_neox_heads(out.data_ptr(), x["cos_sin_cache"].data_ptr(),
                             x["position_ids"].data_ptr(), 4, 2, 128, 0, None) == 2
