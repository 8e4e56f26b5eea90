"""The entry points under HIP graph capture: each call is captured once on
torch's capture stream and replayed several times, with eager work (input
resets) and a synchronisation between replays; every replay must equal the
eager result bit for bit.  The library enqueues kernels only (no allocation,
memset or synchronisation), which is what capture needs."""

import pytest
import torch

import fp8_kv_cache_slot_amd as K
from fp8_kv_cache_slot_amd import inputs as I

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                      # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_prologue(name):
    w = I.DSV4_WORKLOADS[name]
    x = I.make_dsv4(w, DEV)
    q, c, s = x["q"].clone(), x["kv_cache"].clone(), x["kv_scale"].clone()

    def run():
        K.qnorm_rope_kv_quant_insert(q, x["kv"], x["q_weight"], x["kv_weight"],
                                     x["cos_sin_cache"], x["positions"],
                                     x["slot_mapping"], c, s, x["eps"])
    run()
    ref = [t.clone() for t in (q, c, s)]
    g = _capture(run)
    for _ in range(REPLAYS):
        q.copy_(x["q"])
        c.copy_(x["kv_cache"])
        s.copy_(x["kv_scale"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((q, c, s), ref):
            assert torch.equal(got, want)


def test_packed_and_read_side():
    pw = I.PACKED_WORKLOADS["packed_t17"]
    px = I.make_packed(pw, DEV)
    qkv = px["qkv"].clone()
    w = I.DSV4_WORKLOADS["decode"]
    x = I.make_dsv4(w, DEV)
    cache, scale = x["kv_cache"].clone(), x["kv_scale"].clone()
    K.qnorm_rope_kv_quant_insert(x["q"].clone(), x["kv"], x["q_weight"],
                                 x["kv_weight"], x["cos_sin_cache"], x["positions"],
                                 x["slot_mapping"], cache, scale, x["eps"])
    out = torch.empty((w.num_tokens, 512), dtype=torch.bfloat16, device=DEV)
    table = torch.arange(w.num_pages, dtype=torch.int32, device=DEV).view(4, -1).contiguous()
    lens = torch.tensor([100, 0, 64, 3000], dtype=torch.int32, device=DEV)
    offs = torch.tensor([0, 100, 100, 164], dtype=torch.int64, device=DEV)
    pout = torch.empty((2000, 512), dtype=torch.bfloat16, device=DEV)
    sc = torch.tensor([0.0173], dtype=torch.float32, device=DEV)
    sout = torch.empty_like(out)
    spout = torch.empty_like(pout)

    def run():
        K.qk_norm_rope_packed(qkv, pw.num_heads_q, pw.num_heads_k, pw.num_heads_v,
                              pw.head_dim, pw.eps, px["q_weight"], px["k_weight"],
                              px["cos_sin_cache"], True, px["position_ids"])
        K.kv_cache_gather_dequant(cache, scale, x["slot_mapping"], out=out)
        K.kv_cache_gather_dequant_paged(cache, scale, table, lens, offs, pout)
        K.kv_cache_gather_dequant_scalar_scale(cache, sc, x["slot_mapping"], out=sout)
        K.kv_cache_gather_dequant_paged_scalar_scale(cache, sc, table, lens, offs,
                                                     spout)
    pout.zero_()
    spout.zero_()
    run()
    ref_qkv, ref_out, ref_pout = qkv.clone(), out.clone(), pout.clone()
    ref_sout, ref_spout = sout.clone(), spout.clone()
    g = _capture(run)
    for _ in range(REPLAYS):
        qkv.copy_(px["qkv"])
        out.zero_()
        pout.zero_()
        sout.zero_()
        spout.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(qkv, ref_qkv)
        assert torch.equal(out, ref_out)
        assert torch.equal(pout, ref_pout)
        assert torch.equal(sout.view(torch.int16), ref_sout.view(torch.int16))
        assert torch.equal(spout.view(torch.int16), ref_spout.view(torch.int16))


def test_capped_and_token_block_launches():
    # Launches large enough for the occupancy cap (their LDS request is a
    # launch parameter of the captured node): the packed kernel at 32771
    # tokens of 16/8/8 heads and the variants kernel at 131081 tokens of
    # head_dim 64, in one graph.
    pw = I.PackedWorkload("capped", 32771, seed=77)
    px = I.make_packed(pw, DEV)
    qkv = px["qkv"].clone()
    g0 = torch.Generator(device=DEV)
    g0.manual_seed(78)
    T = 131072 + 9
    ex_in = torch.randn((T, 32 * 64), generator=g0, device=DEV).to(torch.float16)
    ex = ex_in.clone()
    ew = (torch.rand(64, generator=g0, device=DEV) + 0.5).to(torch.float16)
    ecs = I.cos_sin_cache(4096, 64, device=DEV)
    epos = torch.randint(0, 4096, (T,), generator=g0, device=DEV)

    # and the variants kernel's token-block form (a small launch whose
    # tokens span several waves: head_dim 256, three blocks per token)
    sm_in = torch.randn((37, 112 * 256), generator=g0, device=DEV).to(torch.bfloat16)
    sm = sm_in.clone()
    sw = (torch.rand(256, generator=g0, device=DEV) + 0.5).to(torch.bfloat16)
    scs = I.cos_sin_cache(4096, 128, device=DEV)
    spos = torch.randint(0, 4096, (37,), generator=g0, device=DEV)

    # and four one-wave tokens per block (head_dim 64, NeoX, 37 tokens)
    fo_in = torch.randn((37, 32 * 64), generator=g0, device=DEV).to(torch.float16)
    fo = fo_in.clone()

    def run():
        K.qk_norm_rope_packed(qkv, pw.num_heads_q, pw.num_heads_k, pw.num_heads_v,
                              pw.head_dim, pw.eps, px["q_weight"], px["k_weight"],
                              px["cos_sin_cache"], True, px["position_ids"])
        K.qk_norm_rope_packed_ex(ex, 16, 8, 8, 64, 1e-6, ew, ew, ecs, False, epos)
        K.qk_norm_rope_packed_ex(sm, 100, 8, 4, 256, 1e-6, sw, sw, scs, True, spos,
                                 rotary_dim=128)
        K.qk_norm_rope_packed_ex(fo, 16, 8, 8, 64, 1e-6, ew, ew, ecs, True, spos)
    run()
    ref_qkv, ref_ex, ref_sm, ref_fo = qkv.clone(), ex.clone(), sm.clone(), fo.clone()
    g = _capture(run)
    for _ in range(REPLAYS):
        qkv.copy_(px["qkv"])
        ex.copy_(ex_in)
        sm.copy_(sm_in)
        fo.copy_(fo_in)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(qkv, ref_qkv)
        assert torch.equal(ex.view(torch.int16), ref_ex.view(torch.int16))
        assert torch.equal(sm.view(torch.int16), ref_sm.view(torch.int16))
        assert torch.equal(fo.view(torch.int16), ref_fo.view(torch.int16))
