"""Every output buffer placed inside a larger allocation with guard bytes on
both sides: each entry point writes exactly its own bytes (the guards keep
their pattern) and gives bit-identical results to the same call on a buffer
of its own."""

import pytest
import torch

import fp8_kv_cache_slot_amd as K
from fp8_kv_cache_slot_amd import inputs as I

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GUARD_BYTES = 4096


def _guarded(t):
    """A copy of contiguous tensor t inside a buffer with GUARD_BYTES of a
    fixed pattern before and after it.  Returns (buffer, view)."""
    nb = t.numel() * t.element_size()
    g = torch.Generator(device=DEV)
    g.manual_seed(nb % 9973)
    buf = torch.randint(0, 256, (nb + 2 * GUARD_BYTES,), dtype=torch.uint8,
                        generator=g, device=DEV)
    view = buf[GUARD_BYTES:GUARD_BYTES + nb].view(t.dtype).view(t.shape)
    view.copy_(t)
    return buf, view


def _guards(buf):
    return torch.cat([buf[:GUARD_BYTES], buf[-GUARD_BYTES:]]).clone()


@pytest.fixture
def tiling():
    """Select a prologue tiling for the test (every call through it) and
    restore the defaults afterwards."""
    def use(shape):
        K.set_dispatch_threshold(0 if shape else -1)
        K.set_tiling(*(shape or (0, 0)))
    yield use
    K.set_dispatch_threshold(-1)
    K.set_tiling(0, 0)


# default dispatch (one head per one-wave block) and a multi-head shape
SHAPES = [None, (4, 2), (8, 4)]
SHAPE_IDS = ["default", "4x2", "8x4"]


@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_prologue(name, shape, tiling):
    tiling(shape)
    w = I.DSV4_WORKLOADS[name]
    x = I.make_dsv4(w, DEV)
    q0, c0, s0 = x["q"].clone(), x["kv_cache"].clone(), x["kv_scale"].clone()
    K.qnorm_rope_kv_quant_insert(q0, x["kv"], x["q_weight"], x["kv_weight"],
                                 x["cos_sin_cache"], x["positions"],
                                 x["slot_mapping"], c0, s0, x["eps"])
    bq, q = _guarded(x["q"])
    bc, c = _guarded(x["kv_cache"])
    bs, s = _guarded(x["kv_scale"])
    before = [_guards(b) for b in (bq, bc, bs)]
    K.qnorm_rope_kv_quant_insert(q, x["kv"], x["q_weight"], x["kv_weight"],
                                 x["cos_sin_cache"], x["positions"],
                                 x["slot_mapping"], c, s, x["eps"])
    torch.cuda.synchronize()
    for b, g in zip((bq, bc, bs), before):
        assert torch.equal(_guards(b), g)
    assert torch.equal(q, q0) and torch.equal(c, c0) and torch.equal(s, s0)


@pytest.mark.parametrize("shape", [None, (4, 2)], ids=["default", "4x2"])
def test_scalar_scale_prologue(shape, tiling):
    tiling(shape)
    w = I.DSV4_WORKLOADS["decode"]
    x = I.make_dsv4(w, DEV)
    sc = torch.tensor([0.02], device=DEV)
    q0, c0 = x["q"].clone(), x["kv_cache"].clone()
    K.qnorm_rope_kv_quant_insert_scalar_scale(
        q0, x["kv"], x["q_weight"], x["kv_weight"], x["cos_sin_cache"],
        x["positions"], x["slot_mapping"], c0, sc, x["eps"])
    bq, q = _guarded(x["q"])
    bc, c = _guarded(x["kv_cache"])
    before = [_guards(b) for b in (bq, bc)]
    K.qnorm_rope_kv_quant_insert_scalar_scale(
        q, x["kv"], x["q_weight"], x["kv_weight"], x["cos_sin_cache"],
        x["positions"], x["slot_mapping"], c, sc, x["eps"])
    torch.cuda.synchronize()
    for b, g in zip((bq, bc), before):
        assert torch.equal(_guards(b), g)
    assert torch.equal(q, q0) and torch.equal(c, c0)


@pytest.mark.parametrize("name", ["packed_t1", "packed_t17", "packed_t8192"])
def test_packed(name):
    pw = I.PACKED_WORKLOADS[name]
    x = I.make_packed(pw, DEV)

    def run(qkv):
        K.qk_norm_rope_packed(qkv, pw.num_heads_q, pw.num_heads_k, pw.num_heads_v,
                              pw.head_dim, pw.eps, x["q_weight"], x["k_weight"],
                              x["cos_sin_cache"], True, x["position_ids"])
    ref = x["qkv"].clone()
    run(ref)
    b, v = _guarded(x["qkv"])
    before = _guards(b)
    run(v)
    torch.cuda.synchronize()
    assert torch.equal(_guards(b), before)
    assert torch.equal(v, ref)


@pytest.mark.parametrize("D,R,neox,dtype", [(64, 64, False, torch.float16),
                                            (256, 128, True, torch.bfloat16)])
def test_packed_ex(D, R, neox, dtype):
    g = torch.Generator(device=DEV)
    g.manual_seed(D + R)
    T, hq, hk, hv = 33, 5, 3, 2
    qkv = torch.randn((T, (hq + hk + hv) * D), generator=g, device=DEV).to(dtype)
    w = (torch.rand(D, generator=g, device=DEV) + 0.5).to(dtype)
    cs = I.cos_sin_cache(64, R, device=DEV)
    pos = torch.randint(0, 64, (T,), generator=g, device=DEV)

    def run(t):
        K.qk_norm_rope_packed_ex(t, hq, hk, hv, D, 1e-6, w, w, cs, neox, pos,
                                 rotary_dim=R)
    ref = qkv.clone()
    run(ref)
    b, v = _guarded(qkv)
    before = _guards(b)
    run(v)
    torch.cuda.synchronize()
    assert torch.equal(_guards(b), before)
    assert torch.equal(v, ref)


def test_read_side_and_stages():
    w = I.DSV4_WORKLOADS["decode"]
    x = I.make_dsv4(w, DEV)
    cache, scale = x["kv_cache"].clone(), x["kv_scale"].clone()
    K.qnorm_rope_kv_quant_insert(x["q"].clone(), x["kv"], x["q_weight"],
                                 x["kv_weight"], x["cos_sin_cache"], x["positions"],
                                 x["slot_mapping"], cache, scale, x["eps"])
    slots = x["slot_mapping"]
    ref = K.kv_cache_gather_dequant(cache, scale, slots)
    b, out = _guarded(torch.zeros_like(ref))
    before = _guards(b)
    K.kv_cache_gather_dequant(cache, scale, slots, out=out)
    torch.cuda.synchronize()
    assert torch.equal(_guards(b), before)
    assert torch.equal(out, ref)
    # the block-table read side into a guarded output: the same rows
    table = torch.arange(16, dtype=torch.int32, device=DEV).view(2, 8)
    lens = torch.tensor([300, 170], dtype=torch.int32, device=DEV)
    offs = torch.tensor([0, 300], dtype=torch.int64, device=DEV)
    pref = torch.zeros((470, 512), dtype=torch.bfloat16, device=DEV)
    K.kv_cache_gather_dequant_paged(cache, scale, table, lens, offs, pref)
    b, pout = _guarded(torch.zeros_like(pref))
    before = _guards(b)
    K.kv_cache_gather_dequant_paged(cache, scale, table, lens, offs, pout)
    torch.cuda.synchronize()
    assert torch.equal(_guards(b), before)
    assert torch.equal(pout, pref)
    # the scalar-scale block-table read side, the same way
    sc = torch.tensor([0.0173], dtype=torch.float32, device=DEV)
    sref = torch.zeros((470, 512), dtype=torch.bfloat16, device=DEV)
    K.kv_cache_gather_dequant_paged_scalar_scale(cache, sc, table, lens, offs, sref)
    b, sout = _guarded(torch.zeros_like(sref))
    before = _guards(b)
    K.kv_cache_gather_dequant_paged_scalar_scale(cache, sc, table, lens, offs, sout)
    torch.cuda.synchronize()
    assert torch.equal(_guards(b), before)
    assert torch.equal(sout.view(torch.int16), sref.view(torch.int16))
    # a separate RMSNorm stage into a guarded output
    nref = K.rms_norm_rows(x["kv"], x["kv_weight"], x["eps"])
    b, nout = _guarded(torch.zeros_like(nref))
    before = _guards(b)
    K.rms_norm_rows(x["kv"], x["kv_weight"], x["eps"], out=nout)
    torch.cuda.synchronize()
    assert torch.equal(_guards(b), before)
    assert torch.equal(nout, nref)
