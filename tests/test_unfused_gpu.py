"""Parity of the separate-stage kernels (the unfused baseline) with the
oracle's stage functions, each on its own seeded inputs, and of the composed
five-launch pipeline stage by stage.  Needs an MI355X."""

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


def _host(x):
    return {k: (I.bits(v).copy() if isinstance(v, torch.Tensor) else v)
            for k, v in x.items()}


# 262147 rows: 131074 one-wave blocks of two rows, a launch that takes the
# occupancy cap
@pytest.mark.parametrize("rows", [1, 7, 8, 9, 1000, 4099, 262147])
def test_rms_norm_rows(rows):
    g = torch.Generator(device=DEV)
    g.manual_seed(60 + rows)
    x = (torch.randn((rows, 512), generator=g, device=DEV) *
         torch.where(torch.rand((rows, 512), generator=g, device=DEV) < 0.01, 50.0, 1.0)
         ).to(torch.bfloat16)
    w = (torch.rand(512, generator=g, device=DEV) + 0.5).to(torch.bfloat16)
    out = K.rms_norm_rows(x, w, 1e-6)
    inplace = x.clone()
    K.rms_norm_rows(inplace, w, 1e-6, out=inplace)
    torch.cuda.synchronize()
    ref = O.rms_norm_rows(I.bits(x), I.bits(w), 1e-6)
    P.check_bf16(I.bits(out), ref, "rms_norm_rows")
    assert torch.equal(out, inplace)


@pytest.mark.parametrize("T,R", [(1, 1), (3, 5), (17, 64), (257, 3)])
def test_rope_rows(T, R):
    g = torch.Generator(device=DEV)
    g.manual_seed(70 + T * R)
    x = (torch.randn((T, R, 512), generator=g, device=DEV) * 2).to(torch.bfloat16)
    cs = I.cos_sin_cache(1000, 64, device=DEV)
    pos = torch.randint(0, 1000, (T,), generator=g, device=DEV)
    got = x.clone()
    K.rope_rows(got, cs, pos)
    torch.cuda.synchronize()
    ref = I.bits(x).copy()
    O.rope_rows(ref, I.bits(cs), I.bits(pos))
    assert torch.equal(got[..., :448], x[..., :448])
    P.check_bf16(I.bits(got), ref, "rope_rows")
    # a token with an out-of-range position is left as it was
    pos[0] = 1000
    got = x.clone()
    K.rope_rows(got, cs, pos)
    torch.cuda.synchronize()
    assert torch.equal(got[0], x[0])


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_kv_quant_insert(name):
    # input rows: the oracle's own normalised and rotated bf16 KV rows
    w = I.DSV4_WORKLOADS[name]
    h = _host(I.make_dsv4(w, "cpu"))
    kv = O.rms_norm_rows(h["kv"], h["kv_weight"], h["eps"])
    O.rope_rows(kv.reshape(-1, 1, 512), h["cos_sin_cache"], h["positions"])
    ref_c, ref_s = h["kv_cache"].copy(), h["kv_scale"].copy()
    O.kv_quant_insert(kv, h["slot_mapping"], ref_c, ref_s)
    cache = torch.from_numpy(h["kv_cache"]).to(DEV)
    scale = torch.from_numpy(h["kv_scale"]).to(DEV)
    K.kv_quant_insert(I.from_bits(kv, DEV), torch.from_numpy(h["slot_mapping"]).to(DEV),
                      cache, scale)
    torch.cuda.synchronize()
    # bf16 inputs are exact in fp32: exponents and codes must be bit-exact
    np.testing.assert_array_equal(I.bits(cache), ref_c)
    np.testing.assert_array_equal(I.bits(scale), ref_s)


def test_golden_example_through_the_stages():
    g = golden_case.load()
    h = golden_case.inputs(g)
    exp = golden_case.expected(g)
    x = {k: (I.from_bits(v, DEV) if isinstance(v, np.ndarray) else v)
         for k, v in h.items()}
    K.unfused_prologue(x["q"], x["kv"], x["q_weight"], x["kv_weight"],
                       x["cos_sin_cache"], x["positions"], x["slot_mapping"],
                       x["kv_cache"], x["kv_scale"], x["eps"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(I.bits(x["q"]), exp["q"])
    np.testing.assert_array_equal(I.bits(x["kv_cache"]), exp["kv_cache"])
    np.testing.assert_array_equal(I.bits(x["kv_scale"]), exp["kv_scale"])


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_pipeline_stage_by_stage(name):
    # Each of the five launches is compared with the oracle's stage on the
    # same input bytes: the norms on q and kv, each rotation on the GPU's own
    # normalised rows, quantise+insert on the GPU's own rotated KV rows (bit
    # for bit: bf16 inputs are exact in fp32).  The GPU and oracle
    # compositions are not compared element by element: where a norm's bf16
    # result is one step from the oracle's, the rotation carries that step
    # into its partner's output and the quantiser may pick the next code.
    # The composed binding gives the same bytes as the launches one by one.
    w = I.DSV4_WORKLOADS[name]
    x = I.make_dsv4(w, DEV)
    h = _host(x)
    cs, pos = h["cos_sin_cache"], h["positions"]
    gq = x["q"].clone()
    K.rms_norm_rows(gq, x["q_weight"], x["eps"], out=gq)
    work = torch.empty((w.num_tokens, 512), dtype=torch.bfloat16, device=DEV)
    K.rms_norm_rows(x["kv"], x["kv_weight"], x["eps"], out=work)
    torch.cuda.synchronize()
    q_mid, kv_mid = I.bits(gq), I.bits(work)
    P.check_bf16(q_mid, O.rms_norm_rows(h["q"], h["q_weight"], h["eps"]), name + " q norm")
    P.check_bf16(kv_mid, O.rms_norm_rows(h["kv"], h["kv_weight"], h["eps"]),
                 name + " kv norm")
    K.rope_rows(gq, x["cos_sin_cache"], x["positions"])
    K.rope_rows(work.view(w.num_tokens, 1, 512), x["cos_sin_cache"], x["positions"])
    torch.cuda.synchronize()
    ref = q_mid.copy()
    O.rope_rows(ref, cs, pos)
    P.check_bf16(I.bits(gq), ref, name + " q rope")
    ref = kv_mid.copy()
    O.rope_rows(ref.reshape(-1, 1, 512), cs, pos)
    kv_rot = I.bits(work)
    P.check_bf16(kv_rot, ref, name + " kv rope")
    gc, gs = x["kv_cache"].clone(), x["kv_scale"].clone()
    K.kv_quant_insert(work, x["slot_mapping"], gc, gs)
    torch.cuda.synchronize()
    ref_c, ref_s = h["kv_cache"].copy(), h["kv_scale"].copy()
    O.kv_quant_insert(kv_rot.copy(), h["slot_mapping"], ref_c, ref_s)
    np.testing.assert_array_equal(I.bits(gc), ref_c)
    np.testing.assert_array_equal(I.bits(gs), ref_s)
    v = P.valid_slots(h["slot_mapping"], w.num_pages * 64)
    P.check_untouched(I.bits(gc), I.bits(gs), h["slot_mapping"][v],
                      I.CACHE_CANARY, I.SCALE_CANARY, name)
    q2, c2, s2 = x["q"].clone(), x["kv_cache"].clone(), x["kv_scale"].clone()
    K.unfused_prologue(q2, x["kv"], x["q_weight"], x["kv_weight"],
                       x["cos_sin_cache"], x["positions"], x["slot_mapping"],
                       c2, s2, x["eps"])
    torch.cuda.synchronize()
    assert torch.equal(q2, gq) and torch.equal(c2, gc) and torch.equal(s2, gs)
    assert np.array_equal(I.bits(x["kv"]), h["kv"])   # kv is only read
