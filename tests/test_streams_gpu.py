"""Stream semantics of the entry points on the GPU: every call is enqueued on
the stream it is given (torch's current stream when none is given), ordered
after earlier work on that stream and before later work, with no
synchronisation of its own; calls on two streams over independent buffers
give the results they give alone."""

import pytest
import torch

import fp8_kv_cache_slot_amd as K
from fp8_kv_cache_slot_amd import inputs as I

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _prologue(x, q, cache, scale, stream=None):
    K.qnorm_rope_kv_quant_insert(q, x["kv"], x["q_weight"], x["kv_weight"],
                                 x["cos_sin_cache"], x["positions"], x["slot_mapping"],
                                 cache, scale, x["eps"], stream=stream)


def _packed(px, pw, qkv, stream=None):
    K.qk_norm_rope_packed(qkv, pw.num_heads_q, pw.num_heads_k, pw.num_heads_v,
                          pw.head_dim, pw.eps, px["q_weight"], px["k_weight"],
                          px["cos_sin_cache"], True, px["position_ids"], stream=stream)


def _reference(x):
    q, c, s = x["q"].clone(), x["kv_cache"].clone(), x["kv_scale"].clone()
    _prologue(x, q, c, s)
    torch.cuda.synchronize()
    return q, c, s


def test_explicit_context_and_raw_streams_agree():
    x = I.make_dsv4(I.DSV4_WORKLOADS["decode"], DEV)
    ref = _reference(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for how in ("argument", "context", "raw handle"):
        q, c, s = x["q"].clone(), x["kv_cache"].clone(), x["kv_scale"].clone()
        side.wait_stream(torch.cuda.current_stream())
        if how == "argument":
            _prologue(x, q, c, s, stream=side)
        elif how == "context":
            with torch.cuda.stream(side):
                _prologue(x, q, c, s)
        else:
            _prologue(x, q, c, s, stream=side.cuda_stream)
        side.synchronize()
        for got, want in zip((q, c, s), ref):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), how


def test_ordered_after_earlier_work_on_the_stream():
    # On a side stream: the inputs are produced by copies enqueued just
    # before the call (the q copy moves 64 MiB), the call follows, and the
    # results are copied out after it; only the side stream is waited for.
    # A call that ran anywhere but in that order would read stale inputs or
    # be read back unfinished.
    x = I.make_dsv4(I.DSV4_WORKLOADS["decode"], DEV)
    ref = _reference(x)
    q = torch.zeros_like(x["q"])
    cache = torch.zeros_like(x["kv_cache"])
    scale = torch.zeros_like(x["kv_scale"])
    out = [torch.empty_like(t) for t in (q, cache, scale)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        q.copy_(x["q"])
        cache.copy_(x["kv_cache"])
        scale.copy_(x["kv_scale"])
        _prologue(x, q, cache, scale)
        for o, t in zip(out, (q, cache, scale)):
            o.copy_(t)
    side.synchronize()
    for got, want in zip(out, ref):
        assert torch.equal(got.view(torch.uint8), want.view(torch.uint8))

    # the packed op the same way, 8192 tokens
    pw = I.PACKED_WORKLOADS["packed_t8192"]
    px = I.make_packed(pw, DEV)
    pref = px["qkv"].clone()
    _packed(px, pw, pref)
    qkv = torch.zeros_like(px["qkv"])
    pout = torch.empty_like(qkv)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        qkv.copy_(px["qkv"])
        _packed(px, pw, qkv)
        pout.copy_(qkv)
    side.synchronize()
    assert torch.equal(pout.view(torch.int16), pref.view(torch.int16))


def test_two_streams_at_once():
    # Independent buffers on two streams, enqueued interleaved: each result
    # equals the call's result alone.
    x = I.make_dsv4(I.DSV4_WORKLOADS["decode"], DEV)
    ref = _reference(x)
    pw = I.PACKED_WORKLOADS["packed_t8192"]
    px = I.make_packed(pw, DEV)
    pref = px["qkv"].clone()
    _packed(px, pw, pref)
    torch.cuda.synchronize()
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    runs = []
    for _ in range(4):
        q, c, s = x["q"].clone(), x["kv_cache"].clone(), x["kv_scale"].clone()
        qkv = px["qkv"].clone()
        runs.append(((q, c, s), qkv))
    torch.cuda.synchronize()
    for (q, c, s), qkv in runs:
        _prologue(x, q, c, s, stream=a)
        _packed(px, pw, qkv, stream=b)
    a.synchronize()
    b.synchronize()
    for (q, c, s), qkv in runs:
        for got, want in zip((q, c, s), ref):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8))
        assert torch.equal(qkv.view(torch.int16), pref.view(torch.int16))
