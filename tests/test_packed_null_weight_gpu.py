"""The packed entry points through the C-ABI with a NULL weight for a group
that has no heads (the header allows it: q_weight may be NULL when Hq = 0,
k_weight when Hk = 0), and a NULL cos/sin cache with no rotary dims.  The
kernels load both weight vectors unconditionally and borrow the other
group's pointer for an empty group, so these calls must match the oracle and
equal, bit for bit, the same call made with a real tensor in the NULL's
place.  Needs an MI355X."""

import ctypes

import numpy as np
import pytest
import torch

import fp8_kv_cache_slot_amd as K
import oracle as O
from fp8_kv_cache_slot_amd import inputs as I
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _case(seed, T, hq, hk, hv, D, R, dtype):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    qkv = torch.randn((T, (hq + hk + hv) * D), generator=g, device=DEV).to(dtype)
    w = (torch.rand(D, generator=g, device=DEV) + 0.5).to(dtype)
    cs = (I.cos_sin_cache(512, R, device=DEV) if R else
          torch.zeros((512, 0), dtype=torch.float32, device=DEV))
    pos = torch.randint(0, 512, (T,), generator=g, device=DEV)
    return qkv, w, cs, pos


def _oracle(qkv, hq, hk, hv, D, R, neox, fp16, w, cs, pos):
    ref = _bits16(qkv).copy()
    O.qk_norm_rope_packed_ex(ref, hq, hk, hv, D, R, int(neox), int(fp16), 1e-6,
                             _bits16(w), _bits16(w), I.bits(cs).copy(), I.bits(pos))
    return ref


@pytest.mark.parametrize("hq,hk", [(16, 0), (0, 8)], ids=["k_null", "q_null"])
def test_guarded_entry_null_weight(hq, hk):
    T, hv, D = 300, 8, 128
    qkv, w, cs, pos = _case(31 + hq, T, hq, hk, hv, D, D, torch.bfloat16)
    print(f"guarded entry: T={T} heads={hq},{hk},{hv}", flush=True)
    got = qkv.clone()
    L = K.lib()
    qw = w.data_ptr() if hq else None
    kw = w.data_ptr() if hk else None
    st = L.qk_norm_rope_packed(got.data_ptr(), T, hq, hk, hv, D, 1e-6, qw, kw,
                               cs.data_ptr(), 1, pos.data_ptr(), -1, cs.shape[0],
                               _stream())
    assert st == 0, L.fp8kv_status_string(st).decode()
    same = qkv.clone()
    K.qk_norm_rope_packed(same, hq, hk, hv, D, 1e-6, w, w, cs, True, pos)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), same.view(torch.int16))
    ref = _oracle(qkv, hq, hk, hv, D, D, True, False, w, cs, pos)
    n = (hq + hk) * D
    out = _bits16(got)
    np.testing.assert_array_equal(out[:, n:], _bits16(qkv)[:, n:])
    P.check_bf16(out[:, :n], ref[:, :n], "guarded entry, NULL weight")


@pytest.mark.parametrize("hq,hk,D,R,neox,dtype", [
    (16, 0, 64, 32, False, torch.float16),
    (0, 8, 256, 128, True, torch.bfloat16),
    (5, 0, 128, 0, True, torch.bfloat16),
], ids=["d64_k_null", "d256_q_null", "d128_no_rotary_k_null"])
def test_variants_entry_null_weight(hq, hk, D, R, neox, dtype):
    T, hv = 257, 3
    qkv, w, cs, pos = _case(41 + D + R, T, hq, hk, hv, D, R, dtype)
    fp16 = dtype == torch.float16
    print(f"variants entry: T={T} heads={hq},{hk},{hv} D={D} R={R} neox={neox} "
          f"{dtype}", flush=True)
    got = qkv.clone()
    L = K.lib()
    qw = w.data_ptr() if hq else None
    kw = w.data_ptr() if hk else None
    st = L.qk_norm_rope_packed_ex(got.data_ptr(), T, hq, hk, hv, D, 1e-6, qw, kw,
                                  cs.data_ptr() if R else None, int(neox),
                                  pos.data_ptr(), R, int(fp16), cs.shape[0],
                                  _stream())
    assert st == 0, L.fp8kv_status_string(st).decode()
    same = qkv.clone()
    K.qk_norm_rope_packed_ex(same, hq, hk, hv, D, 1e-6, w, w, cs, neox, pos,
                             rotary_dim=R)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), same.view(torch.int16))
    ref = _oracle(qkv, hq, hk, hv, D, R, neox, fp16, w, cs, pos)
    n = (hq + hk) * D
    out = _bits16(got)
    np.testing.assert_array_equal(out[:, n:], _bits16(qkv)[:, n:])
    chk = P.check_fp16 if fp16 else P.check_bf16
    chk(out[:, :n], ref[:, :n], "variants entry, NULL weight")
