"""Parity of the general packed Q/K norm + RoPE (head_dim 64/128/256, partial
rotary, NeoX or interleaved, bf16 or fp16) with the oracle's general form.
Needs an MI355X."""

import concurrent.futures as cf
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


def _bits(t):
    t = t.detach().contiguous().cpu()
    return t.view(torch.int16).numpy().view(np.uint16)


def _make(T, hq, hk, hv, D, R, dtype, seed, max_pos=4096):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    qkv = torch.randn((T, (hq + hk + hv) * D), generator=g, device=DEV).to(dtype)
    qw = (torch.rand(D, generator=g, device=DEV) + 0.5).to(dtype)
    kw = (torch.rand(D, generator=g, device=DEV) + 0.5).to(dtype)
    cs = I.cos_sin_cache(max_pos, max(R, 2), device=DEV)
    if R == 0:
        cs = torch.zeros((max_pos, 0), dtype=torch.float32, device=DEV)
    pos = torch.randint(0, max_pos, (T,), generator=g, device=DEV)
    return qkv, qw, kw, cs, pos


def _check(qkv, out, hq, hk, hv, D, R, neox, dtype, qw, kw, cs, pos, what):
    ref = _bits(qkv).copy()
    O.qk_norm_rope_packed_ex(ref, hq, hk, hv, D, R, int(neox),
                             int(dtype == torch.float16), 1e-6, _bits(qw),
                             _bits(kw), I.bits(cs).copy(), I.bits(pos))
    got = _bits(out)
    n = (hq + hk) * D
    np.testing.assert_array_equal(got[:, n:], _bits(qkv)[:, n:],
                                  err_msg=what + ": V changed")
    chk = P.check_fp16 if dtype == torch.float16 else P.check_bf16
    chk(got[:, :n], ref[:, :n], what)


CASES = [(D, R, neox, dt)
         for D in (64, 128, 256)
         for R in sorted({D, D // 2, 16 if D == 64 else 32})
         for neox in (True, False)
         for dt in (torch.bfloat16, torch.float16)]
# rotary widths whose NeoX partner distance (R/16 lanes) is not a power of two
CASES += [(128, 48, True, torch.bfloat16), (128, 48, False, torch.float16),
          (256, 80, True, torch.float16), (256, 208, True, torch.bfloat16)]


@pytest.mark.parametrize("D,R,neox,dtype", CASES,
                         ids=[f"D{c[0]}-R{c[1]}-{'neox' if c[2] else 'inter'}-"
                              f"{'f16' if c[3] == torch.float16 else 'bf16'}"
                              for c in CASES])
def test_variants(D, R, neox, dtype):
    for T, (hq, hk, hv) in [(1, (16, 8, 8)), (33, (5, 3, 1)), (7, (0, 4, 2))]:
        qkv, qw, kw, cs, pos = _make(T, hq, hk, hv, D, R, dtype, seed=D + R + T)
        out = qkv.clone()
        K.qk_norm_rope_packed_ex(out, hq, hk, hv, D, 1e-6, qw, kw, cs, neox, pos,
                                 rotary_dim=R)
        torch.cuda.synchronize()
        _check(qkv, out, hq, hk, hv, D, R, neox, dtype, qw, kw, cs, pos,
               f"D={D} R={R} neox={neox} {dtype} T={T} heads={hq},{hk},{hv}")


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("neox", [True, False], ids=["neox", "inter"])
def test_partial_access_in_the_last_wave_of_a_token(D, neox):
    # 7 + 6 = 13 Q/K heads: at every head width the token's last wave has an
    # access whose upper head slots do not exist (re-read head 0, not stored);
    # at D=128 and D=256 a token spans several waves.  777 tokens.
    hq, hk, hv, T, R = 7, 6, 3, 777, D // 2
    for dtype in (torch.bfloat16, torch.float16):
        qkv, qw, kw, cs, pos = _make(T, hq, hk, hv, D, R, dtype, seed=95 + D)
        out = qkv.clone()
        K.qk_norm_rope_packed_ex(out, hq, hk, hv, D, 1e-6, qw, kw, cs, neox, pos,
                                 rotary_dim=R)
        torch.cuda.synchronize()
        _check(qkv, out, hq, hk, hv, D, R, neox, dtype, qw, kw, cs, pos,
               f"D={D} R={R} neox={neox} {dtype} T={T} heads=7,6,3")


def test_no_rotation_and_large_token_count():
    qkv, qw, kw, cs, pos = _make(2048, 16, 8, 8, 128, 0, torch.float16, seed=91)
    out = qkv.clone()
    K.qk_norm_rope_packed_ex(out, 16, 8, 8, 128, 1e-6, qw, kw, cs, True, pos,
                             rotary_dim=0)
    torch.cuda.synchronize()
    _check(qkv, out, 16, 8, 8, 128, 0, True, torch.float16, qw, kw, cs, pos, "R=0")
    qkv, qw, kw, cs, pos = _make(8192, 32, 8, 8, 64, 64, torch.bfloat16, seed=92)
    out = qkv.clone()
    K.qk_norm_rope_packed_ex(out, 32, 8, 8, 64, 1e-6, qw, kw, cs, False, pos)
    torch.cuda.synchronize()
    _check(qkv, out, 32, 8, 8, 64, 64, False, torch.bfloat16, qw, kw, cs, pos,
           "T=8192 D=64")


def _check_slices(qkv, out, hq, hk, hv, D, R, neox, fp16, qw, kw, cs, pos, what):
    """Every Q/K element against the oracle, in token slices on the host's
    cores; the whole V section unchanged."""
    T = qkv.shape[0]
    n = (hq + hk) * D
    assert torch.equal(out[:, n:], qkv[:, n:])
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    hqw, hkw, hcs = _bits(qw), _bits(kw), I.bits(cs).copy()
    chk = P.check_fp16 if fp16 else P.check_bf16
    st = {"diff": 0}
    with cf.ThreadPoolExecutor(threads) as ex:
        for a in range(0, T, 32768):
            b = min(a + 32768, T)
            ref, hpos = _bits(qkv[a:b]).copy(), I.bits(pos[a:b])
            cuts = [(b - a) * i // threads for i in range(threads + 1)]

            def run(i, ref=ref, hpos=hpos, cuts=cuts):
                u, v = cuts[i], cuts[i + 1]
                O.qk_norm_rope_packed_ex(ref[u:v], hq, hk, hv, D, R, int(neox), int(fp16),
                                         1e-6, hqw, hkw, hcs, hpos[u:v])
            list(ex.map(run, range(threads)))
            got = _bits(out[a:b])[:, :n]
            st["diff"] += int(np.count_nonzero(got != ref[:, :n]))
            chk(got, ref[:, :n], f"{what} tokens {a}..{b}")
    print(f"{what}: all {T * n} Q/K elements checked, {st['diff']} differ in bits",
          flush=True)


@pytest.mark.timeout(600)
def test_past_4_gib():
    # 262144 tokens of 16/8/8 fp16 heads of 256 with interleaved rotation on
    # 128 dims: qkv is 4 GiB, so row offsets run past 2^32 bytes.  The launch
    # is large enough for the occupancy cap.
    T, D, R = 262144, 256, 128
    qkv, qw, kw, cs, pos = _make(T, 16, 8, 8, D, R, torch.float16, seed=93)
    out = qkv.clone()
    K.qk_norm_rope_packed_ex(out, 16, 8, 8, D, 1e-6, qw, kw, cs, False, pos,
                             rotary_dim=R)
    torch.cuda.synchronize()
    _check_slices(qkv, out, 16, 8, 8, D, R, False, True, qw, kw, cs, pos,
                  "T=262144 D=256 fp16")


@pytest.mark.timeout(300)
def test_capped_launch_at_the_threshold():
    # D=64: 24 heads per wave, so one wave per token; 131072 waves and more
    # take the occupancy cap.  A ragged count just past it.
    T, D, R = 131072 + 9, 64, 32
    qkv, qw, kw, cs, pos = _make(T, 16, 8, 8, D, R, torch.bfloat16, seed=94)
    out = qkv.clone()
    K.qk_norm_rope_packed_ex(out, 16, 8, 8, D, 1e-6, qw, kw, cs, True, pos,
                             rotary_dim=R)
    torch.cuda.synchronize()
    _check_slices(qkv, out, 16, 8, 8, D, R, True, False, qw, kw, cs, pos,
                  "capped T=131081 D=64 bf16")


def test_no_rotation_ignores_positions():
    # rotary_dim = 0 is RMSNorm alone: no table row is read, so an empty
    # [0, 0] cos/sin table is enough and any position, in range of nothing,
    # still has its token normalised
    for dtype in (torch.bfloat16, torch.float16):
        qkv, qw, kw, _, _ = _make(37, 5, 3, 2, 128, 0, dtype, seed=96)
        cs = torch.zeros((0, 0), dtype=torch.float32, device=DEV)
        pos = torch.tensor([0, 1, -1, 2 ** 40, -(2 ** 62)] * 7 + [5, 9],
                           dtype=torch.int64, device=DEV)
        out = qkv.clone()
        K.qk_norm_rope_packed_ex(out, 5, 3, 2, 128, 1e-6, qw, kw, cs, True, pos,
                                 rotary_dim=0)
        torch.cuda.synchronize()
        _check(qkv, out, 5, 3, 2, 128, 0, True, dtype, qw, kw, cs, pos,
               f"R=0, empty table, {dtype}")


def test_guarded_case_goes_to_the_tuned_kernel_with_identical_results():
    x = I.make_packed(I.PACKED_WORKLOADS["packed_t17"], DEV)
    a, b = x["qkv"].clone(), x["qkv"].clone()
    K.qk_norm_rope_packed(a, 16, 8, 8, 128, 1e-6, x["q_weight"], x["k_weight"],
                          x["cos_sin_cache"], True, x["position_ids"])
    K.qk_norm_rope_packed_ex(b, 16, 8, 8, 128, 1e-6, x["q_weight"], x["k_weight"],
                             x["cos_sin_cache"], True, x["position_ids"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_rejects_and_out_of_range_positions():
    for R in (40, 136):   # not a multiple of 16 / wider than the head
        qkv, qw, kw, cs, pos = _make(5, 4, 2, 2, 128, R, torch.bfloat16, seed=93)
        before = qkv.clone()
        with pytest.raises(K.Fp8kvError):
            K.qk_norm_rope_packed_ex(qkv, 4, 2, 2, 128, 1e-6, qw, kw, cs, True,
                                     pos, rotary_dim=R)
        assert torch.equal(qkv, before)
    qkv, qw, kw, cs, pos = _make(5, 4, 2, 2, 64, 32, torch.float16, seed=94)
    pos[3] = cs.shape[0]
    out = qkv.clone()
    K.qk_norm_rope_packed_ex(out, 4, 2, 2, 64, 1e-6, qw, kw, cs, False, pos,
                             rotary_dim=32)
    torch.cuda.synchronize()
    assert torch.equal(out[3], qkv[3])
    keep = torch.tensor([0, 1, 2, 4], device=DEV)
    _check(qkv[keep].contiguous(), out[keep].contiguous(), 4, 2, 2, 64, 32, False,
           torch.float16, qw, kw, cs, pos[keep].contiguous(), "in-range tokens")


# (D, heads, T): a launch of at most 8192 waves shares each token's rotary
# row through LDS (a token's waves in one block, or four one-wave tokens per
# block), one of more takes the one-wave form.  T and T + 1 straddle that
# limit; 100/8/4 heads of 256 are 18 waves, three blocks of six per token.
BOUNDARY = [(128, (16, 8, 8), 4096), (256, (16, 8, 8), 2048), (64, (40, 8, 8), 4096),
            (256, (100, 8, 4), 455),
            # one-wave tokens below the limit (rotary rows of up to 64
            # floats): four to a block with NeoX pairs, two with interleaved
            # pairs in bf16, one-wave blocks with interleaved pairs in fp16
            (64, (16, 8, 8), 8192), (128, (8, 2, 2), 8192)]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("D,heads,T", BOUNDARY, ids=[f"D{b[0]}-{b[1][0]}q" for b in BOUNDARY])
def test_both_forms_at_the_token_block_limit(D, heads, T):
    hq, hk, hv = heads
    for n in (T, T + 1):
        for neox, dtype in ((True, torch.bfloat16), (False, torch.float16),
                            (False, torch.bfloat16)):
            R = D // 2
            qkv, qw, kw, cs, pos = _make(n, hq, hk, hv, D, R, dtype, seed=D + n + neox)
            pos[n // 2] = cs.shape[0]       # one token out of range: left as it was
            out = qkv.clone()
            K.qk_norm_rope_packed_ex(out, hq, hk, hv, D, 1e-6, qw, kw, cs, neox, pos,
                                     rotary_dim=R)
            torch.cuda.synchronize()
            assert torch.equal(out[n // 2], qkv[n // 2])
            keep = torch.cat([torch.arange(0, n // 2), torch.arange(n // 2 + 1, n)]).to(DEV)
            _check(qkv[keep].contiguous(), out[keep].contiguous(), hq, hk, hv, D, R, neox,
                   dtype, qw, kw, cs, pos[keep].contiguous(),
                   f"D={D} heads={heads} T={n} neox={neox} {dtype}")


@pytest.mark.parametrize("D,heads,T", BOUNDARY, ids=[f"D{b[0]}-{b[1][0]}q" for b in BOUNDARY])
def test_result_does_not_depend_on_the_form(D, heads, T):
    # The same tokens through the one-wave form (a launch of T + 1 tokens,
    # over the limit) and the token-block form (the first T tokens alone):
    # bit-identical, for every pairing, rotary width and dtype.
    hq, hk, hv = heads
    for R in (D, D // 2, 16):
        for neox in (True, False):
            for dtype in (torch.bfloat16, torch.float16):
                qkv, qw, kw, cs, pos = _make(T + 1, hq, hk, hv, D, R, dtype, seed=D + R)
                big = qkv.clone()
                K.qk_norm_rope_packed_ex(big, hq, hk, hv, D, 1e-6, qw, kw, cs, neox, pos,
                                         rotary_dim=R)
                small = qkv[:T].clone()
                K.qk_norm_rope_packed_ex(small, hq, hk, hv, D, 1e-6, qw, kw, cs, neox,
                                         pos[:T].contiguous(), rotary_dim=R)
                torch.cuda.synchronize()
                assert torch.equal(small.view(torch.int16), big[:T].view(torch.int16)), \
                    f"D={D} heads={heads} R={R} neox={neox} {dtype}"
