"""Parity of the HIP kernels (called through the C ABI via the thin binding)
with the CPU oracle, on seeded synthetic inputs.  Needs an MI355X."""

import concurrent.futures as cf
import os
import time

import numpy as np
import pytest
import torch

import fp8_kv_cache_slot_amd as K
import oracle as O
from fp8_kv_cache_slot_amd import inputs as I
from tests import decision_reach as R
from tests import fp32_decision_case
from tests import golden_case
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SMALL = 2 ** 63 - 1   # threshold sending every call to the small-batch kernel
TILED = 0             # threshold sending every call to the tiled kernel


@pytest.fixture(autouse=True)
def _restore_knobs():
    yield
    K.set_dispatch_threshold(-1)
    K.set_tiling(0, 0)


def _say(msg):
    print(msg, flush=True)


def _run(x, threshold=None):
    q = x["q"].clone()
    cache = x["kv_cache"].clone()
    scale = x["kv_scale"].clone()
    if threshold is not None:
        K.set_dispatch_threshold(threshold)
    K.qnorm_rope_kv_quant_insert(q, x["kv"], x["q_weight"], x["kv_weight"],
                                 x["cos_sin_cache"], x["positions"],
                                 x["slot_mapping"], cache, scale, x["eps"])
    torch.cuda.synchronize()
    return q, cache, scale


def _host(x):
    return {k: (I.bits(v) if isinstance(v, torch.Tensor) else v)
            for k, v in x.items()}


def _oracle(h):
    ref = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in h.items()}
    O.qnorm_rope_kv_quant_insert(
        ref["q"], ref["kv"], ref["q_weight"], ref["kv_weight"],
        ref["cos_sin_cache"], ref["positions"], ref["slot_mapping"],
        ref["kv_cache"], ref["kv_scale"], ref["eps"])
    return ref


def _compare_full(h, ref, got, what):
    q, cache, scale = (I.bits(t) for t in got)
    P.check_bf16(q, ref["q"], what + " q")
    num_slots = h["kv_cache"].shape[0] * 64
    v = P.valid_slots(h["slot_mapping"], num_slots)
    slots = h["slot_mapping"][v]
    y = O.kv_normalised(h["kv"][v].copy(), h["kv_weight"], h["cos_sin_cache"],
                        h["positions"][v].copy(), h["eps"])
    stats = P.check_cache(cache, scale, ref["kv_cache"], ref["kv_scale"], slots, y,
                          I.CACHE_CANARY, I.SCALE_CANARY, what)
    P.check_untouched(cache, scale, slots, I.CACHE_CANARY, I.SCALE_CANARY, what)
    return stats


# ---------------------------------------------------------------------------
# fused prologue
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("threshold", [SMALL, TILED], ids=["small", "tiled"])
def test_golden_worked_example(threshold):
    g = golden_case.load()
    h = golden_case.inputs(g)
    exp = golden_case.expected(g)
    x = {k: (I.from_bits(v, DEV) if isinstance(v, np.ndarray) else v)
         for k, v in h.items()}
    q, cache, scale = _run(x, threshold)
    np.testing.assert_array_equal(I.bits(q), exp["q"])
    np.testing.assert_array_equal(I.bits(scale), exp["kv_scale"])
    np.testing.assert_array_equal(I.bits(cache), exp["kv_cache"])


@pytest.mark.parametrize("threshold", [SMALL, TILED], ids=["small", "tiled"])
def test_quantiser_decides_in_fp32(threshold):
    # A KV row whose block maxima sit a hair (2^-28 relative) above the
    # exponent boundary 1.75 = 448 * 2^-8 and the E4M3 midpoint 232 in
    # double, and exactly on them in fp32: the kernel and the oracle both
    # decide in fp32, so exponents and codes match the hand-derived bytes
    # bit for bit (no boundary-band allowance), for both cache conventions.
    h = fp32_decision_case.inputs()
    x = {k: (I.from_bits(v, DEV) if isinstance(v, np.ndarray) else v)
         for k, v in h.items()}
    q, cache, scale = _run(x, threshold)
    row, sc = I.bits(cache).reshape(-1, 576)[5], I.bits(scale).reshape(-1, 8)[5]
    assert list(sc[:7]) == fp32_decision_case.SCALE_BYTES and sc[7] == 0x5A
    assert list(row[:448]) == fp32_decision_case.CODES
    assert np.all(row[448:].view(np.uint16) == fp32_decision_case.ROPE_BF16)
    ref = _oracle(h)
    np.testing.assert_array_equal(I.bits(q), ref["q"])
    np.testing.assert_array_equal(I.bits(cache), ref["kv_cache"])
    np.testing.assert_array_equal(I.bits(scale), ref["kv_scale"])
    # the scalar-scale convention with kv_cache_scale = 1
    c2 = x["kv_cache"].clone()
    K.qnorm_rope_kv_quant_insert_scalar_scale(
        x["q"].clone(), x["kv"], x["q_weight"], x["kv_weight"],
        x["cos_sin_cache"], x["positions"], x["slot_mapping"], c2,
        torch.ones(1, dtype=torch.float32, device=DEV), x["eps"])
    torch.cuda.synchronize()
    assert list(I.bits(c2).reshape(-1, 576)[5, :448]) == fp32_decision_case.SCALAR_CODES


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_small_workloads_all_paths(name):
    w = I.DSV4_WORKLOADS[name]
    _say(f"workload {name} T={w.num_tokens} H={w.num_heads}")
    x = I.make_dsv4(w, DEV)
    h = _host(x)
    ref = _oracle(h)
    outs = {}
    for label, thr in [("small", SMALL), ("tiled", TILED), ("default", None)]:
        K.set_dispatch_threshold(-1)
        got = _run(x, thr)
        _compare_full(h, ref, got, f"{name}/{label}")
        outs[label] = [I.bits(t) for t in got]
    # repeated launches are deterministic
    again = [I.bits(t) for t in _run(x, TILED)]
    for a, b in zip(again, outs["tiled"]):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("heads", [64, 128])
def test_page_token_counts_both_paths(heads):
    # Token counts that are not multiples of a plausible tiling, plus 1, 4 and
    # 17 tokens pushed through the tiled kernel.
    for T in [1, 4, 17, 511, 512, 777, 1000, 4096]:
        _say(f"T={T} H={heads}")
        w = I.custom_dsv4(T, heads, seed=2000 + T + heads, max_position=8192)
        x = I.make_dsv4(w, DEV)
        h = _host(x)
        ref = _oracle(h)
        for label, thr in [("small", SMALL), ("tiled", TILED)]:
            _compare_full(h, ref, _run(x, thr), f"T={T} H={heads} {label}")


def test_every_built_tiling():
    w = I.custom_dsv4(300, 20, seed=3000, max_position=8192)   # ragged: 20 heads
    x = I.make_dsv4(w, DEV)
    h = _host(x)
    ref = _oracle(h)
    shapes = [(1, 1), (1, 2), (2, 1), (2, 2), (4, 1), (4, 2), (4, 4), (8, 1),
              (8, 2), (8, 4), (16, 1), (16, 2)]
    for wv, qs in shapes:
        _say(f"tiling {wv}x{qs}")
        K.set_tiling(wv, qs)
        _compare_full(h, ref, _run(x, TILED), f"tiling {wv}x{qs}")
    with pytest.raises(K.Fp8kvError):
        K.set_tiling(3, 3)


@pytest.mark.parametrize("heads", [3, 5, 6, 7, 9, 11])
def test_ragged_heads_every_tiling(heads):
    # head counts that are not a multiple of the heads per wave: the last
    # wave of each token holds fewer heads (re-reads the first, stores none)
    w = I.custom_dsv4(37, heads, seed=3100 + heads, max_position=8192)
    x = I.make_dsv4(w, DEV)
    h = _host(x)
    ref = _oracle(h)
    for wv, qs in [(1, 2), (2, 2), (4, 2), (4, 4), (8, 2), (8, 4), (16, 2)]:
        _say(f"H={heads} tiling {wv}x{qs}")
        K.set_tiling(wv, qs)
        _compare_full(h, ref, _run(x, TILED), f"H={heads} tiling {wv}x{qs}")
    K.set_tiling(0, 0)


@pytest.mark.parametrize("heads,T", [(1, 300), (1000, 3), (4099, 2)])
def test_many_heads(heads, T):
    # a token spread over thousands of Q waves (and blocks), or over one
    w = I.custom_dsv4(T, heads, seed=3200 + heads, max_position=8192)
    x = I.make_dsv4(w, DEV)
    h = _host(x)
    ref = _oracle(h)
    for wv, qs in [(1, 1), (4, 2), (16, 2), (8, 4)]:
        _say(f"H={heads} T={T} tiling {wv}x{qs}")
        K.set_tiling(wv, qs)
        _compare_full(h, ref, _run(x, TILED), f"H={heads} tiling {wv}x{qs}")
    K.set_tiling(0, 0)
    _compare_full(h, ref, _run(x, SMALL), f"H={heads} small-batch")


def _oracle_threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["prefill", "wide128", "long64"])
def test_full_size_workloads(name):
    # Full size, default dispatch (the configuration the benchmark times):
    # every q element and every KV row against the oracle, and every byte the
    # call must not write.
    _check_full_size(I.DSV4_WORKLOADS[name])


@pytest.mark.timeout(900)
def test_twice_the_largest_workload():
    # 262144 tokens x 64 heads: 2^33 q elements (16 GiB), twice the largest
    # workload, so q offsets, slot rows and block indices all run past 2^32
    # bytes (4096 pages, every slot written once in a random order).
    _check_full_size(I.Dsv4Workload("max64", 262144, 64, 131072, 4096, False,
                                     "uniform", "permutation", 0, 1023))


def _check_full_size(w):
    name = w.name
    T, H = w.num_tokens, w.num_heads
    _say(f"workload {name} T={T} H={H}")
    x = I.make_dsv4(w, DEV)
    q, cache, scale = _run(x)
    num_slots = w.num_pages * 64
    sm = x["slot_mapping"]
    valid = (sm >= 0) & (sm < num_slots)
    written = sm[valid]
    mask = torch.ones(num_slots, dtype=torch.bool, device=DEV)
    mask[written] = False
    c2, s2 = cache.view(-1, 576), scale.view(-1, 8)
    assert bool((c2[mask] == I.CACHE_CANARY).all())
    assert bool((s2[mask] == I.SCALE_CANARY).all())
    assert bool((s2[:, 7] == I.SCALE_CANARY).all())
    assert bool((s2[written, :7] != I.SCALE_CANARY).all())

    # The whole workload against the oracle in token slices of 512 MiB of q
    # (the pages' own way to run the large shapes with bounded temporaries,
    # FlagGems PR #5321 "The four test and benchmark fixes"); each slice is
    # split over the host's cores (the oracle's entry releases the
    # interpreter lock, and the injective slot map keeps the sub-slices'
    # cache rows disjoint).  q: the bf16 rule on every element.  KV rows:
    # exponents bit-exact outside the boundary band, codes within one step,
    # rotary dims by the bf16 rule.
    qw, kw = I.bits(x["q_weight"]), I.bits(x["kv_weight"])
    cs = I.bits(x["cos_sin_cache"])
    got_c, got_s = I.bits(cache), I.bits(scale)
    ref_c = np.full((w.num_pages, 64, 576), I.CACHE_CANARY, np.uint8)
    ref_s = np.full((w.num_pages, 64, 8), I.SCALE_CANARY, np.uint8)
    threads = _oracle_threads()
    chunk = max(threads, (1 << 29) // (H * 1024))
    qstats = {}
    band = diff = rows = e_prec = c_prec = 0
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(threads) as ex:
        for a in range(0, T, chunk):
            b = min(a + chunk, T)
            hq = I.bits(x["q"][a:b])
            hkv, hpos = I.bits(x["kv"][a:b]), I.bits(x["positions"][a:b])
            hsm = I.bits(sm[a:b])
            cuts = [(b - a) * i // threads for i in range(threads + 1)]

            def run(i, hq=hq, hkv=hkv, hpos=hpos, hsm=hsm, cuts=cuts):
                u, v = cuts[i], cuts[i + 1]
                O.qnorm_rope_kv_quant_insert(hq[u:v], hkv[u:v], qw, kw, cs,
                                             hpos[u:v], hsm[u:v], ref_c, ref_s,
                                             w.eps)
            list(ex.map(run, range(threads)))
            P.check_bf16(I.bits(q[a:b]), hq, f"{name} q tokens {a}..{b}", qstats)
            ok = P.valid_slots(hsm, num_slots)
            yc = O.kv_normalised(hkv[ok].copy(), kw, cs, hpos[ok].copy(), w.eps)
            st = P.check_cache(got_c, got_s, ref_c, ref_s, hsm[ok], yc,
                               I.CACHE_CANARY, I.SCALE_CANARY,
                               f"{name} tokens {a}..{b}")
            band += st["band_blocks"]
            diff += st["code_diff"]
            rows += st["rows"]
            pe, pc = R.decision_differences(yc)
            e_prec += pe
            c_prec += pc
    _say(f"{name}: all {qstats['n']} q elements checked: {qstats['diff']} differ "
         f"in bits ({qstats['diff'] / qstats['n']:.2e}), at most "
         f"{qstats['max_steps']} bf16 step(s) apart where |ref| >= 2^-7, largest "
         f"difference {qstats['max_abs']:.2e}; all {rows} KV rows: {band} "
         f"exponent(s) in the boundary band, {diff} of {rows * 448} codes one step "
         f"apart; deciding in double instead of fp32 would change {e_prec} of "
         f"{rows * 7} exponents and {c_prec} codes; {time.perf_counter() - t0:.0f} s "
         f"on {threads} threads")


def test_cache_past_2_gib():
    # 65536 pages: 2.4 GB of cache rows, so the rows of slots in the last
    # pages start past 2^31 bytes.  Half the tokens go to the last slots of
    # the cache, half to random ones.  The written rows are compared with the
    # oracle (run on a compact cache of one row per token), every other byte
    # keeps its canary, and both read sides return the oracle's dequantised
    # rows.
    pages, T, H = 65536, 64, 2
    num_slots = pages * 64
    w = I.custom_dsv4(T, H, seed=2400, num_pages=pages, max_position=4096,
                      skipped=0)
    _say(f"cache of {pages} pages, T={T} H={H}")
    x = I.make_dsv4(w, DEV)
    rng = np.random.default_rng(2400)
    top = num_slots - 1 - np.arange(T // 2)
    low = rng.choice(num_slots - T, size=T - T // 2, replace=False)
    slots = np.concatenate([top, low]).astype(np.int64)
    assert (slots[: T // 2] * 576 >= 2 ** 31).all()
    x["slot_mapping"] = torch.from_numpy(slots).to(DEV)
    small = {k: v for k, v in x.items() if k not in ("kv_cache", "kv_scale")}
    compact = dict(_host(small), slot_mapping=np.arange(T, dtype=np.int64),
                   kv_cache=np.full((1, 64, 576), I.CACHE_CANARY, np.uint8),
                   kv_scale=np.full((1, 64, 8), I.SCALE_CANARY, np.uint8))
    ref = _oracle(compact)
    y = O.kv_normalised(compact["kv"], compact["kv_weight"],
                        compact["cos_sin_cache"], compact["positions"],
                        compact["eps"])
    for label, thr in [("small", SMALL), ("tiled", TILED)]:
        q, cache, scale = _run(x, thr)
        P.check_bf16(I.bits(q), ref["q"], f"{label} q")
        si = torch.from_numpy(slots).to(DEV)
        c2, s2 = cache.view(-1, 576), scale.view(-1, 8)
        got_c = I.bits(c2[si]).reshape(1, 64, 576)
        got_s = I.bits(s2[si]).reshape(1, 64, 8)
        P.check_cache(got_c, got_s, ref["kv_cache"], ref["kv_scale"],
                      np.arange(T), y, I.CACHE_CANARY, I.SCALE_CANARY, label)
        # every other byte of the 2.4 GB cache is untouched
        c2[si] = I.CACHE_CANARY
        s2[si, :7] = I.SCALE_CANARY
        assert bool((c2 == I.CACHE_CANARY).all()) and bool((s2 == I.SCALE_CANARY).all())
        c2[si] = torch.from_numpy(got_c.reshape(T, 576)).to(DEV)
        s2[si] = torch.from_numpy(got_s.reshape(T, 8)).to(DEV)
        # read side by slot list and through a block table of the last page
        want = O.kv_cache_gather_dequant(got_c, got_s, np.arange(T, dtype=np.int64))
        out = K.kv_cache_gather_dequant(cache, scale, si)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(I.bits(out), want)
        last = torch.full((1, 1), pages - 1, dtype=torch.int32, device=DEV)
        out2 = torch.zeros((64, 512), dtype=torch.bfloat16, device=DEV)
        K.kv_cache_gather_dequant_paged(
            cache, scale, last, torch.tensor([64], dtype=torch.int32, device=DEV),
            torch.zeros(1, dtype=torch.int64, device=DEV), out2)
        ref_last = K.kv_cache_gather_dequant(
            cache, scale, torch.arange(num_slots - 64, num_slots, device=DEV))
        torch.cuda.synchronize()
        assert torch.equal(out2, ref_last)


def test_rows_of_distinct_magnitude():
    # Regression for the cross-row reduction: the four 16-lane rows of a head
    # (dims 0-127, 128-255, 256-383, 384-511) hold very different magnitudes,
    # so a reduction that drops, doubles or swaps a row cannot match.
    w = I.custom_dsv4(8, 4, seed=4010)
    x = I.make_dsv4(w, DEV)
    scale = torch.tensor([1.0, 8.0, 0.125, 64.0], device=DEV).repeat_interleave(128)
    x["q"] = (x["q"].float() * scale).to(torch.bfloat16).contiguous()
    x["kv"] = (x["kv"].float() * scale.flip(0)).to(torch.bfloat16).contiguous()
    h = _host(x)
    ref = _oracle(h)
    for thr in (SMALL, TILED):
        _compare_full(h, ref, _run(x, thr), "row magnitudes")


def test_edge_cases():
    # one token, one head
    w = I.custom_dsv4(1, 1, seed=4000)
    x = I.make_dsv4(w, DEV)
    h = _host(x)
    ref = _oracle(h)
    for thr in (SMALL, TILED):
        _compare_full(h, ref, _run(x, thr), "T=1 H=1")
    # all-zero activations
    w = I.custom_dsv4(9, 3, seed=4001)
    x = I.make_dsv4(w, DEV)
    x["q"].zero_()
    x["kv"].zero_()
    h = _host(x)
    ref = _oracle(h)
    for thr in (SMALL, TILED):
        _compare_full(h, ref, _run(x, thr), "zeros")
    # no token writes the cache; zero pages
    w = I.custom_dsv4(7, 5, seed=4002, num_pages=1)
    x = I.make_dsv4(w, DEV)
    x["slot_mapping"][:] = -1
    x["slot_mapping"][2] = 64          # == num_pages * 64: out of range
    h = _host(x)
    ref = _oracle(h)
    for thr in (SMALL, TILED):
        _compare_full(h, ref, _run(x, thr), "all skipped")
    x["kv_cache"] = torch.empty((0, 64, 576), dtype=torch.uint8, device=DEV)
    x["kv_scale"] = torch.empty((0, 64, 8), dtype=torch.uint8, device=DEV)
    q, _, _ = _run(x)
    P.check_bf16(I.bits(q), ref["q"], "zero pages")
    # zero tokens: nothing happens
    K.qnorm_rope_kv_quant_insert(
        x["q"][:0], x["kv"][:0], x["q_weight"], x["kv_weight"],
        x["cos_sin_cache"], x["positions"][:0], x["slot_mapping"][:0],
        x["kv_cache"], x["kv_scale"], 1e-6)
    torch.cuda.synchronize()


def test_out_of_range_position_leaves_token_untouched():
    w = I.custom_dsv4(12, 6, seed=4003, max_position=64)
    x = I.make_dsv4(w, DEV)
    x["slot_mapping"] = torch.arange(12, device=DEV, dtype=torch.int64)
    bad = [3, 7]
    pos = x["positions"].clone()
    x["positions"][3] = -1
    x["positions"][7] = 64
    for thr in (SMALL, TILED):
        q, cache, scale = _run(x, thr)
        for t in bad:
            assert torch.equal(q[t], x["q"][t])
            assert bool((cache.view(-1, 576)[t] == I.CACHE_CANARY).all())
            assert bool((scale.view(-1, 8)[t] == I.SCALE_CANARY).all())
        # every other token is as the oracle says
        keep = torch.tensor([t for t in range(12) if t not in bad], device=DEV)
        y = dict(x)
        y["positions"] = pos
        h = _host({k: (v[keep] if k in ("q", "kv", "positions", "slot_mapping")
                       else v) for k, v in y.items()})
        ref = _oracle(h)
        P.check_bf16(I.bits(q[keep]), ref["q"], "in-range tokens")


def test_argument_errors_touch_nothing():
    w = I.custom_dsv4(8, 4, seed=4004)
    x = I.make_dsv4(w, DEV)
    q0 = x["q"].clone()
    L = K.lib()
    args = [x["q"].data_ptr(), x["kv"].data_ptr(), x["q_weight"].data_ptr(),
            x["kv_weight"].data_ptr(), x["cos_sin_cache"].data_ptr(),
            x["positions"].data_ptr(), x["slot_mapping"].data_ptr(),
            x["kv_cache"].data_ptr(), x["kv_scale"].data_ptr(), 8, 4, 512, 64,
            x["cos_sin_cache"].shape[0], w.num_pages, 64, 1e-6, None]
    cases = {2: dict(i=9, v=-1), 3: dict(i=11, v=256), 4: dict(i=0, v=args[0] + 2),
             1: dict(i=1, v=None)}
    for want, c in cases.items():
        a = list(args)
        a[c["i"]] = c["v"]
        assert L.qnorm_rope_kv_quant_insert(*a) == want
    torch.cuda.synchronize()
    assert torch.equal(x["q"], q0)
    assert L.qnorm_rope_kv_quant_insert(*args) == 0
    torch.cuda.synchronize()
    assert not torch.equal(x["q"], q0)


# ---------------------------------------------------------------------------
# packed Q/K norm + RoPE
# ---------------------------------------------------------------------------

def _run_packed(x, forced=-1, explicit=True):
    qkv = x["qkv"].clone()
    kw = dict(forced_token_heads_per_warp=forced) if explicit else {}
    K.qk_norm_rope_packed(qkv, x["num_heads_q"], x["num_heads_k"],
                          x["num_heads_v"], x["head_dim"], x["eps"],
                          x["q_weight"], x["k_weight"], x["cos_sin_cache"], True,
                          x["position_ids"], **kw)
    torch.cuda.synchronize()
    return qkv


def _oracle_packed(x):
    qkv = I.bits(x["qkv"]).copy()
    O.qk_norm_rope_packed(qkv, x["num_heads_q"], x["num_heads_k"],
                          x["num_heads_v"], x["head_dim"], x["eps"],
                          I.bits(x["q_weight"]), I.bits(x["k_weight"]),
                          I.bits(x["cos_sin_cache"]), I.bits(x["position_ids"]))
    return qkv


def _compare_packed(x, got, what):
    ref = _oracle_packed(x)
    g = I.bits(got)
    nqk = (x["num_heads_q"] + x["num_heads_k"]) * x["head_dim"]
    np.testing.assert_array_equal(g[:, nqk:], I.bits(x["qkv"])[:, nqk:],
                                  err_msg=what + ": V section changed")
    P.check_bf16(g[:, :nqk], ref[:, :nqk], what)


@pytest.mark.parametrize("name", ["packed_t1", "packed_t17", "packed_t1024",
                                  "packed_t4096", "packed_t8192"])
def test_packed_workloads(name):
    _say(f"workload {name}")
    x = I.make_packed(I.PACKED_WORKLOADS[name], DEV)
    got = _run_packed(x)
    _compare_packed(x, got, name)
    # forced_token_heads_per_warp = -1 passed explicitly or left to the default
    assert torch.equal(got, _run_packed(x, explicit=False))


@pytest.mark.timeout(600)
def test_packed_past_2_gib():
    # 262144 tokens of 16/8/8 heads of 128: qkv is 2 GiB, so row offsets run
    # past 2^31 bytes.  Every Q/K element against the oracle, in token slices
    # on the host's cores; the whole V section unchanged.
    w = I.PackedWorkload("packed_2gib", 262144, seed=1034)
    _say(f"workload {w.name} T={w.num_tokens}")
    x = I.make_packed(w, DEV)
    got = _run_packed(x)
    nqk = (w.num_heads_q + w.num_heads_k) * w.head_dim
    assert torch.equal(got[:, nqk:], x["qkv"][:, nqk:])
    _check_packed_slices(x, got, w.name)


def _check_packed_slices(x, got, what, chunk=32768):
    """Every Q/K element of ``got`` against the oracle, in token slices split
    over the host's cores (one oracle call per sub-slice)."""
    nqk = (x["num_heads_q"] + x["num_heads_k"]) * x["head_dim"]
    qw, kw = I.bits(x["q_weight"]), I.bits(x["k_weight"])
    cs = I.bits(x["cos_sin_cache"])
    threads = _oracle_threads()
    T = x["qkv"].shape[0]
    st = {}
    with cf.ThreadPoolExecutor(threads) as ex:
        for a in range(0, T, chunk):
            b = min(a + chunk, T)
            ref, pos = I.bits(x["qkv"][a:b]), I.bits(x["position_ids"][a:b])
            cuts = [(b - a) * i // threads for i in range(threads + 1)]

            def run(i, ref=ref, pos=pos, cuts=cuts):
                u, v = cuts[i], cuts[i + 1]
                O.qk_norm_rope_packed(ref[u:v], x["num_heads_q"], x["num_heads_k"],
                                      x["num_heads_v"], x["head_dim"], x["eps"],
                                      qw, kw, cs, pos[u:v])
            list(ex.map(run, range(threads)))
            P.check_bf16(I.bits(got[a:b])[:, :nqk], ref[:, :nqk],
                         f"{what} tokens {a}..{b}", st)
    _say(f"{what}: all {st['n']} Q/K elements checked: {st['diff']} differ in bits, "
         f"at most {st['max_steps']} bf16 step(s) apart where |ref| >= 2^-7, "
         f"largest difference {st['max_abs']:.2e}")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("heads,T", [((8, 2, 2), 131077), ((16, 8, 8), 32771),
                                     ((32, 4, 4), 21846), ((40, 8, 8), 16385),
                                     ((48, 8, 8), 13108), ((100, 8, 4), 6554)])
def test_packed_occupancy_capped_launches(heads, T):
    # Launches large enough for the occupancy cap (blocks of one to five
    # waves; the last mix has two blocks of five waves per token), every Q/K
    # element against the oracle, V unchanged.
    hq, hk, hv = heads
    w = I.PackedWorkload("capped", T, hq, hk, hv, seed=5200 + hq)
    _say(f"capped launch heads={heads} T={T}")
    x = I.make_packed(w, DEV)
    got = _run_packed(x)
    nqk = (hq + hk) * w.head_dim
    assert torch.equal(got[:, nqk:], x["qkv"][:, nqk:])
    _check_packed_slices(x, got, f"capped {heads} T={T}")


@pytest.mark.parametrize("heads", [(16, 0, 8), (0, 8, 8), (5, 3, 1), (1, 1, 0),
                                   (32, 8, 8), (40, 4, 4), (7, 6, 2), (20, 5, 0),
                                   (12, 0, 3),
                                   # more than 8 waves of 12 heads: a token
                                   # spans several blocks, each reading the
                                   # position and cos/sin row itself
                                   (100, 8, 4), (200, 0, 1), (96, 0, 0)])
def test_packed_head_mixes(heads):
    hq, hk, hv = heads
    w = I.PackedWorkload("mix", 33, hq, hk, hv, seed=5000 + hq * 7 + hk)
    x = I.make_packed(w, DEV)
    _compare_packed(x, _run_packed(x), f"heads {heads}")


def test_packed_rejects_and_skips():
    x = I.make_packed(I.PackedWorkload("p", 5, seed=5100), DEV)
    for bad in (dict(forced=4), ):
        with pytest.raises(K.Fp8kvError):
            _run_packed(x, forced=bad["forced"])
    qkv = x["qkv"].clone()
    with pytest.raises(K.Fp8kvError):
        K.qk_norm_rope_packed(qkv, 16, 8, 8, 128, 1e-6, x["q_weight"],
                              x["k_weight"], x["cos_sin_cache"], False,
                              x["position_ids"])
    assert torch.equal(qkv, x["qkv"])
    # out-of-range position: that token is untouched
    x["position_ids"][2] = x["cos_sin_cache"].shape[0]
    got = _run_packed(x)
    assert torch.equal(got[2], x["qkv"][2])
    keep = torch.tensor([0, 1, 3, 4], device=DEV)
    y = dict(x)
    y["qkv"] = x["qkv"][keep].contiguous()
    y["position_ids"] = x["position_ids"][keep].contiguous()
    _compare_packed(y, got[keep].contiguous(), "in-range tokens")
