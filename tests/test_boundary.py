"""The C ABI on the CPU: the library loads, exports exactly what
include/fp8kv.h declares, and rejects bad arguments before touching any
device (so these calls never launch).  Also the byte accounting and the
input generators."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

import fp8_kv_cache_slot_amd as K
from fp8_kv_cache_slot_amd import accounting as A
from fp8_kv_cache_slot_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8kv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) -
                  {"defined"})


def test_header_declarations_are_exported():
    names = _declared()
    assert "qnorm_rope_kv_quant_insert" in names and "qk_norm_rope_packed" in names
    lib = ctypes.CDLL(K.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(K.EXPORTED)
    assert K.abi_version() == 2


def test_exports_nothing_else():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", K.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert syms == set(K.EXPORTED)


def test_status_strings():
    for s in range(8):
        assert K.lib().fp8kv_status_string(s).decode()
    assert K.lib().fp8kv_status_string(99) == b"unknown status"


FAKE = 0x10000  # aligned non-NULL address; never dereferenced (validation fails first)


def _prologue(**over):
    a = dict(q=FAKE, kv=FAKE, qw=FAKE, kw=FAKE, cs=FAKE, pos=FAKE, sm=FAKE,
             cache=FAKE, scale=FAKE, T=4, H=8, D=512, R=64, maxp=16, pages=1,
             page=64, eps=1e-6, stream=None)
    a.update(over)
    return K.lib().qnorm_rope_kv_quant_insert(*a.values())


def _packed(**over):
    a = dict(qkv=FAKE, T=4, hq=16, hk=8, hv=8, D=128, eps=1e-6, qw=FAKE, kw=FAKE,
             cs=FAKE, neox=1, pos=FAKE, forced=-1, maxp=16, stream=None)
    a.update(over)
    return K.lib().qk_norm_rope_packed(*a.values())


@pytest.mark.parametrize("over,want", [
    (dict(T=-1), 2), (dict(H=0), 2), (dict(maxp=0), 2), (dict(pages=-1), 2),
    (dict(T=1 << 30, H=64), 2),
    (dict(D=256), 3), (dict(R=32), 3), (dict(page=16), 3),
    (dict(q=None), 1), (dict(kv=None), 1), (dict(qw=None), 1), (dict(kw=None), 1),
    (dict(cs=None), 1), (dict(pos=None), 1), (dict(sm=None), 1),
    (dict(cache=None), 1), (dict(scale=None), 1),
    (dict(q=FAKE + 8), 4), (dict(kv=FAKE + 2), 4), (dict(qw=FAKE + 4), 4),
    (dict(cs=FAKE + 4), 4), (dict(pos=FAKE + 4), 4), (dict(cache=FAKE + 8), 4),
    (dict(T=0, q=None, kv=None), 0),
    (dict(pages=0, cache=None, scale=None, T=0), 0),
])
def test_prologue_argument_errors(over, want):
    assert _prologue(**over) == want


@pytest.mark.parametrize("over,want", [
    (dict(T=-1), 2), (dict(hq=0, hk=0), 2), (dict(hv=-1), 2), (dict(maxp=0), 2),
    (dict(D=64), 3), (dict(neox=0), 3), (dict(forced=0), 3), (dict(forced=4), 3),
    (dict(qkv=None), 1), (dict(cs=None), 1), (dict(pos=None), 1),
    (dict(qw=None), 1), (dict(kw=None), 1),
    (dict(qkv=FAKE + 2), 4), (dict(cs=FAKE + 8), 4), (dict(kw=FAKE + 2), 4),
    (dict(T=0), 0),
])
def test_packed_argument_errors(over, want):
    assert _packed(**over) == want


@pytest.mark.parametrize("eps", [-1e-6, float("nan"), float("inf"), -float("inf")])
def test_eps_must_be_finite_and_non_negative(eps):
    # every entry point that takes eps refuses these before anything else
    assert _prologue(eps=eps) == 7 and _prologue(eps=eps, T=0) == 7
    assert _prologue_scalar(eps=eps) == 7
    assert _packed(eps=eps) == 7 and _packed_ex(eps=eps) == 7
    assert _norm(eps=eps) == 7


def _prologue_scalar(**over):
    a = dict(q=FAKE, kv=FAKE, qw=FAKE, kw=FAKE, cs=FAKE, pos=FAKE, sm=FAKE,
             cache=FAKE, scale=FAKE, T=4, H=8, D=512, R=64, maxp=16, pages=1,
             page=64, eps=1e-6, stream=None)
    a.update(over)
    return K.lib().qnorm_rope_kv_quant_insert_scalar_scale(*a.values())


def _dequant_scalar(**over):
    a = dict(cache=FAKE, scale=FAKE, pages=2, page=64, slots=FAKE, rows=10,
             out=FAKE, stream=None)
    a.update(over)
    return K.lib().kv_cache_gather_dequant_scalar_scale(*a.values())


@pytest.mark.parametrize("fn,over,want", [
    (_prologue_scalar, dict(T=-1), 2), (_prologue_scalar, dict(D=256), 3),
    (_prologue_scalar, dict(scale=None), 1), (_prologue_scalar, dict(cache=None), 1),
    (_prologue_scalar, dict(scale=FAKE + 2), 4), (_prologue_scalar, dict(q=FAKE + 8), 4),
    (_prologue_scalar, dict(T=0, q=None), 0),
    (_dequant_scalar, dict(rows=-1), 2), (_dequant_scalar, dict(page=16), 3),
    (_dequant_scalar, dict(scale=None), 1), (_dequant_scalar, dict(scale=FAKE + 2), 4),
    (_dequant_scalar, dict(rows=0, slots=None), 0),
])
def test_scalar_scale_argument_errors(fn, over, want):
    assert fn(**over) == want


def _packed_ex(**over):
    a = dict(qkv=FAKE, T=4, hq=16, hk=8, hv=8, D=128, eps=1e-6, qw=FAKE, kw=FAKE,
             cs=FAKE, neox=1, pos=FAKE, R=64, dtype=0, maxp=16, stream=None)
    a.update(over)
    return K.lib().qk_norm_rope_packed_ex(*a.values())


@pytest.mark.parametrize("over,want", [
    (dict(T=-1), 2), (dict(hq=0, hk=0), 2), (dict(maxp=0), 2),
    (dict(D=96), 3), (dict(D=512), 3), (dict(R=24), 3), (dict(R=144), 3),
    (dict(R=-16), 3), (dict(neox=2), 3), (dict(dtype=2), 3),
    (dict(qkv=None), 1), (dict(pos=None), 1), (dict(cs=None), 1),
    (dict(qw=None), 1), (dict(qkv=FAKE + 8), 4), (dict(cs=FAKE + 4), 4),
    (dict(T=0), 0),
])
def test_packed_ex_argument_errors(over, want):
    assert _packed_ex(**over) == want


def _dequant(**over):
    a = dict(cache=FAKE, scale=FAKE, pages=2, page=64, slots=FAKE, rows=10,
             out=FAKE, stream=None)
    a.update(over)
    return K.lib().kv_cache_gather_dequant(*a.values())


@pytest.mark.parametrize("over,want", [
    (dict(rows=-1), 2), (dict(pages=-1), 2), (dict(rows=1 << 31), 2),
    (dict(page=32), 3),
    (dict(slots=None), 1), (dict(out=None), 1), (dict(cache=None), 1),
    (dict(scale=None), 1),
    (dict(slots=FAKE + 4), 4), (dict(out=FAKE + 8), 4), (dict(cache=FAKE + 8), 4),
    (dict(scale=FAKE + 4), 4),
    (dict(rows=0, slots=None, out=None), 0),
])
def test_dequant_argument_errors(over, want):
    assert _dequant(**over) == want


def _norm(**over):
    a = dict(x=FAKE, out=FAKE, w=FAKE, rows=10, dim=512, eps=1e-6, stream=None)
    a.update(over)
    return K.lib().rms_norm_rows(*a.values())


def _rope(**over):
    a = dict(x=FAKE, cs=FAKE, pos=FAKE, T=3, R=4, dim=512, rope=64, maxp=8,
             stream=None)
    a.update(over)
    return K.lib().rope_rows(*a.values())


def _quant(**over):
    a = dict(kv=FAKE, sm=FAKE, cache=FAKE, scale=FAKE, T=3, pages=1, page=64,
             stream=None)
    a.update(over)
    return K.lib().kv_quant_insert(*a.values())


@pytest.mark.parametrize("fn,over,want", [
    (_norm, dict(rows=-1), 2), (_norm, dict(dim=256), 3), (_norm, dict(x=None), 1),
    (_norm, dict(out=None), 1), (_norm, dict(w=None), 1), (_norm, dict(out=FAKE + 8), 4),
    (_norm, dict(rows=0, x=None), 0),
    (_rope, dict(T=-1), 2), (_rope, dict(R=0), 2), (_rope, dict(maxp=0), 2),
    (_rope, dict(dim=128), 3), (_rope, dict(rope=32), 3), (_rope, dict(x=None), 1),
    (_rope, dict(cs=None), 1), (_rope, dict(pos=None), 1), (_rope, dict(x=FAKE + 2), 4),
    (_rope, dict(T=0, x=None), 0),
    (_quant, dict(T=-1), 2), (_quant, dict(pages=-1), 2), (_quant, dict(page=32), 3),
    (_quant, dict(kv=None), 1), (_quant, dict(sm=None), 1), (_quant, dict(cache=None), 1),
    (_quant, dict(kv=FAKE + 8), 4), (_quant, dict(T=0, kv=None), 0),
])
def test_stage_argument_errors(fn, over, want):
    assert fn(**over) == want


def _norm_heads(**over):
    a = dict(x=FAKE, stride=4096, out=FAKE, w=FAKE, T=5, H=16, D=128, eps=1e-6,
             stream=None)
    a.update(over)
    return K.lib().rms_norm_heads(*a.values())


def _rope_heads(**over):
    a = dict(x=FAKE, cs=FAKE, pos=FAKE, T=5, H=16, D=128, maxp=8, stream=None)
    a.update(over)
    return K.lib().rope_neox_heads(*a.values())


@pytest.mark.parametrize("fn,over,want", [
    (_norm_heads, dict(T=-1), 2), (_norm_heads, dict(H=-1), 2),
    (_norm_heads, dict(stride=2047), 2), (_norm_heads, dict(T=2 ** 27, H=16), 2),
    (_norm_heads, dict(D=64), 3), (_norm_heads, dict(eps=-1.0), 7),
    (_norm_heads, dict(eps=float("nan")), 7),
    (_norm_heads, dict(x=None), 1), (_norm_heads, dict(out=None), 1),
    (_norm_heads, dict(w=None), 1), (_norm_heads, dict(x=FAKE + 8), 4),
    (_norm_heads, dict(stride=4100), 4), (_norm_heads, dict(T=0, x=None), 0),
    (_norm_heads, dict(H=0, x=None, stride=0), 0),
    (_rope_heads, dict(T=-1), 2), (_rope_heads, dict(maxp=0), 2),
    (_rope_heads, dict(D=256), 3), (_rope_heads, dict(x=None), 1),
    (_rope_heads, dict(cs=None), 1), (_rope_heads, dict(pos=None), 1),
    (_rope_heads, dict(cs=FAKE + 4), 4), (_rope_heads, dict(pos=FAKE + 4), 4),
    (_rope_heads, dict(T=0, x=None), 0),
])
def test_packed_stage_argument_errors(fn, over, want):
    assert fn(**over) == want


def _paged(**over):
    a = dict(cache=FAKE, scale=FAKE, pages=2, page=64, table=FAKE, S=3, M=4,
             lens=FAKE, offs=FAKE, N=100, out=FAKE, stream=None)
    a.update(over)
    return K.lib().kv_cache_gather_dequant_paged(*a.values())


@pytest.mark.parametrize("over,want", [
    (dict(pages=-1), 2), (dict(S=-1), 2), (dict(S=65536), 2), (dict(M=-1), 2),
    (dict(M=(1 << 24) + 1), 2), (dict(N=-1), 2), (dict(page=32), 3),
    (dict(table=None), 1), (dict(lens=None), 1), (dict(offs=None), 1),
    (dict(out=None), 1), (dict(cache=None), 1), (dict(scale=None), 1),
    (dict(table=FAKE + 2), 4), (dict(lens=FAKE + 1), 4), (dict(offs=FAKE + 4), 4),
    (dict(out=FAKE + 8), 4), (dict(cache=FAKE + 8), 4), (dict(scale=FAKE + 4), 4),
    (dict(S=0, table=None, lens=None, offs=None), 0), (dict(M=0, table=None), 0),
    (dict(N=0, out=None), 0),
])
def test_paged_dequant_argument_errors(over, want):
    assert _paged(**over) == want


def _paged_scalar(**over):
    a = dict(cache=FAKE, scale=FAKE, pages=2, page=64, table=FAKE, S=3, M=4,
             lens=FAKE, offs=FAKE, N=100, out=FAKE, stream=None)
    a.update(over)
    return K.lib().kv_cache_gather_dequant_paged_scalar_scale(*a.values())


@pytest.mark.parametrize("over,want", [
    (dict(pages=-1), 2), (dict(S=65536), 2), (dict(page=32), 3),
    (dict(table=None), 1), (dict(cache=None), 1), (dict(scale=None), 1),
    (dict(scale=FAKE + 2), 4), (dict(out=FAKE + 8), 4),
    (dict(S=0, table=None, lens=None, offs=None), 0), (dict(N=0, out=None), 0),
])
def test_paged_scalar_dequant_argument_errors(over, want):
    assert _paged_scalar(**over) == want


def _copy(**over):
    a = dict(dst=FAKE, src=FAKE + 4096, nb=4096, stream=None)
    a.update(over)
    return K.lib().fp8kv_stream_copy(*a.values())


def _rmw(**over):
    a = dict(buf=FAKE, nb=4096, mask=0, stream=None)
    a.update(over)
    return K.lib().fp8kv_stream_rmw(*a.values())


@pytest.mark.parametrize("fn,over,want", [
    (_copy, dict(nb=-16), 2), (_copy, dict(nb=24), 2), (_copy, dict(dst=None), 1),
    (_copy, dict(src=None), 1), (_copy, dict(dst=FAKE + 8), 4),
    (_copy, dict(src=FAKE + 4), 4), (_copy, dict(nb=0, dst=None, src=None), 0),
    (_rmw, dict(nb=-16), 2), (_rmw, dict(nb=8), 2), (_rmw, dict(buf=None), 1),
    (_rmw, dict(buf=FAKE + 2), 4), (_rmw, dict(nb=0, buf=None), 0),
])
def test_stream_reference_argument_errors(fn, over, want):
    assert fn(**over) == want


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is present")
def test_no_device_is_reported_not_launched():
    # valid-looking arguments reach the device check, which fails without a
    # GPU; nothing is dereferenced
    assert _prologue() == 5
    assert _packed() == 5
    assert _dequant() == 5
    assert _dequant(pages=0, cache=None, scale=None) == 5
    assert _norm() == 5 and _rope() == 5 and _quant() == 5
    assert _norm_heads() == 5 and _rope_heads() == 5
    assert _packed_ex() == 5 and _packed_ex(R=0, cs=None) == 5
    # without rotary dims no table is indexed: an empty one is accepted
    assert _packed_ex(R=0, cs=None, maxp=0) == 5
    assert _prologue_scalar() == 5 and _dequant_scalar() == 5
    assert _prologue_scalar(pages=0, cache=None, scale=None) == 5
    assert _copy() == 5 and _rmw() == 5
    assert _paged() == 5 and _paged(pages=0, cache=None, scale=None) == 5
    assert _paged_scalar() == 5
    assert _paged_scalar(pages=0, cache=None, scale=None) == 5
    # the scalar scale is one float: 4-byte alignment is enough
    assert _paged_scalar(scale=FAKE + 4) == 5 and _dequant_scalar(scale=FAKE + 4) == 5


def test_knobs():
    K.set_dispatch_threshold(123)
    assert K.get_dispatch_threshold() == 123
    K.set_dispatch_threshold(-1)
    # no crossover on MI355X: by default every call takes the tiled path,
    # whose default shape is the small-batch shape
    assert K.get_dispatch_threshold() == 0
    assert K.get_tiling() == (1, 1)
    K.set_tiling(4, 2)
    assert K.get_tiling() == (4, 2)
    with pytest.raises(K.Fp8kvError):
        K.set_tiling(3, 5)
    assert K.get_tiling() == (4, 2)
    K.set_tiling(0, 0)


@pytest.mark.parametrize("value,want", [("4096", 4096), ("0", 0), ("-5", None),
                                        ("12x", None), ("", None)])
def test_threshold_from_environment(value, want):
    # a fresh process loads the library with the variable set
    import subprocess
    import sys
    code = ("import ctypes,sys; L=ctypes.CDLL(sys.argv[1]); "
            "L.fp8kv_get_dispatch_threshold.restype=ctypes.c_int64; "
            "print(L.fp8kv_get_dispatch_threshold())")
    env = dict(os.environ, FP8KV_DISPATCH_THRESHOLD=value)
    out = subprocess.run([sys.executable, "-c", code, K.LIB_PATH], env=env,
                         capture_output=True, text=True, check=True).stdout
    env.pop("FP8KV_DISPATCH_THRESHOLD")
    default = subprocess.run([sys.executable, "-c", code, K.LIB_PATH], env=env,
                             capture_output=True, text=True, check=True).stdout
    assert int(out) == (int(default) if want is None else want)


def test_c_driver_builds_and_links():
    # the plain C caller of the library compiles against include/fp8kv.h and
    # resolves libfp8kv.so and the HIP runtime (usage error: no GPU touched)
    import subprocess
    from tests import build_c_driver
    exe = build_c_driver.build()
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 1 and "usage" in r.stderr


def test_binding_rejects_host_tensors():
    x = I.make_dsv4(I.DSV4_WORKLOADS["tiny"], "cpu")
    with pytest.raises(ValueError, match="device tensor"):
        K.qnorm_rope_kv_quant_insert(x["q"], x["kv"], x["q_weight"],
                                     x["kv_weight"], x["cos_sin_cache"],
                                     x["positions"], x["slot_mapping"],
                                     x["kv_cache"], x["kv_scale"], x["eps"])


def test_binding_requires_one_device_per_call():
    # tensors on two different devices never reach the library (it launches on
    # the current device); the check runs before any device is touched
    a, b = torch.zeros(4), torch.zeros(4, device="meta")
    with pytest.raises(ValueError, match="one device"):
        K._call("fp8kv_stream_rmw", (a, b), None, 0, 0, 0)
    assert K._device(a, torch.ones(2)) == a.device


def test_scalar_read_side_bytes():
    # the blockwise count without the 7 exponent bytes per valid row, plus
    # the 4-byte scale
    assert A.dequant_scalar_bytes(10, 7) == A.dequant_bytes(10, 7) - 49 + 4
    assert A.dequant_scalar_bytes(131072, 131072) == 131072 * (8 + 1024 + 576) + 4


def test_byte_accounting_totals():
    # per-token formula applied to each workload's actual slot mapping
    expect = {"tiny": 553_186, "prefill": 4_356_540_416,
              "wide128": 8_651_507_712, "long64": 17_426_155_520}
    for name, total in expect.items():
        w = I.DSV4_WORKLOADS[name]
        written = w.num_tokens - w.num_skipped
        assert A.dsv4_bytes(w.num_tokens, w.num_heads, written) == total, name
    assert A.dsv4_bytes(1024, 64, 973) == 136_061_915
    for T, total in [(1, 13_320), (17, 218_248), (8192, 104_923_648)]:
        assert A.packed_bytes(T, 16, 8, 128) == total


def test_generators_shapes_and_slot_maps():
    for name in ("tiny", "decode"):
        w = I.DSV4_WORKLOADS[name]
        x = I.make_dsv4(w, "cpu")
        sm = x["slot_mapping"].numpy()
        assert (sm == -1).sum() == w.num_skipped
        v = sm[sm >= 0]
        assert len(set(v.tolist())) == len(v) and v.max() < w.num_pages * 64
        assert x["q"].shape == (w.num_tokens, w.num_heads, 512)
        assert int(x["positions"].max()) < w.max_position
    # sequence layout: page-contiguous within each sequence, distinct pages
    w = I.Dsv4Workload("seq", 512, 2, 1024, 16, False, "arange", "sequences", 0,
                       7, num_sequences=4)
    sm = I.make_dsv4(w, "cpu")["slot_mapping"].numpy().reshape(4, 128)
    assert np.all(sm[:, 1:64] - sm[:, :63] == 1)
    pages = sm[:, ::64] // 64
    assert len(set(pages.ravel().tolist())) == 8
    # packed
    p = I.make_packed(I.PACKED_WORKLOADS["packed_t17"], "cpu")
    assert p["qkv"].shape == (17, 32 * 128)
    assert p["cos_sin_cache"].shape == (8192, 128)


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_bench_refuses_more_than_one_gpu(gpus):
    """bench.py measures one GPU: any other --gpus exits with status 2 and a
    message, before touching a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", gpus], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
