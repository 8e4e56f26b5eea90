"""The C ABI from a plain C program (tests/c_abi_driver, built by
__graft_entry__.build()): no Python or torch in the calling process, device
memory from hipMalloc, a HIP stream of the caller's own.  Its outputs are
compared with the CPU oracle by the same rules as the Python-side parity."""

import os
import subprocess

import numpy as np
import pytest
import torch

import oracle as O
from fp8_kv_cache_slot_amd import inputs as I
from tests import parity as P

pytestmark = pytest.mark.gpu
# FP8KV_C_DRIVER names another build of the driver (e.g. the CMake one).
DRIVER = os.environ.get(
    "FP8KV_C_DRIVER",
    os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_driver"))


@pytest.mark.parametrize("T,H,seed", [(16, 16, 6000), (40, 64, 6001), (9, 7, 6002)])
def test_c_caller_matches_oracle(tmp_path, T, H, seed):
    assert os.path.exists(DRIVER), f"{DRIVER} is not built (run build())"
    w = I.custom_dsv4(T, H, seed=seed, max_position=512)
    x = {k: (I.bits(v).copy() if isinstance(v, torch.Tensor) else v)
         for k, v in I.make_dsv4(w, "cpu").items()}
    pages = x["kv_cache"].shape[0]
    maxp = x["cos_sin_cache"].shape[0]
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([T, H, pages, maxp], np.int64).tobytes())
        f.write(np.array([w.eps], np.float64).tobytes())
        for k in ("q", "kv", "q_weight", "kv_weight", "cos_sin_cache", "positions",
                  "slot_mapping", "kv_cache", "kv_scale"):
            f.write(np.ascontiguousarray(x[k]).tobytes())
    r = subprocess.run([DRIVER, str(src), str(dst)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(dst, np.uint8)
    nq = T * H * 512 * 2
    nc = pages * 64 * 576
    ns = pages * 64 * 8
    q = raw[:nq].view(np.uint16).reshape(T, H, 512)
    cache = raw[nq:nq + nc].reshape(pages, 64, 576)
    scale = raw[nq + nc:nq + nc + ns].reshape(pages, 64, 8)
    readback = raw[nq + nc + ns:].view(np.uint16).reshape(pages * 64, 512)

    ref = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in x.items()}
    O.qnorm_rope_kv_quant_insert(ref["q"], ref["kv"], ref["q_weight"],
                                 ref["kv_weight"], ref["cos_sin_cache"],
                                 ref["positions"], ref["slot_mapping"],
                                 ref["kv_cache"], ref["kv_scale"], ref["eps"])
    P.check_bf16(q, ref["q"], "C caller q")
    v = P.valid_slots(x["slot_mapping"], pages * 64)
    y = O.kv_normalised(x["kv"][v].copy(), x["kv_weight"], x["cos_sin_cache"],
                        x["positions"][v].copy(), w.eps)
    P.check_cache(cache, scale, ref["kv_cache"], ref["kv_scale"],
                  x["slot_mapping"][v], y, I.CACHE_CANARY, I.SCALE_CANARY,
                  "C caller cache")
    P.check_untouched(cache, scale, x["slot_mapping"][v], I.CACHE_CANARY,
                      I.SCALE_CANARY, "C caller")
    # the C caller's block-table read-back of the cache it wrote equals the
    # oracle's read of those same bytes, bit for bit
    want = np.zeros((pages * 64, 512), np.uint16)
    O.kv_cache_gather_dequant_paged(cache.copy(), scale.copy(),
                                    np.arange(pages, dtype=np.int32)[None, :],
                                    np.array([pages * 64], np.int32),
                                    np.array([0], np.int64), want)
    np.testing.assert_array_equal(readback, want)
