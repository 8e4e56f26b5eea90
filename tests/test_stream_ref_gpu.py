"""The reference streaming kernels (the bandwidth ceiling of the benchmark)
on the GPU: exact byte results over ragged sizes, bytes outside the range
untouched."""

import pytest
import torch

import fp8_kv_cache_slot_amd as K

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bytes(n, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g, device=DEV)


@pytest.mark.parametrize("n16", [1, 255, 256, 257, 4097, 100_003])
def test_copy_exact_with_guards(n16):
    src = _bytes(n16 * 16 + 64, n16)
    dst = torch.full((n16 * 16 + 64,), 0x5A, dtype=torch.uint8, device=DEV)
    # a 16-byte aligned window; 32 guard bytes on either side
    K.stream_copy(dst[32:32 + n16 * 16], src[32:32 + n16 * 16])
    torch.cuda.synchronize()
    assert torch.equal(dst[32:32 + n16 * 16], src[32:32 + n16 * 16])
    assert bool((dst[:32] == 0x5A).all()) and bool((dst[32 + n16 * 16:] == 0x5A).all())


# 8_388_608 vectors (128 MiB) and more take the occupancy cap
@pytest.mark.parametrize("n16", [1, 257, 100_003, 8_388_608])
def test_rmw_exact_with_guards(n16):
    buf = _bytes(n16 * 16 + 64, 7 + n16)
    ref = buf.clone()
    win = buf[32:32 + n16 * 16]
    K.stream_rmw(win, 0)
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)
    K.stream_rmw(win, 0xFFFFFFFF)
    torch.cuda.synchronize()
    assert torch.equal(buf[32:32 + n16 * 16], ref[32:32 + n16 * 16] ^ 0xFF)
    assert torch.equal(buf[:32], ref[:32]) and torch.equal(buf[32 + n16 * 16:],
                                                           ref[32 + n16 * 16:])
    w32 = win.view(torch.int32)
    before = w32.clone()
    K.stream_rmw(win, 0x01020304)
    torch.cuda.synchronize()
    assert torch.equal(w32, before ^ 0x01020304)
