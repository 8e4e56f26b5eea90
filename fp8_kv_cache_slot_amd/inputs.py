"""Seeded synthetic inputs for the fused attention prologue and the packed
Q/K norm+RoPE.

This module only draws random numbers and lays them out; it holds none of the
operators' arithmetic.  Both the GPU library's tests/benchmark and the CPU
oracle's tests take their inputs from here, so parity always compares the two
on the same bytes.

Generation runs on whatever device is asked for (``torch.Generator`` of that
device), token chunk by token chunk, so multi-GiB inputs are drawn on the GPU
without host memory.  Values for a given seed are reproducible per device;
parity never needs CPU and GPU draws to agree because inputs are copied to the
host from the device they were drawn on.

Workloads (tokens x heads, head width 512, one latent KV head per token):
  tiny       16 x 16,      outliers, positions U[0,4096),   4 pages, 2 skipped
  decode     1024 x 64,    outliers, positions U[0,32768), 256 pages, 5% skipped
  prefill    32768 x 64,   outliers, positions arange, 1024 pages, 8 sequences
             of 4096 tokens written page-contiguously in seeded page order
  wide128    32768 x 128,  N(0,1), positions U[0,131072), 2048 pages
  long64     131072 x 64,  N(0,1), positions U[0,131072), 2048 pages, every
             slot of the cache written (a full permutation)
Packed workloads: qkv [T, (16+8+8)*128] for T in {1, 17, 1024, 4096, 8192}
(1024, 4096 and 8192 are the token counts InfiniOps PR #1019 "Benchmark /
Performance Impact" measures).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

HEAD_DIM = 512
ROPE_DIM = 64
PAGE_SIZE = 64
ROW_BYTES = 576
SCALE_BYTES = 8
THETA = 10000.0

CACHE_CANARY = 0xA5   # fill byte of kv_cache before a call
SCALE_CANARY = 0xEE   # fill byte of kv_scale before a call


@dataclasses.dataclass(frozen=True)
class Dsv4Workload:
    name: str
    num_tokens: int
    num_heads: int
    max_position: int
    num_pages: int
    outliers: bool          # 1% of q/kv entries scaled by 50
    positions: str          # "uniform" | "arange"
    slots: str              # "random" | "sequences" | "permutation"
    num_skipped: int        # slot_mapping entries set to -1 ("random" only)
    seed: int
    num_sequences: int = 1  # "sequences" only
    eps: float = 1e-6


@dataclasses.dataclass(frozen=True)
class PackedWorkload:
    name: str
    num_tokens: int
    num_heads_q: int = 16
    num_heads_k: int = 8
    num_heads_v: int = 8
    head_dim: int = 128
    max_position: int = 8192
    seed: int = 1004
    eps: float = 1e-6


DSV4_WORKLOADS = {
    w.name: w
    for w in [
        Dsv4Workload("tiny", 16, 16, 4096, 4, True, "uniform", "random", 2, 1000),
        Dsv4Workload("decode", 1024, 64, 32768, 256, True, "uniform", "random",
                     51, 1001),
        Dsv4Workload("prefill", 32768, 64, 32768, 1024, True, "arange",
                     "sequences", 0, 1002, num_sequences=8),
        Dsv4Workload("wide128", 32768, 128, 131072, 2048, False, "uniform",
                     "random", 0, 1003),
        Dsv4Workload("long64", 131072, 64, 131072, 2048, False, "uniform",
                     "permutation", 0, 1013),
    ]
}

PACKED_WORKLOADS = {
    w.name: w
    for w in [
        PackedWorkload("packed_t1", 1, seed=1004),
        PackedWorkload("packed_t17", 17, seed=1014),
        PackedWorkload("packed_t1024", 1024, seed=1044),
        PackedWorkload("packed_t4096", 4096, seed=1054),
        PackedWorkload("packed_t8192", 8192, seed=1024),
    ]
}


def custom_dsv4(num_tokens, num_heads, seed, *, num_pages=None, outliers=True,
                max_position=4096, skipped=None, name="custom"):
    """A workload of any size with the tiny/decode layout (random injective
    slots, a few skipped, uniform positions)."""
    if num_pages is None:
        num_pages = max(1, math.ceil(num_tokens * 2 / PAGE_SIZE))
    if skipped is None:
        skipped = min(num_tokens, max(0, num_tokens // 20))
    return Dsv4Workload(name, num_tokens, num_heads, max_position, num_pages,
                        outliers, "uniform", "random", skipped, seed)


# ---------------------------------------------------------------------------
# primitive draws
# ---------------------------------------------------------------------------

def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _activations(g, shape, outliers, device, chunk_rows=2048):
    """bf16 N(0,1) with 1% of entries scaled by 50 when ``outliers``, drawn in
    chunks along dim 0 to bound the fp32 temporaries."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    n = shape[0]
    for s in range(0, n, chunk_rows):
        e = min(n, s + chunk_rows)
        x = torch.randn((e - s,) + tuple(shape[1:]), generator=g,
                        device=device, dtype=torch.float32)
        if outliers:
            m = torch.rand(x.shape, generator=g, device=device) < 0.01
            x = torch.where(m, x * 50.0, x)
        out[s:e].copy_(x.to(torch.bfloat16))
        del x
    return out


def _weights(g, n, device):
    w = torch.rand(n, generator=g, device=device, dtype=torch.float32) + 0.5
    return w.to(torch.bfloat16)


def cos_sin_cache(max_position, rot_dim, theta=THETA, device="cpu"):
    """fp32 [max_position, rot_dim]: row p = cos(p f_i) for i < rot_dim/2, then
    sin(p f_i), with f_i = theta^(-2i/rot_dim), evaluated in float64 on the
    host.  The table is an input of the operators, not part of them."""
    half = rot_dim // 2
    inv_freq = theta ** (-(np.arange(half, dtype=np.float64) * 2.0) / rot_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv_freq[None, :]
    tab = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    return torch.from_numpy(np.ascontiguousarray(tab)).to(device)


def _slot_mapping(w: Dsv4Workload, g, device):
    T = w.num_tokens
    num_slots = w.num_pages * PAGE_SIZE
    if w.slots == "random" or w.slots == "permutation":
        if T > num_slots:
            raise ValueError("more tokens than cache slots")
        sm = torch.randperm(num_slots, generator=g, device=device)[:T]
        sm = sm.to(torch.int64)
        if w.num_skipped:
            idx = torch.randperm(T, generator=g, device=device)[: w.num_skipped]
            sm[idx] = -1
        return sm
    if w.slots == "sequences":
        per_seq = T // w.num_sequences
        if per_seq * w.num_sequences != T or per_seq % PAGE_SIZE:
            raise ValueError("sequences must tile whole pages")
        pages_per_seq = per_seq // PAGE_SIZE
        if pages_per_seq * w.num_sequences > w.num_pages:
            raise ValueError("not enough pages")
        perm = torch.randperm(w.num_pages, generator=g, device=device)
        j = torch.arange(per_seq, device=device)
        rows = []
        for s in range(w.num_sequences):
            page = perm[s * pages_per_seq + j // PAGE_SIZE]
            rows.append(page * PAGE_SIZE + j % PAGE_SIZE)
        return torch.cat(rows).to(torch.int64)
    raise ValueError(w.slots)


def _positions(w, g, device):
    if w.positions == "arange":
        if w.num_tokens > w.max_position:
            raise ValueError("arange positions exceed the cos/sin table")
        return torch.arange(w.num_tokens, device=device, dtype=torch.int64)
    return torch.randint(0, w.max_position, (w.num_tokens,), generator=g,
                         device=device, dtype=torch.int64)


def make_dsv4(w: Dsv4Workload, device="cpu"):
    """All inputs of one call, on ``device``.  kv_cache / kv_scale are filled
    with canary bytes so untouched slots can be recognised."""
    g = _gen(device, w.seed)
    T, H = w.num_tokens, w.num_heads
    q = _activations(g, (T, H, HEAD_DIM), w.outliers, device)
    kv = _activations(g, (T, HEAD_DIM), w.outliers, device)
    q_weight = _weights(g, HEAD_DIM, device)
    kv_weight = _weights(g, HEAD_DIM, device)
    positions = _positions(w, g, device)
    slot_mapping = _slot_mapping(w, g, device)
    kv_cache = torch.full((w.num_pages, PAGE_SIZE, ROW_BYTES), CACHE_CANARY,
                          dtype=torch.uint8, device=device)
    kv_scale = torch.full((w.num_pages, PAGE_SIZE, SCALE_BYTES), SCALE_CANARY,
                          dtype=torch.uint8, device=device)
    return dict(q=q, kv=kv, q_weight=q_weight, kv_weight=kv_weight,
                cos_sin_cache=cos_sin_cache(w.max_position, ROPE_DIM,
                                            device=device),
                positions=positions, slot_mapping=slot_mapping,
                kv_cache=kv_cache, kv_scale=kv_scale, eps=w.eps)


def make_packed(w: PackedWorkload, device="cpu"):
    g = _gen(device, w.seed)
    width = (w.num_heads_q + w.num_heads_k + w.num_heads_v) * w.head_dim
    qkv = _activations(g, (w.num_tokens, width), False, device)
    q_weight = _weights(g, w.head_dim, device)
    k_weight = _weights(g, w.head_dim, device)
    position_ids = torch.randint(0, w.max_position, (w.num_tokens,),
                                 generator=g, device=device, dtype=torch.int64)
    return dict(qkv=qkv, q_weight=q_weight, k_weight=k_weight,
                cos_sin_cache=cos_sin_cache(w.max_position, w.head_dim,
                                            device=device),
                position_ids=position_ids, eps=w.eps,
                num_heads_q=w.num_heads_q, num_heads_k=w.num_heads_k,
                num_heads_v=w.num_heads_v, head_dim=w.head_dim)


def bits(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a tensor's bytes: bf16 -> uint16 bit patterns,
    other dtypes unchanged.  Copies to the host if needed."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def from_bits(a: np.ndarray, device="cpu") -> torch.Tensor:
    """Inverse of :func:`bits` for uint16 arrays (-> bf16 tensor)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)
