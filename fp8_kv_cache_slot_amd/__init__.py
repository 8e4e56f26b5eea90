"""fp8_kv_cache_slot_amd — fused DeepSeek-V4 attention prologue (Q/KV RMSNorm,
RoPE, FP8 E4M3 + UE8M0 blockwise quantisation and paged-cache insert) and the
packed-QKV Q/K norm+RoPE, as hand-written HIP kernels for MI355X (gfx950).

This module is the thin Python binding of ``libfp8kv.so``: it checks that the
torch tensors it is given are device tensors of the right dtype and shape,
passes their device pointers, sizes and the current HIP stream to the C ABI
declared in ``include/fp8kv.h``, and raises on a non-zero status.  Every step
of the computation runs in the library's kernels; there is no fallback.  If
the library has not been built the first call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8kv.so")

HEAD_DIM = 512
ROPE_DIM = 64
PAGE_SIZE = 64
ROW_BYTES = 576
SCALE_BYTES = 8
PACKED_HEAD_DIM = 128

STATUS = {0: "FP8KV_OK", 1: "FP8KV_ERR_NULL", 2: "FP8KV_ERR_SHAPE",
          3: "FP8KV_ERR_UNSUPPORTED", 4: "FP8KV_ERR_ALIGN",
          5: "FP8KV_ERR_DEVICE", 6: "FP8KV_ERR_LAUNCH", 7: "FP8KV_ERR_VALUE"}

EXPORTED = ["qnorm_rope_kv_quant_insert", "qk_norm_rope_packed",
            "kv_cache_gather_dequant", "rms_norm_rows", "rope_rows",
            "qk_norm_rope_packed_ex",
            "qnorm_rope_kv_quant_insert_scalar_scale",
            "kv_cache_gather_dequant_scalar_scale",
            "kv_quant_insert",
            "fp8kv_status_string", "fp8kv_abi_version",
            "fp8kv_set_dispatch_threshold", "fp8kv_get_dispatch_threshold",
            "fp8kv_set_tiling", "fp8kv_get_tiling",
            "fp8kv_stream_copy", "fp8kv_stream_rmw",
            "kv_cache_gather_dequant_paged",
            "kv_cache_gather_dequant_paged_scalar_scale",
            "rms_norm_heads", "rope_neox_heads"]


class Fp8kvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} "
                         f"({lib().fp8kv_status_string(status).decode()})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded ``libfp8kv.so`` with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m fp8_kv_cache_slot_amd.build`"
            " (the HIP kernels are the only implementation)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    L.qnorm_rope_kv_quant_insert.argtypes = [
        P, P, P, P, P, P, P, P, P, I64, I32, I32, I32, I64, I64, I32, F, P]
    L.qnorm_rope_kv_quant_insert.restype = ctypes.c_int
    L.qk_norm_rope_packed.argtypes = [
        P, I64, I32, I32, I32, I32, F, P, P, P, I32, P, I32, I64, P]
    L.qk_norm_rope_packed.restype = ctypes.c_int
    L.qnorm_rope_kv_quant_insert_scalar_scale.argtypes = [
        P, P, P, P, P, P, P, P, P, I64, I32, I32, I32, I64, I64, I32, F, P]
    L.qnorm_rope_kv_quant_insert_scalar_scale.restype = ctypes.c_int
    L.kv_cache_gather_dequant_scalar_scale.argtypes = [P, P, I64, I32, P, I64, P, P]
    L.kv_cache_gather_dequant_scalar_scale.restype = ctypes.c_int
    L.qk_norm_rope_packed_ex.argtypes = [
        P, I64, I32, I32, I32, I32, F, P, P, P, I32, P, I32, I32, I64, P]
    L.qk_norm_rope_packed_ex.restype = ctypes.c_int
    L.kv_cache_gather_dequant.argtypes = [P, P, I64, I32, P, I64, P, P]
    L.kv_cache_gather_dequant.restype = ctypes.c_int
    L.kv_cache_gather_dequant_paged.argtypes = [P, P, I64, I32, P, I32, I32, P, P,
                                                I64, P, P]
    L.kv_cache_gather_dequant_paged.restype = ctypes.c_int
    L.kv_cache_gather_dequant_paged_scalar_scale.argtypes = [
        P, P, I64, I32, P, I32, I32, P, P, I64, P, P]
    L.kv_cache_gather_dequant_paged_scalar_scale.restype = ctypes.c_int
    L.rms_norm_rows.argtypes = [P, P, P, I64, I32, F, P]
    L.rms_norm_rows.restype = ctypes.c_int
    L.rope_rows.argtypes = [P, P, P, I64, I32, I32, I32, I64, P]
    L.rope_rows.restype = ctypes.c_int
    L.kv_quant_insert.argtypes = [P, P, P, P, I64, I64, I32, P]
    L.kv_quant_insert.restype = ctypes.c_int
    L.rms_norm_heads.argtypes = [P, I64, P, P, I64, I32, I32, F, P]
    L.rms_norm_heads.restype = ctypes.c_int
    L.rope_neox_heads.argtypes = [P, P, P, I64, I32, I32, I64, P]
    L.rope_neox_heads.restype = ctypes.c_int
    L.fp8kv_status_string.argtypes = [ctypes.c_int]
    L.fp8kv_status_string.restype = ctypes.c_char_p
    L.fp8kv_abi_version.argtypes = []
    L.fp8kv_abi_version.restype = ctypes.c_int
    L.fp8kv_set_dispatch_threshold.argtypes = [I64]
    L.fp8kv_set_dispatch_threshold.restype = ctypes.c_int
    L.fp8kv_get_dispatch_threshold.argtypes = []
    L.fp8kv_get_dispatch_threshold.restype = I64
    L.fp8kv_set_tiling.argtypes = [I32, I32]
    L.fp8kv_set_tiling.restype = ctypes.c_int
    L.fp8kv_get_tiling.argtypes = [ctypes.POINTER(I32), ctypes.POINTER(I32)]
    L.fp8kv_get_tiling.restype = None
    L.fp8kv_stream_copy.argtypes = [P, P, I64, P]
    L.fp8kv_stream_copy.restype = ctypes.c_int
    L.fp8kv_stream_rmw.argtypes = [P, I64, ctypes.c_uint32, P]
    L.fp8kv_stream_rmw.restype = ctypes.c_int
    _lib = L
    return L


def _check(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _device(*tensors) -> torch.device:
    """The one device every tensor of a call is on (the library launches on
    the current device, so a pointer from another device must never reach
    it)."""
    dev = tensors[0].device
    for t in tensors[1:]:
        if t.device != dev:
            raise ValueError(f"all tensors of a call must be on one device, got "
                             f"{dev} and {t.device}")
    return dev


def _stream(stream, dev) -> int:
    if stream is None:
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        if stream.device != dev:
            raise ValueError(f"stream is on {stream.device}, tensors on {dev}")
        return stream.cuda_stream
    return int(stream)


def _call(name: str, tensors, stream, *args) -> None:
    """Call C entry point ``name`` with ``args`` and the stream, with the
    tensors' device current; raise on a non-zero status."""
    dev = _device(*tensors)
    with torch.cuda.device(dev):
        st = getattr(lib(), name)(*args, _stream(stream, dev))
    if st:
        raise Fp8kvError(st, name)


def qnorm_rope_kv_quant_insert(q, kv, q_weight, kv_weight, cos_sin_cache,
                               positions, slot_mapping, kv_cache, kv_scale,
                               eps: float = 1e-6, stream=None) -> None:
    """Fused DeepSeek-V4 prologue, in place on ``q`` (bf16 [T,H,512]),
    ``kv_cache`` (uint8 [pages,64,576]) and ``kv_scale`` (uint8
    [pages,64,8]).  See ``include/fp8kv.h`` for the exact semantics."""
    if q.dim() != 3:
        raise ValueError("q must be [T, H, 512]")
    T, H, D = q.shape
    _check(q, "q", torch.bfloat16)
    _check(kv, "kv", torch.bfloat16, (T, D))
    _check(q_weight, "q_weight", torch.bfloat16, (D,))
    _check(kv_weight, "kv_weight", torch.bfloat16, (D,))
    _check(cos_sin_cache, "cos_sin_cache", torch.float32)
    if cos_sin_cache.dim() != 2:
        raise ValueError("cos_sin_cache must be [max_position, rope_dim]")
    _check(positions, "positions", torch.int64, (T,))
    _check(slot_mapping, "slot_mapping", torch.int64, (T,))
    _check(kv_cache, "kv_cache", torch.uint8)
    if kv_cache.dim() != 3:
        raise ValueError("kv_cache must be [num_pages, page_size, 576]")
    pages, page_size, row = kv_cache.shape
    if row != ROW_BYTES:
        raise ValueError("kv_cache rows must be 576 bytes")
    _check(kv_scale, "kv_scale", torch.uint8, (pages, page_size, SCALE_BYTES))
    _call("qnorm_rope_kv_quant_insert",
          (q, kv, q_weight, kv_weight, cos_sin_cache, positions, slot_mapping,
           kv_cache, kv_scale), stream,
          q.data_ptr(), kv.data_ptr(), q_weight.data_ptr(), kv_weight.data_ptr(),
          cos_sin_cache.data_ptr(), positions.data_ptr(), slot_mapping.data_ptr(),
          kv_cache.data_ptr(), kv_scale.data_ptr(), T, H, D,
          cos_sin_cache.shape[1], cos_sin_cache.shape[0], pages, page_size,
          float(eps))


def qnorm_rope_kv_quant_insert_scalar_scale(q, kv, q_weight, kv_weight,
                                            cos_sin_cache, positions,
                                            slot_mapping, kv_cache,
                                            kv_cache_scale, eps: float = 1e-6,
                                            stream=None) -> None:
    """The fused prologue writing the scalar-scale FP8 cache: codes of
    y / kv_cache_scale (a one-element fp32 device tensor), no exponents."""
    if q.dim() != 3:
        raise ValueError("q must be [T, H, 512]")
    T, H, D = q.shape
    _check(q, "q", torch.bfloat16)
    _check(kv, "kv", torch.bfloat16, (T, D))
    _check(q_weight, "q_weight", torch.bfloat16, (D,))
    _check(kv_weight, "kv_weight", torch.bfloat16, (D,))
    _check(cos_sin_cache, "cos_sin_cache", torch.float32)
    if cos_sin_cache.dim() != 2:
        raise ValueError("cos_sin_cache must be [max_position, rope_dim]")
    _check(positions, "positions", torch.int64, (T,))
    _check(slot_mapping, "slot_mapping", torch.int64, (T,))
    _check(kv_cache, "kv_cache", torch.uint8)
    if kv_cache.dim() != 3 or kv_cache.shape[2] != ROW_BYTES:
        raise ValueError("kv_cache must be [num_pages, page_size, 576]")
    pages, page_size, _ = kv_cache.shape
    _check(kv_cache_scale, "kv_cache_scale", torch.float32, (1,))
    _call("qnorm_rope_kv_quant_insert_scalar_scale",
          (q, kv, q_weight, kv_weight, cos_sin_cache, positions, slot_mapping,
           kv_cache, kv_cache_scale), stream,
          q.data_ptr(), kv.data_ptr(), q_weight.data_ptr(), kv_weight.data_ptr(),
          cos_sin_cache.data_ptr(), positions.data_ptr(), slot_mapping.data_ptr(),
          kv_cache.data_ptr(), kv_cache_scale.data_ptr(), T, H, D,
          cos_sin_cache.shape[1], cos_sin_cache.shape[0], pages, page_size,
          float(eps))


def kv_cache_gather_dequant_scalar_scale(kv_cache, kv_cache_scale, slots,
                                         out=None, stream=None):
    """Read side of the scalar-scale cache: bf16 [N, 512]."""
    _check(kv_cache, "kv_cache", torch.uint8)
    if kv_cache.dim() != 3 or kv_cache.shape[2] != ROW_BYTES:
        raise ValueError("kv_cache must be [num_pages, page_size, 576]")
    pages, page_size, _ = kv_cache.shape
    _check(kv_cache_scale, "kv_cache_scale", torch.float32, (1,))
    if slots.dim() != 1:
        raise ValueError("slots must be one-dimensional")
    _check(slots, "slots", torch.int64)
    n = slots.shape[0]
    if out is None:
        out = torch.empty((n, HEAD_DIM), dtype=torch.bfloat16, device=slots.device)
    _check(out, "out", torch.bfloat16, (n, HEAD_DIM))
    _call("kv_cache_gather_dequant_scalar_scale",
          (kv_cache, kv_cache_scale, slots, out), stream,
          kv_cache.data_ptr(), kv_cache_scale.data_ptr(), pages, page_size,
          slots.data_ptr(), n, out.data_ptr())
    return out


def qk_norm_rope_packed(qkv, num_heads_q: int, num_heads_k: int,
                        num_heads_v: int, head_dim: int, eps: float, q_weight,
                        k_weight, cos_sin_cache, is_neox: bool, position_ids,
                        forced_token_heads_per_warp: int = -1,
                        stream=None) -> None:
    """Packed-QKV Q/K RMSNorm + NeoX RoPE in place on ``qkv`` (bf16
    [T,(Hq+Hk+Hv)*D]); V heads untouched.  Parameter order as vLLM's
    fused_qk_norm_rope."""
    if qkv.dim() != 2:
        raise ValueError("qkv must be [T, (Hq+Hk+Hv)*D]")
    T = qkv.shape[0]
    _check(qkv, "qkv", torch.bfloat16,
           (T, (num_heads_q + num_heads_k + num_heads_v) * head_dim))
    _check(q_weight, "q_weight", torch.bfloat16, (head_dim,))
    _check(k_weight, "k_weight", torch.bfloat16, (head_dim,))
    _check(cos_sin_cache, "cos_sin_cache", torch.float32)
    if cos_sin_cache.dim() != 2 or cos_sin_cache.shape[1] != head_dim:
        raise ValueError("cos_sin_cache must be [max_position, head_dim]")
    _check(position_ids, "position_ids", torch.int64, (T,))
    _call("qk_norm_rope_packed",
          (qkv, q_weight, k_weight, cos_sin_cache, position_ids), stream,
          qkv.data_ptr(), T, num_heads_q, num_heads_k, num_heads_v, head_dim,
          float(eps), q_weight.data_ptr(), k_weight.data_ptr(),
          cos_sin_cache.data_ptr(), int(bool(is_neox)), position_ids.data_ptr(),
          int(forced_token_heads_per_warp), cos_sin_cache.shape[0])


def qk_norm_rope_packed_ex(qkv, num_heads_q: int, num_heads_k: int,
                           num_heads_v: int, head_dim: int, eps: float,
                           q_weight, k_weight, cos_sin_cache, is_neox: bool,
                           position_ids, rotary_dim: int | None = None,
                           stream=None) -> None:
    """Packed Q/K RMSNorm + RoPE for head_dim 64/128/256, partial rotary
    (``rotary_dim``, default the whole head), NeoX or interleaved pairs, bf16
    or fp16 (the dtype of ``qkv``), in place; V heads untouched."""
    if qkv.dim() != 2:
        raise ValueError("qkv must be [T, (Hq+Hk+Hv)*D]")
    dtypes = {torch.bfloat16: 0, torch.float16: 1}
    if qkv.dtype not in dtypes:
        raise TypeError("qkv must be bfloat16 or float16")
    T = qkv.shape[0]
    R = head_dim if rotary_dim is None else int(rotary_dim)
    _check(qkv, "qkv", qkv.dtype,
           (T, (num_heads_q + num_heads_k + num_heads_v) * head_dim))
    _check(q_weight, "q_weight", qkv.dtype, (head_dim,))
    _check(k_weight, "k_weight", qkv.dtype, (head_dim,))
    _check(cos_sin_cache, "cos_sin_cache", torch.float32)
    if cos_sin_cache.dim() != 2 or cos_sin_cache.shape[1] != R:
        raise ValueError("cos_sin_cache must be [max_position, rotary_dim]")
    _check(position_ids, "position_ids", torch.int64, (T,))
    _call("qk_norm_rope_packed_ex",
          (qkv, q_weight, k_weight, cos_sin_cache, position_ids), stream,
          qkv.data_ptr(), T, num_heads_q, num_heads_k, num_heads_v, head_dim,
          float(eps), q_weight.data_ptr(), k_weight.data_ptr(),
          cos_sin_cache.data_ptr() if R else None, int(bool(is_neox)),
          position_ids.data_ptr(), R, dtypes[qkv.dtype],
          cos_sin_cache.shape[0])


def kv_cache_gather_dequant(kv_cache, kv_scale, slots, out=None,
                            stream=None):
    """Gather rows of the paged FP8/UE8M0 cache by slot and dequantise them
    to bf16 [N, 512]; invalid slots give zero rows.  Returns ``out``."""
    _check(kv_cache, "kv_cache", torch.uint8)
    if kv_cache.dim() != 3 or kv_cache.shape[2] != ROW_BYTES:
        raise ValueError("kv_cache must be [num_pages, page_size, 576]")
    pages, page_size, _ = kv_cache.shape
    _check(kv_scale, "kv_scale", torch.uint8, (pages, page_size, SCALE_BYTES))
    if slots.dim() != 1:
        raise ValueError("slots must be one-dimensional")
    _check(slots, "slots", torch.int64)
    n = slots.shape[0]
    if out is None:
        out = torch.empty((n, HEAD_DIM), dtype=torch.bfloat16, device=slots.device)
    _check(out, "out", torch.bfloat16, (n, HEAD_DIM))
    _call("kv_cache_gather_dequant", (kv_cache, kv_scale, slots, out), stream,
          kv_cache.data_ptr(), kv_scale.data_ptr(), pages, page_size,
          slots.data_ptr(), n, out.data_ptr())
    return out


def kv_cache_gather_dequant_paged(kv_cache, kv_scale, block_table, seq_lens,
                                  out_offsets, out, stream=None):
    """Read the cache through block tables into ``out`` (bf16 [N, 512]):
    token j of sequence s (slot block_table[s, j // 64] * 64 + j % 64) goes
    to row out_offsets[s] + j.  Rows no sequence covers are left as they are.
    Returns ``out``."""
    _check(kv_cache, "kv_cache", torch.uint8)
    if kv_cache.dim() != 3 or kv_cache.shape[2] != ROW_BYTES:
        raise ValueError("kv_cache must be [num_pages, page_size, 576]")
    pages, page_size, _ = kv_cache.shape
    _check(kv_scale, "kv_scale", torch.uint8, (pages, page_size, SCALE_BYTES))
    _check(block_table, "block_table", torch.int32)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [num_seqs, max_blocks_per_seq]")
    S, M = block_table.shape
    _check(seq_lens, "seq_lens", torch.int32, (S,))
    _check(out_offsets, "out_offsets", torch.int64, (S,))
    _check(out, "out", torch.bfloat16)
    if out.dim() != 2 or out.shape[1] != HEAD_DIM:
        raise ValueError("out must be [N, 512]")
    _call("kv_cache_gather_dequant_paged",
          (kv_cache, kv_scale, block_table, seq_lens, out_offsets, out), stream,
          kv_cache.data_ptr(), kv_scale.data_ptr(), pages, page_size,
          block_table.data_ptr(), S, M, seq_lens.data_ptr(), out_offsets.data_ptr(),
          out.shape[0], out.data_ptr())
    return out


def kv_cache_gather_dequant_paged_scalar_scale(kv_cache, kv_cache_scale,
                                               block_table, seq_lens,
                                               out_offsets, out, stream=None):
    """The scalar-scale read side through block tables (the walk of
    :func:`kv_cache_gather_dequant_paged`, rows dequantised with the one
    fp32 scale in ``kv_cache_scale``).  Returns ``out``."""
    _check(kv_cache, "kv_cache", torch.uint8)
    if kv_cache.dim() != 3 or kv_cache.shape[2] != ROW_BYTES:
        raise ValueError("kv_cache must be [num_pages, page_size, 576]")
    pages, page_size, _ = kv_cache.shape
    _check(kv_cache_scale, "kv_cache_scale", torch.float32, (1,))
    _check(block_table, "block_table", torch.int32)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [num_seqs, max_blocks_per_seq]")
    S, M = block_table.shape
    _check(seq_lens, "seq_lens", torch.int32, (S,))
    _check(out_offsets, "out_offsets", torch.int64, (S,))
    _check(out, "out", torch.bfloat16)
    if out.dim() != 2 or out.shape[1] != HEAD_DIM:
        raise ValueError("out must be [N, 512]")
    _call("kv_cache_gather_dequant_paged_scalar_scale",
          (kv_cache, kv_cache_scale, block_table, seq_lens, out_offsets, out), stream,
          kv_cache.data_ptr(), kv_cache_scale.data_ptr(), pages, page_size,
          block_table.data_ptr(), S, M, seq_lens.data_ptr(), out_offsets.data_ptr(),
          out.shape[0], out.data_ptr())
    return out


def rms_norm_rows(x, weight, eps: float = 1e-6, out=None, stream=None):
    """bf16 rows [..., 512] -> normalised, weighted bf16 rows (``out`` may be
    ``x`` for an in-place update).  Returns ``out``."""
    _check(x, "x", torch.bfloat16)
    if x.shape[-1] != HEAD_DIM:
        raise ValueError("rows must be 512 wide")
    _check(weight, "weight", torch.bfloat16, (HEAD_DIM,))
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", torch.bfloat16, tuple(x.shape))
    _call("rms_norm_rows", (x, weight, out), stream,
          x.data_ptr(), out.data_ptr(), weight.data_ptr(),
          x.numel() // HEAD_DIM, HEAD_DIM, float(eps))
    return out


def rope_rows(x, cos_sin_cache, positions, stream=None) -> None:
    """In place: interleaved RoPE on dims 448..511 of bf16 x [T, R, 512]."""
    if x.dim() != 3:
        raise ValueError("x must be [T, rows_per_token, 512]")
    T, R, D = x.shape
    _check(x, "x", torch.bfloat16)
    _check(cos_sin_cache, "cos_sin_cache", torch.float32)
    if cos_sin_cache.dim() != 2:
        raise ValueError("cos_sin_cache must be [max_position, 64]")
    _check(positions, "positions", torch.int64, (T,))
    _call("rope_rows", (x, cos_sin_cache, positions), stream,
          x.data_ptr(), cos_sin_cache.data_ptr(),
          positions.data_ptr(), T, R, D, cos_sin_cache.shape[1],
          cos_sin_cache.shape[0])


def kv_quant_insert(kv, slot_mapping, kv_cache, kv_scale, stream=None) -> None:
    """Quantise already normalised + rotated bf16 KV rows [T, 512] into the
    paged cache (the fused call's quantiser, as its own launch)."""
    if kv.dim() != 2:
        raise ValueError("kv must be [T, 512]")
    T = kv.shape[0]
    _check(kv, "kv", torch.bfloat16, (T, HEAD_DIM))
    _check(slot_mapping, "slot_mapping", torch.int64, (T,))
    _check(kv_cache, "kv_cache", torch.uint8)
    if kv_cache.dim() != 3 or kv_cache.shape[2] != ROW_BYTES:
        raise ValueError("kv_cache must be [num_pages, page_size, 576]")
    pages, page_size, _ = kv_cache.shape
    _check(kv_scale, "kv_scale", torch.uint8, (pages, page_size, SCALE_BYTES))
    _call("kv_quant_insert", (kv, slot_mapping, kv_cache, kv_scale), stream,
          kv.data_ptr(), slot_mapping.data_ptr(),
          kv_cache.data_ptr(), kv_scale.data_ptr(), T,
          pages, page_size)


def unfused_prologue(q, kv, q_weight, kv_weight, cos_sin_cache, positions,
                     slot_mapping, kv_cache, kv_scale, eps: float = 1e-6,
                     kv_work=None, stream=None) -> None:
    """The prologue as five separate launches (norm q, norm kv into a work
    buffer, rope q, rope kv, quantise+insert): the unfused baseline.  Same
    arguments as :func:`qnorm_rope_kv_quant_insert`; ``kv_work`` is an
    optional bf16 [T, 512] scratch tensor."""
    T, H, D = q.shape
    if kv_work is None:
        kv_work = torch.empty((T, D), dtype=torch.bfloat16, device=q.device)
    rms_norm_rows(q, q_weight, eps, out=q, stream=stream)
    rms_norm_rows(kv, kv_weight, eps, out=kv_work, stream=stream)
    rope_rows(q, cos_sin_cache, positions, stream=stream)
    rope_rows(kv_work.view(T, 1, D), cos_sin_cache, positions, stream=stream)
    kv_quant_insert(kv_work, slot_mapping, kv_cache, kv_scale, stream=stream)


def rms_norm_heads(qkv, first_head: int, num_heads: int, head_dim: int, weight,
                   out, eps: float = 1e-6, stream=None):
    """RMSNorm of heads ``first_head .. first_head + num_heads - 1`` of every
    row of ``qkv`` (bf16 [T, W]) into ``out`` (bf16 [T, num_heads,
    head_dim]).  Returns ``out``."""
    if qkv.dim() != 2:
        raise ValueError("qkv must be [T, W]")
    T, W = qkv.shape
    _check(qkv, "qkv", torch.bfloat16)
    if first_head < 0 or num_heads < 0 or (first_head + num_heads) * head_dim > W:
        raise ValueError("heads outside the row")
    _check(weight, "weight", torch.bfloat16, (head_dim,))
    _check(out, "out", torch.bfloat16, (T, num_heads, head_dim))
    _call("rms_norm_heads", (qkv, weight, out), stream,
          qkv.data_ptr() + first_head * head_dim * qkv.element_size(), W,
          out.data_ptr(), weight.data_ptr(), T, num_heads, head_dim, float(eps))
    return out


def rope_neox_heads(x, cos_sin_cache, positions, stream=None) -> None:
    """In place: NeoX RoPE on every head of bf16 ``x`` [T, H, head_dim]."""
    if x.dim() != 3:
        raise ValueError("x must be [T, H, head_dim]")
    T, H, D = x.shape
    _check(x, "x", torch.bfloat16)
    _check(cos_sin_cache, "cos_sin_cache", torch.float32)
    if cos_sin_cache.dim() != 2 or cos_sin_cache.shape[1] != D:
        raise ValueError("cos_sin_cache must be [max_position, head_dim]")
    _check(positions, "positions", torch.int64, (T,))
    _call("rope_neox_heads", (x, cos_sin_cache, positions), stream,
          x.data_ptr(), cos_sin_cache.data_ptr(), positions.data_ptr(), T, H, D,
          cos_sin_cache.shape[0])


def unfused_qk_norm_rope_packed(qkv, num_heads_q: int, num_heads_k: int,
                                num_heads_v: int, head_dim: int, eps: float,
                                q_weight, k_weight, cos_sin_cache, position_ids,
                                q_out=None, k_out=None, stream=None):
    """The packed Q/K norm + NeoX RoPE as four separate launches (RMSNorm of
    the Q heads and of the K heads into ``q_out`` [T, Hq, D] and ``k_out``
    [T, Hk, D], then RoPE of each in place): the separate-launch baseline of
    :func:`qk_norm_rope_packed`.  ``qkv`` is only read.  Returns
    (q_out, k_out)."""
    T = qkv.shape[0]
    if q_out is None:
        q_out = torch.empty((T, num_heads_q, head_dim), dtype=qkv.dtype,
                            device=qkv.device)
    if k_out is None:
        k_out = torch.empty((T, num_heads_k, head_dim), dtype=qkv.dtype,
                            device=qkv.device)
    if qkv.dim() != 2 or qkv.shape[1] != (num_heads_q + num_heads_k + num_heads_v) * head_dim:
        raise ValueError("qkv must be [T, (Hq + Hk + Hv) * head_dim]")
    rms_norm_heads(qkv, 0, num_heads_q, head_dim, q_weight, q_out, eps, stream)
    rms_norm_heads(qkv, num_heads_q, num_heads_k, head_dim, k_weight, k_out, eps,
                   stream)
    rope_neox_heads(q_out, cos_sin_cache, position_ids, stream)
    rope_neox_heads(k_out, cos_sin_cache, position_ids, stream)
    return q_out, k_out


def set_dispatch_threshold(programs: int) -> None:
    lib().fp8kv_set_dispatch_threshold(int(programs))


def get_dispatch_threshold() -> int:
    return lib().fp8kv_get_dispatch_threshold()


def set_tiling(waves_per_block: int, slots_per_wave: int) -> None:
    st = lib().fp8kv_set_tiling(int(waves_per_block), int(slots_per_wave))
    if st:
        raise Fp8kvError(st, "set_tiling")


def get_tiling():
    w, s = ctypes.c_int32(), ctypes.c_int32()
    lib().fp8kv_get_tiling(ctypes.byref(w), ctypes.byref(s))
    return w.value, s.value


def abi_version() -> int:
    return lib().fp8kv_abi_version()


def stream_copy(dst, src, stream=None) -> None:
    """Reference streaming copy (16 bytes per lane): dst[:] = src[:], both
    contiguous device tensors of the same byte size (a multiple of 16)."""
    for t, name in ((dst, "dst"), (src, "src")):
        if not (isinstance(t, torch.Tensor) and t.device.type == "cuda"
                and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    nb = dst.numel() * dst.element_size()
    if src.numel() * src.element_size() != nb:
        raise ValueError("dst and src must have the same byte size")
    _call("fp8kv_stream_copy", (dst, src), stream,
          dst.data_ptr(), src.data_ptr(), nb)


def stream_rmw(buf, mask: int = 0, stream=None) -> None:
    """Reference in-place streaming read-modify-write (16 bytes per lane):
    every 32-bit word of ``buf`` is XORed with ``mask`` (0 keeps the bytes)."""
    if not (isinstance(buf, torch.Tensor) and buf.device.type == "cuda"
            and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous device tensor")
    _call("fp8kv_stream_rmw", (buf,), stream,
          buf.data_ptr(), buf.numel() * buf.element_size(),
          int(mask) & 0xFFFFFFFF)
