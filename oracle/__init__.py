"""CPU oracle for the fused attention prologue (test infrastructure only).

Thin ctypes wrapper around ``liboracle.so`` (built from ``oracle.cpp`` by
``oracle/build.py``).  The oracle is a plain single-threaded double-precision
statement of the operators; only the tests, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  It shares no code
with the GPU library (``fp8_kv_cache_slot_amd``) and never imports it.

Arrays are numpy arrays on the host.  bf16 tensors are passed as ``uint16``
arrays of their bit patterns; the caller owns every buffer.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I64, I32, D = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = D
    lib.oracle_bf16_rne.argtypes = [D]
    lib.oracle_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_fp16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_fp16_to_double.restype = D
    lib.oracle_fp16_rne.argtypes = [D]
    lib.oracle_fp16_rne.restype = ctypes.c_uint16
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = D
    lib.oracle_e4m3_encode.argtypes = [D]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_ue8m0_exponent.argtypes = [D]
    lib.oracle_ue8m0_exponent.restype = I32
    lib.oracle_qnorm_rope_kv_quant_insert.argtypes = [
        P, P, P, P, P, P, P, P, P, I64, I32, I64, D]
    lib.oracle_qnorm_rope_kv_quant_insert.restype = None
    lib.oracle_qnorm_rope_kv_quant_insert_scalar.argtypes = [
        P, P, P, P, P, P, P, P, ctypes.c_float, I64, I32, I64, D]
    lib.oracle_qnorm_rope_kv_quant_insert_scalar.restype = None
    lib.oracle_kv_normalised.argtypes = [P, P, P, P, I64, D, P]
    lib.oracle_kv_normalised.restype = None
    lib.oracle_rms_norm_rows.argtypes = [P, P, P, I64, D]
    lib.oracle_rms_norm_rows.restype = None
    lib.oracle_rope_rows.argtypes = [P, P, P, I64, I32]
    lib.oracle_rope_rows.restype = None
    lib.oracle_kv_quant_insert.argtypes = [P, P, P, P, I64, I64]
    lib.oracle_kv_quant_insert.restype = None
    lib.oracle_kv_cache_gather_dequant.argtypes = [P, P, P, I64, I64, P]
    lib.oracle_kv_cache_gather_dequant_paged.argtypes = [
        P, P, I64, P, I32, I32, P, P, I64, P]
    lib.oracle_kv_cache_gather_dequant_paged.restype = None
    lib.oracle_kv_cache_gather_dequant_scalar.argtypes = [
        P, ctypes.c_float, P, I64, I64, P]
    lib.oracle_kv_cache_gather_dequant_scalar.restype = None
    lib.oracle_kv_cache_gather_dequant_paged_scalar.argtypes = [
        P, ctypes.c_float, I64, P, I32, I32, P, P, I64, P]
    lib.oracle_kv_cache_gather_dequant_paged_scalar.restype = None
    lib.oracle_kv_cache_gather_dequant.restype = None
    lib.oracle_qk_norm_rope_packed.argtypes = [
        P, I64, I32, I32, I32, I32, D, P, P, P, P]
    lib.oracle_qk_norm_rope_packed.restype = None
    lib.oracle_qk_norm_rope_packed_ex.argtypes = [
        P, I64, I32, I32, I32, I32, I32, I32, I32, D, P, P, P, P]
    lib.oracle_qk_norm_rope_packed_ex.restype = None
    lib.oracle_rms_norm_heads.argtypes = [P, I64, P, P, I64, I32, I32, D]
    lib.oracle_rms_norm_heads.restype = None
    lib.oracle_rope_neox_heads.argtypes = [P, P, P, I64, I32, I32]
    lib.oracle_rope_neox_heads.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray, dtype, writable=False):
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    if not a.flags.c_contiguous:
        raise ValueError("array must be C-contiguous")
    if writable and not a.flags.writeable:
        raise ValueError("array must be writeable")
    return a.ctypes.data_as(ctypes.c_void_p)


# ---- number formats ---------------------------------------------------------

def bf16_to_double(bits: int) -> float:
    return _load().oracle_bf16_to_double(int(bits))


def bf16_rne(v: float) -> int:
    return _load().oracle_bf16_rne(float(v))


def fp16_to_double(bits: int) -> float:
    return _load().oracle_fp16_to_double(int(bits))


def fp16_rne(v: float) -> int:
    return _load().oracle_fp16_rne(float(v))


def e4m3_decode(code: int) -> float:
    return _load().oracle_e4m3_decode(int(code))


def e4m3_encode(v: float) -> int:
    return _load().oracle_e4m3_encode(float(v))


def ue8m0_exponent(amax: float) -> int:
    return _load().oracle_ue8m0_exponent(float(amax))


# ---- entry points -----------------------------------------------------------

def qnorm_rope_kv_quant_insert(q, kv, q_weight, kv_weight, cos_sin_cache,
                               positions, slot_mapping, kv_cache, kv_scale,
                               eps):
    """In place on ``q`` (uint16 [T,H,512]), ``kv_cache`` (uint8
    [pages,64,576]) and ``kv_scale`` (uint8 [pages,64,8])."""
    T, H, D = q.shape
    if D != 512 or kv.shape != (T, 512):
        raise ValueError("q must be [T,H,512] and kv [T,512]")
    if cos_sin_cache.ndim != 2 or cos_sin_cache.shape[1] != 64:
        raise ValueError("cos_sin_cache must be [max_position, 64]")
    if positions.shape != (T,) or slot_mapping.shape != (T,):
        raise ValueError("positions and slot_mapping must be [T]")
    pages = kv_cache.shape[0]
    if kv_cache.shape != (pages, 64, 576) or kv_scale.shape != (pages, 64, 8):
        raise ValueError("cache must be [pages,64,576], scale [pages,64,8]")
    if T and (positions.min() < 0 or positions.max() >= cos_sin_cache.shape[0]):
        raise ValueError("position out of range")
    _load().oracle_qnorm_rope_kv_quant_insert(
        _ptr(q, np.uint16, True), _ptr(kv, np.uint16), _ptr(q_weight, np.uint16),
        _ptr(kv_weight, np.uint16), _ptr(cos_sin_cache, np.float32),
        _ptr(positions, np.int64), _ptr(slot_mapping, np.int64),
        _ptr(kv_cache, np.uint8, True), _ptr(kv_scale, np.uint8, True),
        T, H, pages, float(eps))


def qnorm_rope_kv_quant_insert_scalar(q, kv, q_weight, kv_weight,
                                      cos_sin_cache, positions, slot_mapping,
                                      kv_cache, kv_cache_scale, eps):
    """Scalar-scale cache convention: in place on ``q`` and ``kv_cache``
    (uint8 [pages,64,576]); no exponent tensor."""
    T, H, D = q.shape
    if D != 512 or kv.shape != (T, 512):
        raise ValueError("q must be [T,H,512] and kv [T,512]")
    if positions.shape != (T,) or slot_mapping.shape != (T,):
        raise ValueError("positions and slot_mapping must be [T]")
    pages = kv_cache.shape[0]
    if kv_cache.shape != (pages, 64, 576):
        raise ValueError("cache must be [pages,64,576]")
    if not (kv_cache_scale > 0 and np.isfinite(kv_cache_scale)):
        raise ValueError("kv_cache_scale must be positive and finite")
    if T and (positions.min() < 0 or positions.max() >= cos_sin_cache.shape[0]):
        raise ValueError("position out of range")
    _load().oracle_qnorm_rope_kv_quant_insert_scalar(
        _ptr(q, np.uint16, True), _ptr(kv, np.uint16), _ptr(q_weight, np.uint16),
        _ptr(kv_weight, np.uint16), _ptr(cos_sin_cache, np.float32),
        _ptr(positions, np.int64), _ptr(slot_mapping, np.int64),
        _ptr(kv_cache, np.uint8, True), float(kv_cache_scale), T, H, pages,
        float(eps))


def kv_normalised(kv, kv_weight, cos_sin_cache, positions, eps):
    """Unrounded normalised + rotated KV rows, float64 [T, 512]."""
    T = kv.shape[0]
    if kv.shape != (T, 512) or positions.shape != (T,):
        raise ValueError("kv must be [T,512], positions [T]")
    if T and (positions.min() < 0 or positions.max() >= cos_sin_cache.shape[0]):
        raise ValueError("position out of range")
    y = np.empty((T, 512), np.float64)
    _load().oracle_kv_normalised(
        _ptr(kv, np.uint16), _ptr(kv_weight, np.uint16),
        _ptr(cos_sin_cache, np.float32), _ptr(positions, np.int64), T,
        float(eps), _ptr(y, np.float64, True))
    return y


def rms_norm_rows(x, weight, eps):
    """bf16 [..., 512] -> new array of normalised, weighted bf16 rows."""
    if x.shape[-1] != 512 or weight.shape != (512,):
        raise ValueError("rows must be 512 wide")
    x = np.ascontiguousarray(x, np.uint16)
    out = np.empty_like(x)
    _load().oracle_rms_norm_rows(_ptr(x, np.uint16), _ptr(weight, np.uint16),
                                 _ptr(out, np.uint16, True), x.size // 512, float(eps))
    return out


def rope_rows(x, cos_sin_cache, positions):
    """In place on bf16 x [T, rows_per_token, 512] (rotary dims 448..511)."""
    T, R, D = x.shape
    if D != 512 or positions.shape != (T,) or cos_sin_cache.shape[1] != 64:
        raise ValueError("x must be [T, R, 512], cache [max_pos, 64]")
    if T and (positions.min() < 0 or positions.max() >= cos_sin_cache.shape[0]):
        raise ValueError("position out of range")
    _load().oracle_rope_rows(_ptr(x, np.uint16, True), _ptr(cos_sin_cache, np.float32),
                             _ptr(positions, np.int64), T, R)


def kv_quant_insert(kv, slot_mapping, kv_cache, kv_scale):
    """Quantise already normalised + rotated bf16 rows kv [T, 512] into the
    cache (in place on kv_cache / kv_scale)."""
    T = kv.shape[0]
    pages = kv_cache.shape[0]
    if kv.shape != (T, 512) or slot_mapping.shape != (T,):
        raise ValueError("kv must be [T, 512], slot_mapping [T]")
    if kv_cache.shape != (pages, 64, 576) or kv_scale.shape != (pages, 64, 8):
        raise ValueError("cache must be [pages,64,576], scale [pages,64,8]")
    _load().oracle_kv_quant_insert(_ptr(kv, np.uint16), _ptr(slot_mapping, np.int64),
                                   _ptr(kv_cache, np.uint8, True),
                                   _ptr(kv_scale, np.uint8, True), T, pages)


def kv_cache_gather_dequant(kv_cache, kv_scale, slots):
    """bf16 bit patterns [N, 512] of the dequantised rows of ``slots``."""
    pages = kv_cache.shape[0]
    if kv_cache.shape != (pages, 64, 576) or kv_scale.shape != (pages, 64, 8):
        raise ValueError("cache must be [pages,64,576], scale [pages,64,8]")
    slots = np.ascontiguousarray(slots, np.int64)
    out = np.empty((slots.shape[0], 512), np.uint16)
    _load().oracle_kv_cache_gather_dequant(
        _ptr(kv_cache, np.uint8), _ptr(kv_scale, np.uint8), _ptr(slots, np.int64),
        slots.shape[0], pages, _ptr(out, np.uint16, True))
    return out


def kv_cache_gather_dequant_paged(kv_cache, kv_scale, block_table, seq_lens,
                                  out_offsets, out):
    """Block-table read side, in place on ``out`` (uint16 [N, 512]): token j
    of sequence s (slot block_table[s, j // 64] * 64 + j % 64) goes to row
    out_offsets[s] + j; rows no sequence covers are left as they are."""
    pages = kv_cache.shape[0]
    if kv_cache.shape != (pages, 64, 576) or kv_scale.shape != (pages, 64, 8):
        raise ValueError("cache must be [pages,64,576], scale [pages,64,8]")
    block_table = np.ascontiguousarray(block_table, np.int32)
    if block_table.ndim != 2:
        raise ValueError("block_table must be [num_seqs, max_blocks_per_seq]")
    S, M = block_table.shape
    seq_lens = np.ascontiguousarray(seq_lens, np.int32)
    out_offsets = np.ascontiguousarray(out_offsets, np.int64)
    if seq_lens.shape != (S,) or out_offsets.shape != (S,):
        raise ValueError("seq_lens and out_offsets must be [num_seqs]")
    if out.ndim != 2 or out.shape[1] != 512:
        raise ValueError("out must be [N, 512]")
    _load().oracle_kv_cache_gather_dequant_paged(
        _ptr(kv_cache, np.uint8), _ptr(kv_scale, np.uint8), pages,
        _ptr(block_table, np.int32), S, M, _ptr(seq_lens, np.int32),
        _ptr(out_offsets, np.int64), out.shape[0], _ptr(out, np.uint16, True))
    return out


def kv_cache_gather_dequant_scalar(kv_cache, kv_cache_scale, slots):
    """Scalar-scale read side: bf16 bit patterns [N, 512]."""
    pages = kv_cache.shape[0]
    if kv_cache.shape != (pages, 64, 576):
        raise ValueError("cache must be [pages,64,576]")
    slots = np.ascontiguousarray(slots, np.int64)
    out = np.empty((slots.shape[0], 512), np.uint16)
    _load().oracle_kv_cache_gather_dequant_scalar(
        _ptr(kv_cache, np.uint8), float(kv_cache_scale), _ptr(slots, np.int64),
        slots.shape[0], pages, _ptr(out, np.uint16, True))
    return out


def kv_cache_gather_dequant_paged_scalar(kv_cache, kv_cache_scale, block_table,
                                         seq_lens, out_offsets, out):
    """Scalar-scale read side through block tables, in place on ``out``
    (uint16 [N, 512]); the walk of :func:`kv_cache_gather_dequant_paged`."""
    pages = kv_cache.shape[0]
    if kv_cache.shape != (pages, 64, 576):
        raise ValueError("cache must be [pages,64,576]")
    block_table = np.ascontiguousarray(block_table, np.int32)
    if block_table.ndim != 2:
        raise ValueError("block_table must be [num_seqs, max_blocks_per_seq]")
    S, M = block_table.shape
    seq_lens = np.ascontiguousarray(seq_lens, np.int32)
    out_offsets = np.ascontiguousarray(out_offsets, np.int64)
    if seq_lens.shape != (S,) or out_offsets.shape != (S,):
        raise ValueError("seq_lens and out_offsets must be [num_seqs]")
    if out.ndim != 2 or out.shape[1] != 512:
        raise ValueError("out must be [N, 512]")
    _load().oracle_kv_cache_gather_dequant_paged_scalar(
        _ptr(kv_cache, np.uint8), float(kv_cache_scale), pages,
        _ptr(block_table, np.int32), S, M, _ptr(seq_lens, np.int32),
        _ptr(out_offsets, np.int64), out.shape[0], _ptr(out, np.uint16, True))
    return out


def qk_norm_rope_packed(qkv, num_heads_q, num_heads_k, num_heads_v, head_dim,
                        eps, q_weight, k_weight, cos_sin_cache, position_ids):
    """In place on ``qkv`` (uint16 [T,(Hq+Hk+Hv)*D]); V heads untouched."""
    T = qkv.shape[0]
    if qkv.shape[1] != (num_heads_q + num_heads_k + num_heads_v) * head_dim:
        raise ValueError("qkv width does not match the head counts")
    if head_dim % 2 or cos_sin_cache.shape[1] != head_dim:
        raise ValueError("cos_sin_cache must be [max_position, head_dim]")
    if position_ids.shape != (T,):
        raise ValueError("position_ids must be [T]")
    if T and (position_ids.min() < 0
              or position_ids.max() >= cos_sin_cache.shape[0]):
        raise ValueError("position out of range")
    _load().oracle_qk_norm_rope_packed(
        _ptr(qkv, np.uint16, True), T, num_heads_q, num_heads_k, num_heads_v,
        head_dim, float(eps), _ptr(q_weight, np.uint16),
        _ptr(k_weight, np.uint16), _ptr(cos_sin_cache, np.float32),
        _ptr(position_ids, np.int64))


def qk_norm_rope_packed_ex(qkv, num_heads_q, num_heads_k, num_heads_v,
                           head_dim, rotary_dim, is_neox, is_fp16, eps,
                           q_weight, k_weight, cos_sin_cache, position_ids):
    """In place on ``qkv`` (uint16 bit patterns of bf16 or fp16
    [T,(Hq+Hk+Hv)*D]); V heads untouched."""
    T = qkv.shape[0]
    if qkv.shape[1] != (num_heads_q + num_heads_k + num_heads_v) * head_dim:
        raise ValueError("qkv width does not match the head counts")
    if rotary_dim % 2 or rotary_dim > head_dim or cos_sin_cache.shape[1] != rotary_dim:
        raise ValueError("cos_sin_cache must be [max_position, rotary_dim]")
    if position_ids.shape != (T,):
        raise ValueError("position_ids must be [T]")
    if T and rotary_dim and (position_ids.min() < 0
                             or position_ids.max() >= cos_sin_cache.shape[0]):
        raise ValueError("position out of range")
    _load().oracle_qk_norm_rope_packed_ex(
        _ptr(qkv, np.uint16, True), T, num_heads_q, num_heads_k, num_heads_v,
        head_dim, rotary_dim, int(is_neox), int(is_fp16), float(eps),
        _ptr(q_weight, np.uint16), _ptr(k_weight, np.uint16),
        _ptr(cos_sin_cache, np.float32), _ptr(position_ids, np.int64))


def rms_norm_heads(qkv, first_head, num_heads, head_dim, weight, eps):
    """Separate-launch RMSNorm of heads first_head .. first_head+num_heads-1
    of every row of ``qkv`` (uint16 [T, W]) -> new uint16 [T, num_heads,
    head_dim]."""
    T, W = qkv.shape
    if first_head < 0 or num_heads < 0 or (first_head + num_heads) * head_dim > W:
        raise ValueError("heads outside the row")
    if weight.shape != (head_dim,):
        raise ValueError("weight must be [head_dim]")
    out = np.empty((T, num_heads, head_dim), np.uint16)
    lib = _load()
    _ptr(qkv, np.uint16)
    base = qkv.ctypes.data + first_head * head_dim * 2
    lib.oracle_rms_norm_heads(ctypes.c_void_p(base), W, _ptr(weight, np.uint16),
                              _ptr(out, np.uint16, True), T, num_heads, head_dim,
                              float(eps))
    return out


def rope_neox_heads(x, cos_sin_cache, positions):
    """Separate-launch NeoX RoPE, in place on ``x`` (uint16 [T, H, D])."""
    T, H, D = x.shape
    if cos_sin_cache.ndim != 2 or cos_sin_cache.shape[1] != D or D % 2:
        raise ValueError("cos_sin_cache must be [max_position, head_dim]")
    if positions.shape != (T,):
        raise ValueError("positions must be [T]")
    if T and (positions.min() < 0 or positions.max() >= cos_sin_cache.shape[0]):
        raise ValueError("position out of range")
    _load().oracle_rope_neox_heads(_ptr(x, np.uint16, True),
                                   _ptr(cos_sin_cache, np.float32),
                                   _ptr(positions, np.int64), T, H, D)
