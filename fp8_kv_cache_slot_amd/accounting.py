"""Algorithmic byte counts: the bytes each operator must move, read plus write,
with every input read once.  Used to turn a kernel time into HBM GB/s.

Fused prologue, per token: q read + written (2 * 2 * H * 512 B), the position
and the slot index (8 + 8 B), one cos/sin row shared by all heads (64 fp32 =
256 B); per token whose slot is written: the kv row (1024 B), 448 code bytes,
the 64 bf16 rotary dims (128 B) and 7 exponent bytes; plus both weight vectors
once (2 * 1024 B).

The scalar-scale cache convention moves the same bytes minus the 7
exponent bytes per written token or read row (plus one 4-byte scale).

Cache read side (gather + dequantise), per output row: the slot index (8 B)
and the bf16 row written (1024 B); per row whose slot is valid also the 576
cache bytes and the 7 exponent bytes read.

Packed Q/K norm+RoPE, per token: the Q and K heads read + written
(2 * 2 * (Hq + Hk) * D B), the position (8 B) and one cos/sin row (4 * D B);
the V heads are never touched; plus both weight vectors once (2 * 2 * D B).
"""

from __future__ import annotations

HEAD_DIM = 512
ROPE_DIM = 64


def dsv4_token_bytes(num_heads: int, slot_written: bool) -> int:
    b = 4 * num_heads * HEAD_DIM + 8 + 8 + 4 * ROPE_DIM
    if slot_written:
        b += 2 * HEAD_DIM + 448 + 2 * ROPE_DIM + 7
    return b


def dsv4_bytes(num_tokens: int, num_heads: int, num_written: int) -> int:
    return (num_tokens * dsv4_token_bytes(num_heads, False)
            + num_written * (dsv4_token_bytes(num_heads, True)
                             - dsv4_token_bytes(num_heads, False))
            + 2 * 2 * HEAD_DIM)


def packed_bytes(num_tokens: int, num_heads_q: int, num_heads_k: int,
                 head_dim: int, rotary_dim: int | None = None) -> int:
    """Per token: Q and K heads read + written (2-byte elements), the
    position, one cos/sin row of rotary_dim fp32 (default the whole head)."""
    r = head_dim if rotary_dim is None else rotary_dim
    per_token = 4 * (num_heads_q + num_heads_k) * head_dim + 8 + 4 * r
    return num_tokens * per_token + 2 * 2 * head_dim


def dequant_bytes(num_rows: int, num_valid: int) -> int:
    return num_rows * (8 + 2 * HEAD_DIM) + num_valid * (448 + 2 * ROPE_DIM + 7)


def dequant_paged_bytes(num_rows: int, num_valid: int, table_entries: int,
                        num_seqs: int) -> int:
    """Block-table read side: per row the bf16 output (and the cache row and
    exponents when its page is valid); the block table (4 B per entry read)
    and a length (4 B) and output offset (8 B) per sequence."""
    return (num_rows * 2 * HEAD_DIM + num_valid * (448 + 2 * ROPE_DIM + 7)
            + 4 * table_entries + 12 * num_seqs)


def dsv4_scalar_bytes(num_tokens: int, num_heads: int, num_written: int) -> int:
    return dsv4_bytes(num_tokens, num_heads, num_written) - 7 * num_written + 4


def dequant_scalar_bytes(num_rows: int, num_valid: int) -> int:
    """Scalar-scale read side: as the blockwise one without the 7 exponent
    bytes per valid row, plus the one 4-byte scale."""
    return dequant_bytes(num_rows, num_valid) - 7 * num_valid + 4
