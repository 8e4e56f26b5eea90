"""A KV row whose quantiser decisions differ between double and fp32.

The FP8 quantiser's two integer decisions, the UE8M0 block exponent and the
E4M3 code, are taken on fp32 values, the precision the operator computes in.
This case sits where that matters.  The expected bytes below are derived by
hand, not by running anything.

Inputs, one token, one Q head, position 0 (cos 1, sin 0: no rotation):
  kv[d] = 1.0 for d < 448 and 0.5 for the 64 rotary dims;
  kv_weight[d] = 1.75 in block 0 (dims 0..63), 1.8125 in block 1 (64..127)
  and 1.0 elsewhere (all exact in bf16);
  eps = 3/32 - 2^-27 (exact in fp32: the fp32 neighbour below 3/32).

Mean square: (448 * 1 + 64 * 0.25) / 512 = 464 / 512 = 0.90625 = 29/32, so
mean square + eps = 1 - 2^-27 and r = 1/sqrt(1 - 2^-27) = 1 + 2^-28 + O(2^-55).
The normalised values are y = w r (rotary dims 0.5 r).  fp32 keeps 24 bits, so
w r = w (1 + 2^-28) rounds to w itself (the error 1.8125 * 2^-28 is far below
half an fp32 step, 2^-24, at [1, 2)):
  block 0: fp32(y) = 1.75 = 448 * 2^-8, so e = -8 (byte 119) and every code is
           E4M3(1.75 * 2^8 = 448) = 0x7E.  Decided in double, y > 1.75 would
           need e = -7 (byte 120) and code E4M3(224 (1 + 2^-28)) = 0x76.
  block 1: fp32(y) = 1.8125, e = -7 (1.75 < 1.8125 <= 3.5: byte 120), and
           1.8125 * 2^7 = 232 lies exactly halfway between the E4M3 values 224
           (mantissa 6) and 240 (mantissa 7): ties to even give 224 = 0x76.
           Decided in double, 232 (1 + 2^-28) rounds up to 240 = 0x77.
  blocks 2..6: fp32(y) = 1.0, e = -8 (0.875 < 1 <= 1.75: byte 119), code
           E4M3(256) = 0x78.
  rotary dims: bf16(0.5 (1 + 2^-28)) = 0.5 = 0x3F00.
Scalar-scale convention with kv_cache_scale = 1: the code of block 1 is
E4M3(fp32(1.8125)) = E4M3(1.8125), again halfway, between 1.75 (0x3E) and
1.875 (0x3F): 0x3E (double would give 0x3F); block 0 gives E4M3(1.75) = 0x3E,
the other blocks E4M3(1.0) = 0x38.
"""

import numpy as np

EPS = 3.0 / 32.0 - 2.0 ** -27

# hand-derived stored bytes (see above)
SCALE_BYTES = [119, 120, 119, 119, 119, 119, 119]
CODES = [0x7E] * 64 + [0x76] * 64 + [0x78] * 320
ROPE_BF16 = 0x3F00
SCALAR_CODES = [0x3E] * 64 + [0x3E] * 64 + [0x38] * 320

# the bytes a decision in double would have given (for the record)
DOUBLE_SCALE_BYTES = [120, 120, 119, 119, 119, 119, 119]


def bf16_bits(v):
    """bf16 pattern of a value that bf16 holds exactly (checked)."""
    b = int(np.array([v], np.float32).view(np.uint32)[0])
    assert b & 0xFFFF == 0, v
    return b >> 16


def inputs(pages=1, slot=5):
    kv = np.full((1, 512), bf16_bits(1.0), np.uint16)
    kv[0, 448:] = bf16_bits(0.5)
    kv_w = np.full(512, bf16_bits(1.0), np.uint16)
    kv_w[0:64] = bf16_bits(1.75)
    kv_w[64:128] = bf16_bits(1.8125)
    cs = np.zeros((1, 64), np.float32)
    cs[0, :32] = 1.0
    return dict(
        q=np.array(kv.reshape(1, 1, 512)),
        kv=kv,
        q_weight=np.full(512, bf16_bits(1.0), np.uint16),
        kv_weight=kv_w,
        cos_sin_cache=cs,
        positions=np.zeros(1, np.int64),
        slot_mapping=np.array([slot], np.int64),
        kv_cache=np.full((pages, 64, 576), 0xA5, np.uint8),
        kv_scale=np.full((pages, 64, 8), 0x5A, np.uint8),
        eps=EPS,
    )
