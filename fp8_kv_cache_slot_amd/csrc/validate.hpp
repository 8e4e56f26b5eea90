// Host-side argument checks of the two entry points.  Pure C++ (no HIP
// types or calls), so every error path is reachable without a GPU.
#pragma once

#include <cstdint>

#include "fp8kv.h"

namespace fp8kv {

constexpr int kHeadDim = 512;
constexpr int kRopeDim = 64;
constexpr int kPageSize = 64;
constexpr int kRowBytes = 576;   // 448 E4M3 codes + 64 bf16
constexpr int kScaleBytes = 8;   // 7 UE8M0 exponents + 1 reserved byte
constexpr int kPackedHeadDim = 128;

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// eps must be finite and non-negative (a NaN fails both comparisons).
inline bool valid_eps(float eps) {
  return eps >= 0.0f && eps <= 3.4028234663852886e38f;
}

inline int validate_prologue(const void* q, const void* kv,
                             const void* q_weight, const void* kv_weight,
                             const float* cos_sin_cache,
                             const int64_t* positions,
                             const int64_t* slot_mapping,
                             const uint8_t* kv_cache, const uint8_t* kv_scale,
                             int64_t num_tokens, int32_t num_heads,
                             int32_t head_dim, int32_t rope_dim,
                             int64_t max_position, int64_t num_pages,
                             int32_t page_size) {
  if (num_tokens < 0 || num_heads < 1 || max_position < 1 || num_pages < 0)
    return FP8KV_ERR_SHAPE;
  if (head_dim != kHeadDim || rope_dim != kRopeDim || page_size != kPageSize)
    return FP8KV_ERR_UNSUPPORTED;
  // Every slot index (token * (heads + 1)) and every token index fits in
  // 31 bits; byte offsets are formed in 64 bits.
  if (num_tokens > 0 &&
      num_tokens > (int64_t{1} << 31) / (static_cast<int64_t>(num_heads) + 1) - 1)
    return FP8KV_ERR_SHAPE;
  if (num_pages > (int64_t{1} << 40)) return FP8KV_ERR_SHAPE;
  if (num_tokens == 0) return FP8KV_OK;
  if (!q || !kv || !q_weight || !kv_weight || !cos_sin_cache || !positions ||
      !slot_mapping)
    return FP8KV_ERR_NULL;
  if (num_pages > 0 && (!kv_cache || !kv_scale)) return FP8KV_ERR_NULL;
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(q_weight, 16) ||
      !aligned(kv_weight, 16) || !aligned(cos_sin_cache, 16) ||
      !aligned(positions, 8) || !aligned(slot_mapping, 8) ||
      (kv_cache && !aligned(kv_cache, 16)))
    return FP8KV_ERR_ALIGN;
  return FP8KV_OK;
}

inline int validate_packed(const void* qkv, int64_t num_tokens,
                           int32_t num_heads_q, int32_t num_heads_k,
                           int32_t num_heads_v, int32_t head_dim,
                           const void* q_weight, const void* k_weight,
                           const float* cos_sin_cache, int32_t is_neox,
                           const int64_t* position_ids,
                           int32_t forced_token_heads_per_warp,
                           int64_t max_position) {
  if (num_tokens < 0 || num_heads_q < 0 || num_heads_k < 0 ||
      num_heads_v < 0 || int64_t{num_heads_q} + num_heads_k < 1 || max_position < 1)
    return FP8KV_ERR_SHAPE;
  if (head_dim != kPackedHeadDim || is_neox != 1 ||
      forced_token_heads_per_warp != -1)
    return FP8KV_ERR_UNSUPPORTED;
  const int64_t heads = static_cast<int64_t>(num_heads_q) + num_heads_k;
  if (num_tokens > 0 && (num_tokens > ((int64_t{1} << 31) - 1) / heads ||
                         static_cast<int64_t>(num_heads_q) + num_heads_k +
                                 num_heads_v > (1 << 20)))
    return FP8KV_ERR_SHAPE;
  if (num_tokens == 0) return FP8KV_OK;
  if (!qkv || !cos_sin_cache || !position_ids) return FP8KV_ERR_NULL;
  if ((num_heads_q > 0 && !q_weight) || (num_heads_k > 0 && !k_weight))
    return FP8KV_ERR_NULL;
  if (!aligned(qkv, 16) || !aligned(cos_sin_cache, 16) ||
      !aligned(position_ids, 8) || (q_weight && !aligned(q_weight, 16)) ||
      (k_weight && !aligned(k_weight, 16)))
    return FP8KV_ERR_ALIGN;
  return FP8KV_OK;
}

inline int validate_packed_ex(const void* qkv, int64_t num_tokens,
                              int32_t num_heads_q, int32_t num_heads_k,
                              int32_t num_heads_v, int32_t head_dim,
                              const void* q_weight, const void* k_weight,
                              const float* cos_sin_cache, int32_t is_neox,
                              const int64_t* position_ids, int32_t rotary_dim,
                              int32_t dtype, int64_t max_position) {
  if (num_tokens < 0 || num_heads_q < 0 || num_heads_k < 0 ||
      num_heads_v < 0 || int64_t{num_heads_q} + num_heads_k < 1 ||
      (rotary_dim > 0 && max_position < 1))  // R = 0 indexes no table
    return FP8KV_ERR_SHAPE;
  if ((head_dim != 64 && head_dim != 128 && head_dim != 256) ||
      rotary_dim < 0 || rotary_dim > head_dim || rotary_dim % 16 != 0 ||
      (is_neox != 0 && is_neox != 1) ||
      (dtype != FP8KV_DTYPE_BF16 && dtype != FP8KV_DTYPE_FP16))
    return FP8KV_ERR_UNSUPPORTED;
  const int64_t heads = static_cast<int64_t>(num_heads_q) + num_heads_k;
  if (num_tokens > 0 &&
      (num_tokens > ((int64_t{1} << 31) - 1) / heads ||
       (heads + num_heads_v) * head_dim > (int64_t{1} << 30)))
    return FP8KV_ERR_SHAPE;
  if (num_tokens == 0) return FP8KV_OK;
  if (!qkv || !position_ids || (rotary_dim > 0 && !cos_sin_cache))
    return FP8KV_ERR_NULL;
  if ((num_heads_q > 0 && !q_weight) || (num_heads_k > 0 && !k_weight))
    return FP8KV_ERR_NULL;
  if (!aligned(qkv, 16) || !aligned(position_ids, 8) ||
      (cos_sin_cache && !aligned(cos_sin_cache, 16)) ||
      (q_weight && !aligned(q_weight, 16)) || (k_weight && !aligned(k_weight, 16)))
    return FP8KV_ERR_ALIGN;
  return FP8KV_OK;
}

// scale_align: 8 for the exponent tensor, 4 for the scalar-scale float that
// takes its place.
inline int validate_gather_dequant(const uint8_t* kv_cache,
                                   const uint8_t* kv_scale, int64_t num_pages,
                                   int32_t page_size, const int64_t* slots,
                                   int64_t num_rows, const void* out,
                                   uintptr_t scale_align = 8) {
  if (num_pages < 0 || num_rows < 0 || num_rows > 0x7FFFFFFF ||
      num_pages > (int64_t{1} << 40))
    return FP8KV_ERR_SHAPE;
  if (page_size != kPageSize) return FP8KV_ERR_UNSUPPORTED;
  if (num_rows == 0) return FP8KV_OK;
  if (!slots || !out) return FP8KV_ERR_NULL;
  if (num_pages > 0 && (!kv_cache || !kv_scale)) return FP8KV_ERR_NULL;
  if (!aligned(slots, 8) || !aligned(out, 16) ||
      (kv_cache && !aligned(kv_cache, 16)) ||
      (kv_scale && !aligned(kv_scale, scale_align)))
    return FP8KV_ERR_ALIGN;
  return FP8KV_OK;
}

inline int validate_gather_dequant_paged(
    const uint8_t* kv_cache, const uint8_t* kv_scale, int64_t num_pages,
    int32_t page_size, const int32_t* block_table, int32_t num_seqs,
    int32_t max_blocks_per_seq, const int32_t* seq_lens,
    const int64_t* out_offsets, int64_t num_rows, const void* out,
    uintptr_t scale_align = 8) {
  if (num_pages < 0 || num_pages > (int64_t{1} << 40) || num_seqs < 0 ||
      num_seqs > 65535 || max_blocks_per_seq < 0 ||
      max_blocks_per_seq > (int32_t{1} << 24) || num_rows < 0 ||
      num_rows > (int64_t{1} << 40))
    return FP8KV_ERR_SHAPE;
  if (page_size != kPageSize) return FP8KV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_blocks_per_seq == 0 || num_rows == 0) return FP8KV_OK;
  if (!block_table || !seq_lens || !out_offsets || !out) return FP8KV_ERR_NULL;
  if (num_pages > 0 && (!kv_cache || !kv_scale)) return FP8KV_ERR_NULL;
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(out_offsets, 8) ||
      !aligned(out, 16) || (kv_cache && !aligned(kv_cache, 16)) ||
      (kv_scale && !aligned(kv_scale, scale_align)))
    return FP8KV_ERR_ALIGN;
  return FP8KV_OK;
}

inline int validate_rms_norm_rows(const void* x, const void* out,
                                  const void* weight, int64_t num_rows,
                                  int32_t row_dim) {
  if (num_rows < 0 || num_rows > (int64_t{1} << 40)) return FP8KV_ERR_SHAPE;
  if (row_dim != kHeadDim) return FP8KV_ERR_UNSUPPORTED;
  if (num_rows == 0) return FP8KV_OK;
  if (!x || !out || !weight) return FP8KV_ERR_NULL;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(weight, 16))
    return FP8KV_ERR_ALIGN;
  return FP8KV_OK;
}

inline int validate_rope_rows(const void* x, const float* cos_sin_cache,
                              const int64_t* positions, int64_t num_tokens,
                              int32_t rows_per_token, int32_t row_dim,
                              int32_t rope_dim, int64_t max_position) {
  if (num_tokens < 0 || rows_per_token < 1 || max_position < 1 ||
      num_tokens > (int64_t{1} << 40) / rows_per_token)
    return FP8KV_ERR_SHAPE;
  if (row_dim != kHeadDim || rope_dim != kRopeDim) return FP8KV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return FP8KV_OK;
  if (!x || !cos_sin_cache || !positions) return FP8KV_ERR_NULL;
  if (!aligned(x, 16) || !aligned(cos_sin_cache, 16) || !aligned(positions, 8))
    return FP8KV_ERR_ALIGN;
  return FP8KV_OK;
}

// The packed operator's separate stages: heads of 128, at most 2^31 - 1
// heads in all; a head starts on a 16-byte boundary.
inline int validate_heads(int64_t num_tokens, int32_t num_heads, int32_t head_dim) {
  if (num_tokens < 0 || num_heads < 0) return FP8KV_ERR_SHAPE;
  if (head_dim != 128) return FP8KV_ERR_UNSUPPORTED;
  if (num_heads > 0 && num_tokens > 0x7FFFFFFF / num_heads) return FP8KV_ERR_SHAPE;
  return FP8KV_OK;
}

inline int validate_rms_norm_heads(const void* x, int64_t x_token_stride,
                                   const void* out, const void* weight,
                                   int64_t num_tokens, int32_t num_heads,
                                   int32_t head_dim) {
  int st = validate_heads(num_tokens, num_heads, head_dim);
  if (st != FP8KV_OK) return st;
  if (num_tokens > 0 && num_heads > 0 &&
      (x_token_stride < int64_t{num_heads} * head_dim ||
       x_token_stride > (int64_t{1} << 40) / num_tokens))
    return FP8KV_ERR_SHAPE;
  if (num_tokens == 0 || num_heads == 0) return FP8KV_OK;
  if (!x || !out || !weight) return FP8KV_ERR_NULL;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(weight, 16) ||
      x_token_stride % 8 != 0)
    return FP8KV_ERR_ALIGN;
  return FP8KV_OK;
}

inline int validate_rope_neox_heads(const void* x, const float* cos_sin_cache,
                                    const int64_t* positions, int64_t num_tokens,
                                    int32_t num_heads, int32_t head_dim,
                                    int64_t max_position) {
  int st = validate_heads(num_tokens, num_heads, head_dim);
  if (st != FP8KV_OK) return st;
  if (max_position < 1) return FP8KV_ERR_SHAPE;
  if (num_tokens == 0 || num_heads == 0) return FP8KV_OK;
  if (!x || !cos_sin_cache || !positions) return FP8KV_ERR_NULL;
  if (!aligned(x, 16) || !aligned(cos_sin_cache, 16) || !aligned(positions, 8))
    return FP8KV_ERR_ALIGN;
  return FP8KV_OK;
}

inline int validate_kv_quant_insert(const void* kv, const int64_t* slot_mapping,
                                    const uint8_t* kv_cache,
                                    const uint8_t* kv_scale, int64_t num_tokens,
                                    int64_t num_pages, int32_t page_size) {
  if (num_tokens < 0 || num_tokens > 0x7FFFFFFF || num_pages < 0 ||
      num_pages > (int64_t{1} << 40))
    return FP8KV_ERR_SHAPE;
  if (page_size != kPageSize) return FP8KV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return FP8KV_OK;
  if (!kv || !slot_mapping) return FP8KV_ERR_NULL;
  if (num_pages > 0 && (!kv_cache || !kv_scale)) return FP8KV_ERR_NULL;
  if (!aligned(kv, 16) || !aligned(slot_mapping, 8) ||
      (kv_cache && !aligned(kv_cache, 16)))
    return FP8KV_ERR_ALIGN;
  return FP8KV_OK;
}

}  // namespace fp8kv
