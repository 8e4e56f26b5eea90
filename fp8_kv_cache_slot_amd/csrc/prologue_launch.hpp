// Internal launch interface between the C ABI (capi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fp8kv.h"

namespace fp8kv {

struct PrologueArgs {
  uint16_t* q;
  const uint16_t* kv;
  const uint16_t* q_weight;
  const uint16_t* kv_weight;
  const float* cos_sin;
  const int64_t* positions;
  const int64_t* slot_mapping;
  uint8_t* kv_cache;
  uint8_t* kv_scale;           // blockwise exponents (unused when scalar)
  const float* scalar_scale;   // one device float: the scalar-scale convention
  bool scalar;                 // use scalar_scale instead of kv_scale
  int32_t num_tokens;
  int32_t num_heads;
  int64_t num_cache_slots;  // num_pages * 64
  int64_t max_position;
  float eps;
};

struct PackedArgs {
  uint16_t* qkv;
  const uint16_t* q_weight;
  const uint16_t* k_weight;
  const float* cos_sin;
  const int64_t* position_ids;
  int32_t num_tokens;
  int32_t num_heads_q;
  int32_t num_heads_k;
  int32_t row_elems;  // (Hq + Hk + Hv) * 128
  int64_t max_position;
  float eps;
};

struct PackedExArgs {
  uint16_t* qkv;
  const uint16_t* q_weight;
  const uint16_t* k_weight;
  const float* cos_sin;
  const int64_t* position_ids;
  int32_t num_tokens;
  int32_t num_heads_q;
  int32_t num_heads_k;
  int32_t row_elems;  // (Hq + Hk + Hv) * head_dim
  int32_t head_dim;   // 64, 128 or 256
  int32_t rotary_dim; // multiple of 16, <= head_dim
  int32_t is_neox;
  int32_t is_fp16;
  int64_t max_position;
  float eps;
};

struct DequantArgs {
  const uint8_t* kv_cache;
  const uint8_t* kv_scale;       // blockwise exponents (unused when scalar)
  const float* scalar_scale;     // one device float: the scalar-scale convention
  bool scalar;                   // use scalar_scale instead of kv_scale
  const int64_t* slots;
  uint16_t* out;
  int32_t num_rows;
  int64_t num_cache_slots;  // num_pages * 64
};

// Launch the fused prologue with `waves` 64-lane waves per block and `qs`
// Q heads per wave.  Returns FP8KV_ERR_UNSUPPORTED for a shape not built.
int launch_prologue(const PrologueArgs& a, int waves, int qs, hipStream_t stream);
bool prologue_shape_built(int waves, int qs);

int launch_packed(const PackedArgs& a, hipStream_t stream);
int launch_gather_dequant(const DequantArgs& a, hipStream_t stream);

struct PagedDequantArgs {
  const uint8_t* kv_cache;
  const uint8_t* kv_scale;       // blockwise exponents (unused when scalar)
  const float* scalar_scale;     // one device float: the scalar-scale convention
  bool scalar;                   // use scalar_scale instead of kv_scale
  const int32_t* block_table;   // [num_seqs, max_blocks_per_seq]
  const int32_t* seq_lens;      // [num_seqs]
  const int64_t* out_offsets;   // [num_seqs]: first output row of each sequence
  uint16_t* out;                // [num_rows, 512]
  int32_t num_seqs;
  int32_t max_blocks_per_seq;
  int64_t num_pages;
  int64_t num_rows;
};
int launch_gather_dequant_paged(const PagedDequantArgs& a, hipStream_t stream);
int launch_packed_ex(const PackedExArgs& a, hipStream_t stream);

// The prologue's stages as separate launches (the unfused baseline).
int launch_rms_norm_rows(const uint16_t* x, uint16_t* out, const uint16_t* weight,
                         int64_t num_rows, float eps, hipStream_t stream);
int launch_rope_rows(uint16_t* x, const float* cos_sin, const int64_t* positions,
                     int64_t num_tokens, int32_t rows_per_token,
                     int64_t max_position, hipStream_t stream);
int launch_kv_quant_insert(const uint16_t* kv, const int64_t* slot_mapping,
                           uint8_t* kv_cache, uint8_t* kv_scale, int32_t num_tokens,
                           int64_t num_cache_slots, hipStream_t stream);

// Reference streaming kernels (16-byte vectors; n16 = number of vectors).
int launch_rms_norm_heads(const uint16_t* x, int64_t x_token_stride, uint16_t* out,
                          const uint16_t* weight, int32_t num_tokens,
                          int32_t num_heads, float eps, hipStream_t stream);
int launch_rope_neox_heads(uint16_t* x, const float* cos_sin,
                           const int64_t* positions, int32_t num_tokens,
                           int32_t num_heads, int64_t max_position,
                           hipStream_t stream);
int launch_stream_copy(void* dst, const void* src, int64_t n16, hipStream_t stream);
int launch_stream_rmw(void* buf, int64_t n16, uint32_t mask, hipStream_t stream);

}  // namespace fp8kv
