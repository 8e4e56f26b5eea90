// C ABI of libfp8kv.so (declared in include/fp8kv.h): argument validation on
// the host, a cached gfx950 device check, the program-count dispatch between
// the small-batch and the tiled prologue kernels (on MI355X both default to
// one kernel: there is no crossover), and the launches.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cerrno>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "fp8kv.h"
#include "prologue_launch.hpp"
#include "validate.hpp"

#define FP8KV_API extern "C" __attribute__((visibility("default")))

namespace fp8kv {
namespace {

// Programs = num_tokens * (num_heads + 1) below which the small-batch kernel
// runs (the quantity FlagGems PR #5449 "Dispatch threshold" dispatches on).
// MI355X has no crossover: the small-batch shape (one head per one-wave
// block) is the fastest shape at every size measured, from 1 to 262144
// tokens at 16 to 128 heads (level with the others up to ~2k tokens, ahead
// from ~4k), so the default threshold is 0 and every call takes the tiled
// path, whose default shape is that same kernel.  The threshold and the
// tiled shape stay settable for measurement.
constexpr int64_t kDefaultThreshold = 0;
// Tiled shape: one wave per block, one Q head per wave (the small-batch
// shape).  Measured on MI355X, each launch after a cache-flushing read:
// 672 us at 32768x64, 1322 us at 32768x128 and 2686 us at 131072x64, against
// 688-690, 1379-1385 and 2792-2825 us for the best multi-head shapes (2x2,
// 4x2, 8x2) and 710-713 / 1388-1399 / 2843-2893 us for 2-8 waves of one
// head per block; from 32 to 2048 tokens at 64 and 128 heads the shapes are
// within +-0.3 us of each other in no consistent order.  A block of one wave
// is scheduled as soon as any wave slot of a CU frees up.
constexpr int kDefaultWaves = 1;
constexpr int kDefaultSlots = 1;

// The threshold in force when the library loads: FP8KV_DISPATCH_THRESHOLD
// if it holds a non-negative decimal integer, else the built-in default.
int64_t initial_threshold() {
  const char* e = std::getenv("FP8KV_DISPATCH_THRESHOLD");
  if (!e || !*e) return kDefaultThreshold;
  char* end = nullptr;
  errno = 0;
  const long long v = std::strtoll(e, &end, 10);
  if (errno != 0 || *end != '\0' || v < 0) return kDefaultThreshold;
  return static_cast<int64_t>(v);
}

std::atomic<int64_t> g_threshold{initial_threshold()};
std::atomic<int32_t> g_tiling{(kDefaultWaves << 16) | kDefaultSlots};

constexpr int kMaxDevices = 64;
std::atomic<int8_t> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return FP8KV_ERR_DEVICE;
  int8_t state = g_device_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8KV_ERR_DEVICE;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? FP8KV_OK : FP8KV_ERR_DEVICE;
}

}  // namespace
}  // namespace fp8kv

namespace fp8kv {
namespace {

int prologue(void* q, const void* kv, const void* q_weight, const void* kv_weight,
             const float* cos_sin_cache, const int64_t* positions,
             const int64_t* slot_mapping, uint8_t* kv_cache, uint8_t* kv_scale,
             bool scalar, const float* scalar_scale, int64_t num_tokens,
             int32_t num_heads,
             int32_t head_dim, int32_t rope_dim, int64_t max_position,
             int64_t num_pages, int32_t page_size, float eps, void* stream) {
  // For the scalar-scale convention the scale pointer takes the exponent
  // tensor's place in the NULL check (required when the cache has pages).
  if (!valid_eps(eps)) return FP8KV_ERR_VALUE;
  const uint8_t* scale_ptr =
      scalar ? reinterpret_cast<const uint8_t*>(scalar_scale) : kv_scale;
  int st = validate_prologue(q, kv, q_weight, kv_weight, cos_sin_cache,
                             positions, slot_mapping, kv_cache, scale_ptr,
                             num_tokens, num_heads, head_dim, rope_dim,
                             max_position, num_pages, page_size);
  if (st != FP8KV_OK || num_tokens == 0) return st;
  if (scalar && scalar_scale && !aligned(scalar_scale, 4)) return FP8KV_ERR_ALIGN;
  st = check_device();
  if (st != FP8KV_OK) return st;

  PrologueArgs a;
  a.q = static_cast<uint16_t*>(q);
  a.kv = static_cast<const uint16_t*>(kv);
  a.q_weight = static_cast<const uint16_t*>(q_weight);
  a.kv_weight = static_cast<const uint16_t*>(kv_weight);
  a.cos_sin = cos_sin_cache;
  a.positions = positions;
  a.slot_mapping = slot_mapping;
  a.kv_cache = kv_cache;
  a.kv_scale = scalar ? nullptr : kv_scale;
  a.scalar_scale = scalar ? scalar_scale : nullptr;
  a.scalar = scalar;
  a.num_tokens = static_cast<int32_t>(num_tokens);
  a.num_heads = num_heads;
  a.num_cache_slots = num_pages * kPageSize;
  a.max_position = max_position;
  a.eps = eps;

  const int64_t programs = num_tokens * (static_cast<int64_t>(num_heads) + 1);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (programs < g_threshold.load(std::memory_order_relaxed))
    return launch_prologue(a, 1, 1, s);
  const int32_t tiling = g_tiling.load(std::memory_order_relaxed);
  return launch_prologue(a, tiling >> 16, tiling & 0xFFFF, s);
}

}  // namespace
}  // namespace fp8kv

FP8KV_API int qnorm_rope_kv_quant_insert(
    void* q, const void* kv, const void* q_weight, const void* kv_weight,
    const float* cos_sin_cache, const int64_t* positions,
    const int64_t* slot_mapping, uint8_t* kv_cache, uint8_t* kv_scale,
    int64_t num_tokens, int32_t num_heads, int32_t head_dim, int32_t rope_dim,
    int64_t max_position, int64_t num_pages, int32_t page_size, float eps,
    void* stream) {
  return fp8kv::prologue(q, kv, q_weight, kv_weight, cos_sin_cache, positions,
                         slot_mapping, kv_cache, kv_scale, false, nullptr,
                         num_tokens,
                         num_heads, head_dim, rope_dim, max_position, num_pages,
                         page_size, eps, stream);
}

FP8KV_API int qnorm_rope_kv_quant_insert_scalar_scale(
    void* q, const void* kv, const void* q_weight, const void* kv_weight,
    const float* cos_sin_cache, const int64_t* positions,
    const int64_t* slot_mapping, uint8_t* kv_cache, const float* kv_cache_scale,
    int64_t num_tokens, int32_t num_heads, int32_t head_dim, int32_t rope_dim,
    int64_t max_position, int64_t num_pages, int32_t page_size, float eps,
    void* stream) {
  return fp8kv::prologue(q, kv, q_weight, kv_weight, cos_sin_cache, positions,
                         slot_mapping, kv_cache, nullptr, true, kv_cache_scale,
                         num_tokens,
                         num_heads, head_dim, rope_dim, max_position, num_pages,
                         page_size, eps, stream);
}

FP8KV_API int qk_norm_rope_packed(
    void* qkv, int64_t num_tokens, int32_t num_heads_q, int32_t num_heads_k,
    int32_t num_heads_v, int32_t head_dim, float eps, const void* q_weight,
    const void* k_weight, const float* cos_sin_cache, int32_t is_neox,
    const int64_t* position_ids, int32_t forced_token_heads_per_warp,
    int64_t max_position, void* stream) {
  using namespace fp8kv;
  if (!valid_eps(eps)) return FP8KV_ERR_VALUE;
  int st = validate_packed(qkv, num_tokens, num_heads_q, num_heads_k,
                           num_heads_v, head_dim, q_weight, k_weight,
                           cos_sin_cache, is_neox, position_ids,
                           forced_token_heads_per_warp, max_position);
  if (st != FP8KV_OK || num_tokens == 0) return st;
  st = check_device();
  if (st != FP8KV_OK) return st;
  PackedArgs a;
  a.qkv = static_cast<uint16_t*>(qkv);
  a.q_weight = static_cast<const uint16_t*>(q_weight);
  a.k_weight = static_cast<const uint16_t*>(k_weight);
  a.cos_sin = cos_sin_cache;
  a.position_ids = position_ids;
  a.num_tokens = static_cast<int32_t>(num_tokens);
  a.num_heads_q = num_heads_q;
  a.num_heads_k = num_heads_k;
  a.row_elems = (num_heads_q + num_heads_k + num_heads_v) * kPackedHeadDim;
  a.max_position = max_position;
  a.eps = eps;
  return launch_packed(a, static_cast<hipStream_t>(stream));
}

FP8KV_API int qk_norm_rope_packed_ex(
    void* qkv, int64_t num_tokens, int32_t num_heads_q, int32_t num_heads_k,
    int32_t num_heads_v, int32_t head_dim, float eps, const void* q_weight,
    const void* k_weight, const float* cos_sin_cache, int32_t is_neox,
    const int64_t* position_ids, int32_t rotary_dim, int32_t dtype,
    int64_t max_position, void* stream) {
  using namespace fp8kv;
  if (!valid_eps(eps)) return FP8KV_ERR_VALUE;
  int st = validate_packed_ex(qkv, num_tokens, num_heads_q, num_heads_k,
                              num_heads_v, head_dim, q_weight, k_weight,
                              cos_sin_cache, is_neox, position_ids, rotary_dim,
                              dtype, max_position);
  if (st != FP8KV_OK || num_tokens == 0) return st;
  st = check_device();
  if (st != FP8KV_OK) return st;
  // The guarded case (bf16, 128 wide, full NeoX) has its own tuned kernel.
  if (dtype == FP8KV_DTYPE_BF16 && head_dim == kPackedHeadDim &&
      rotary_dim == kPackedHeadDim && is_neox == 1) {
    PackedArgs a;
    a.qkv = static_cast<uint16_t*>(qkv);
    a.q_weight = static_cast<const uint16_t*>(q_weight);
    a.k_weight = static_cast<const uint16_t*>(k_weight);
    a.cos_sin = cos_sin_cache;
    a.position_ids = position_ids;
    a.num_tokens = static_cast<int32_t>(num_tokens);
    a.num_heads_q = num_heads_q;
    a.num_heads_k = num_heads_k;
    a.row_elems = (num_heads_q + num_heads_k + num_heads_v) * kPackedHeadDim;
    a.max_position = max_position;
    a.eps = eps;
    return launch_packed(a, static_cast<hipStream_t>(stream));
  }
  PackedExArgs a;
  a.qkv = static_cast<uint16_t*>(qkv);
  a.q_weight = static_cast<const uint16_t*>(q_weight);
  a.k_weight = static_cast<const uint16_t*>(k_weight);
  a.cos_sin = cos_sin_cache;
  a.position_ids = position_ids;
  a.num_tokens = static_cast<int32_t>(num_tokens);
  a.num_heads_q = num_heads_q;
  a.num_heads_k = num_heads_k;
  a.row_elems = (num_heads_q + num_heads_k + num_heads_v) * head_dim;
  a.head_dim = head_dim;
  a.rotary_dim = rotary_dim;
  a.is_neox = is_neox;
  a.is_fp16 = dtype == FP8KV_DTYPE_FP16;
  a.max_position = max_position;
  a.eps = eps;
  return launch_packed_ex(a, static_cast<hipStream_t>(stream));
}

FP8KV_API int kv_cache_gather_dequant(const uint8_t* kv_cache,
                                     const uint8_t* kv_scale, int64_t num_pages,
                                     int32_t page_size, const int64_t* slots,
                                     int64_t num_rows, void* out, void* stream) {
  using namespace fp8kv;
  int st = validate_gather_dequant(kv_cache, kv_scale, num_pages, page_size,
                                   slots, num_rows, out);
  if (st != FP8KV_OK || num_rows == 0) return st;
  st = check_device();
  if (st != FP8KV_OK) return st;
  DequantArgs a;
  a.kv_cache = kv_cache;
  a.kv_scale = kv_scale;
  a.scalar_scale = nullptr;
  a.scalar = false;
  a.slots = slots;
  a.out = static_cast<uint16_t*>(out);
  a.num_rows = static_cast<int32_t>(num_rows);
  a.num_cache_slots = num_pages * kPageSize;
  return launch_gather_dequant(a, static_cast<hipStream_t>(stream));
}

FP8KV_API int kv_cache_gather_dequant_paged(
    const uint8_t* kv_cache, const uint8_t* kv_scale, int64_t num_pages,
    int32_t page_size, const int32_t* block_table, int32_t num_seqs,
    int32_t max_blocks_per_seq, const int32_t* seq_lens,
    const int64_t* out_offsets, int64_t num_rows, void* out, void* stream) {
  using namespace fp8kv;
  int st = validate_gather_dequant_paged(kv_cache, kv_scale, num_pages, page_size,
                                         block_table, num_seqs, max_blocks_per_seq,
                                         seq_lens, out_offsets, num_rows, out);
  if (st != FP8KV_OK || num_seqs == 0 || max_blocks_per_seq == 0 || num_rows == 0)
    return st;
  st = check_device();
  if (st != FP8KV_OK) return st;
  PagedDequantArgs a;
  a.kv_cache = kv_cache;
  a.kv_scale = kv_scale;
  a.scalar_scale = nullptr;
  a.scalar = false;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out_offsets = out_offsets;
  a.out = static_cast<uint16_t*>(out);
  a.num_seqs = num_seqs;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_pages = num_pages;
  a.num_rows = num_rows;
  return launch_gather_dequant_paged(a, static_cast<hipStream_t>(stream));
}

FP8KV_API int kv_cache_gather_dequant_paged_scalar_scale(
    const uint8_t* kv_cache, const float* kv_cache_scale, int64_t num_pages,
    int32_t page_size, const int32_t* block_table, int32_t num_seqs,
    int32_t max_blocks_per_seq, const int32_t* seq_lens,
    const int64_t* out_offsets, int64_t num_rows, void* out, void* stream) {
  using namespace fp8kv;
  // the scale pointer takes the exponent tensor's place in the NULL check
  int st = validate_gather_dequant_paged(
      kv_cache, reinterpret_cast<const uint8_t*>(kv_cache_scale), num_pages,
      page_size, block_table, num_seqs, max_blocks_per_seq, seq_lens,
      out_offsets, num_rows, out, 4);
  if (st != FP8KV_OK || num_seqs == 0 || max_blocks_per_seq == 0 || num_rows == 0)
    return st;
  st = check_device();
  if (st != FP8KV_OK) return st;
  PagedDequantArgs a;
  a.kv_cache = kv_cache;
  a.kv_scale = nullptr;
  a.scalar_scale = kv_cache_scale;  // read only when num_pages > 0
  a.scalar = true;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out_offsets = out_offsets;
  a.out = static_cast<uint16_t*>(out);
  a.num_seqs = num_seqs;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_pages = num_pages;
  a.num_rows = num_rows;
  return launch_gather_dequant_paged(a, static_cast<hipStream_t>(stream));
}

FP8KV_API int rms_norm_rows(const void* x, void* out, const void* weight,
                            int64_t num_rows, int32_t row_dim, float eps,
                            void* stream) {
  using namespace fp8kv;
  if (!valid_eps(eps)) return FP8KV_ERR_VALUE;
  int st = validate_rms_norm_rows(x, out, weight, num_rows, row_dim);
  if (st != FP8KV_OK || num_rows == 0) return st;
  st = check_device();
  if (st != FP8KV_OK) return st;
  return launch_rms_norm_rows(static_cast<const uint16_t*>(x),
                              static_cast<uint16_t*>(out),
                              static_cast<const uint16_t*>(weight), num_rows, eps,
                              static_cast<hipStream_t>(stream));
}

FP8KV_API int rope_rows(void* x, const float* cos_sin_cache,
                        const int64_t* positions, int64_t num_tokens,
                        int32_t rows_per_token, int32_t row_dim, int32_t rope_dim,
                        int64_t max_position, void* stream) {
  using namespace fp8kv;
  int st = validate_rope_rows(x, cos_sin_cache, positions, num_tokens,
                              rows_per_token, row_dim, rope_dim, max_position);
  if (st != FP8KV_OK || num_tokens == 0) return st;
  st = check_device();
  if (st != FP8KV_OK) return st;
  return launch_rope_rows(static_cast<uint16_t*>(x), cos_sin_cache, positions,
                          num_tokens, rows_per_token, max_position,
                          static_cast<hipStream_t>(stream));
}

FP8KV_API int rms_norm_heads(const void* x, int64_t x_token_stride, void* out,
                             const void* weight, int64_t num_tokens,
                             int32_t num_heads, int32_t head_dim, float eps,
                             void* stream) {
  using namespace fp8kv;
  if (!valid_eps(eps)) return FP8KV_ERR_VALUE;
  int st = validate_rms_norm_heads(x, x_token_stride, out, weight, num_tokens,
                                   num_heads, head_dim);
  if (st != FP8KV_OK || num_tokens == 0 || num_heads == 0) return st;
  st = check_device();
  if (st != FP8KV_OK) return st;
  return launch_rms_norm_heads(static_cast<const uint16_t*>(x), x_token_stride,
                               static_cast<uint16_t*>(out),
                               static_cast<const uint16_t*>(weight),
                               static_cast<int32_t>(num_tokens), num_heads, eps,
                               static_cast<hipStream_t>(stream));
}

FP8KV_API int rope_neox_heads(void* x, const float* cos_sin_cache,
                              const int64_t* positions, int64_t num_tokens,
                              int32_t num_heads, int32_t head_dim,
                              int64_t max_position, void* stream) {
  using namespace fp8kv;
  int st = validate_rope_neox_heads(x, cos_sin_cache, positions, num_tokens,
                                    num_heads, head_dim, max_position);
  if (st != FP8KV_OK || num_tokens == 0 || num_heads == 0) return st;
  st = check_device();
  if (st != FP8KV_OK) return st;
  return launch_rope_neox_heads(static_cast<uint16_t*>(x), cos_sin_cache, positions,
                                static_cast<int32_t>(num_tokens), num_heads,
                                max_position, static_cast<hipStream_t>(stream));
}

FP8KV_API int kv_quant_insert(const void* kv, const int64_t* slot_mapping,
                              uint8_t* kv_cache, uint8_t* kv_scale,
                              int64_t num_tokens, int64_t num_pages,
                              int32_t page_size, void* stream) {
  using namespace fp8kv;
  int st = validate_kv_quant_insert(kv, slot_mapping, kv_cache, kv_scale,
                                    num_tokens, num_pages, page_size);
  if (st != FP8KV_OK || num_tokens == 0) return st;
  st = check_device();
  if (st != FP8KV_OK) return st;
  return launch_kv_quant_insert(static_cast<const uint16_t*>(kv), slot_mapping,
                                kv_cache, kv_scale,
                                static_cast<int32_t>(num_tokens),
                                num_pages * kPageSize,
                                static_cast<hipStream_t>(stream));
}

FP8KV_API int kv_cache_gather_dequant_scalar_scale(
    const uint8_t* kv_cache, const float* kv_cache_scale, int64_t num_pages,
    int32_t page_size, const int64_t* slots, int64_t num_rows, void* out,
    void* stream) {
  using namespace fp8kv;
  int st = validate_gather_dequant(
      kv_cache, reinterpret_cast<const uint8_t*>(kv_cache_scale), num_pages,
      page_size, slots, num_rows, out, 4);
  if (st != FP8KV_OK || num_rows == 0) return st;
  st = check_device();
  if (st != FP8KV_OK) return st;
  DequantArgs a;
  a.kv_cache = kv_cache;
  a.kv_scale = nullptr;
  a.scalar_scale = kv_cache_scale;  // read only for valid slots (num_pages > 0)
  a.scalar = true;
  a.slots = slots;
  a.out = static_cast<uint16_t*>(out);
  a.num_rows = static_cast<int32_t>(num_rows);
  a.num_cache_slots = num_pages * kPageSize;
  return launch_gather_dequant(a, static_cast<hipStream_t>(stream));
}

FP8KV_API const char* fp8kv_status_string(int status) {
  switch (status) {
    case FP8KV_OK: return "ok";
    case FP8KV_ERR_NULL: return "a required pointer is NULL";
    case FP8KV_ERR_SHAPE: return "invalid or too large size argument";
    case FP8KV_ERR_UNSUPPORTED: return "unsupported layout parameter";
    case FP8KV_ERR_ALIGN: return "pointer not aligned as required";
    case FP8KV_ERR_DEVICE: return "no current HIP device or device is not gfx950";
    case FP8KV_ERR_LAUNCH: return "kernel launch failed";
    case FP8KV_ERR_VALUE: return "eps is negative, infinite or NaN";
    default: return "unknown status";
  }
}

FP8KV_API int fp8kv_abi_version(void) { return FP8KV_ABI_VERSION; }

FP8KV_API int fp8kv_set_dispatch_threshold(int64_t programs) {
  fp8kv::g_threshold.store(programs < 0 ? fp8kv::kDefaultThreshold : programs,
                           std::memory_order_relaxed);
  return FP8KV_OK;
}

FP8KV_API int64_t fp8kv_get_dispatch_threshold(void) {
  return fp8kv::g_threshold.load(std::memory_order_relaxed);
}

FP8KV_API int fp8kv_set_tiling(int32_t waves_per_block, int32_t slots_per_wave) {
  if (waves_per_block == 0 && slots_per_wave == 0) {
    waves_per_block = fp8kv::kDefaultWaves;
    slots_per_wave = fp8kv::kDefaultSlots;
  }
  if (!fp8kv::prologue_shape_built(waves_per_block, slots_per_wave))
    return FP8KV_ERR_UNSUPPORTED;
  fp8kv::g_tiling.store((waves_per_block << 16) | slots_per_wave,
                        std::memory_order_relaxed);
  return FP8KV_OK;
}

FP8KV_API void fp8kv_get_tiling(int32_t* waves_per_block, int32_t* slots_per_wave) {
  const int32_t t = fp8kv::g_tiling.load(std::memory_order_relaxed);
  if (waves_per_block) *waves_per_block = t >> 16;
  if (slots_per_wave) *slots_per_wave = t & 0xFFFF;
}

FP8KV_API int fp8kv_stream_copy(void* dst, const void* src, int64_t bytes,
                                void* stream) {
  using namespace fp8kv;
  if (bytes < 0 || bytes % 16 != 0) return FP8KV_ERR_SHAPE;
  if (bytes == 0) return FP8KV_OK;
  if (!dst || !src) return FP8KV_ERR_NULL;
  if (!aligned(dst, 16) || !aligned(src, 16)) return FP8KV_ERR_ALIGN;
  int st = check_device();
  if (st != FP8KV_OK) return st;
  return launch_stream_copy(dst, src, bytes / 16, static_cast<hipStream_t>(stream));
}

FP8KV_API int fp8kv_stream_rmw(void* buf, int64_t bytes, uint32_t mask,
                               void* stream) {
  using namespace fp8kv;
  if (bytes < 0 || bytes % 16 != 0) return FP8KV_ERR_SHAPE;
  if (bytes == 0) return FP8KV_OK;
  if (!buf) return FP8KV_ERR_NULL;
  if (!aligned(buf, 16)) return FP8KV_ERR_ALIGN;
  int st = check_device();
  if (st != FP8KV_OK) return st;
  return launch_stream_rmw(buf, bytes / 16, mask, static_cast<hipStream_t>(stream));
}
