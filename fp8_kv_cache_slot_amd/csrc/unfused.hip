// The DeepSeek-V4 prologue taken apart into separate launches, the unfused
// baseline the fused kernel is measured against (FlagGems PR #5449
// "Performance": one fused launch against the baseline's two; InfiniOps PR
// #1019 "Benchmark / Performance Impact": separate RmsNorm and
// RotaryEmbedding calls).  Each stage reads and writes bf16 in HBM:
//
//   rms_norm_rows    out[r, :] = bf16(x[r, :] / rms(x[r, :]) * w), rows of 512
//   rope_rows        in place, interleaved pairs on dims 448..511 of every
//                    row of token t, rotated by cos_sin_cache[positions[t]]
//   kv_quant_insert  already normalised and rotated bf16 KV rows -> FP8 E4M3
//                    codes + 7 UE8M0 exponents + bf16 rotary dims, scattered
//                    through slot_mapping (the fused kernel's own quantiser)
//
// The layouts follow the fused kernel: a 512-wide row is one 16-byte vector
// per lane of a wave; the 64 rotary dims of a row are 8 lanes x 16 bytes, so
// the RoPE stage covers 8 rows per wave and touches only those 128 bytes.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kv_quant.hpp"
#include "occupancy.hpp"
#include "prologue_launch.hpp"
#include "wave_ops.hpp"

namespace fp8kv {
namespace {

// One wave per block, two rows per wave for the RMSNorm stage: the five-launch
// pipeline took 800 us at 32768 x 64 with this shape on MI355X (caches cold),
// against 816 us with four waves of two rows, 824 us with one row per
// one-wave block and 834 us with two waves of one row; within 1 us of each
// other at 1024 x 64 (38.3-39.5 us).  Issuing the RoPE stage's row load
// before its position wait and the quantiser's row load with its slot load
// (below) then took the pipeline from 802.6 to 797.4 us (38.9 to 38.1 us at
// 1024 x 64).  The baseline is tuned like the fused kernel it is compared
// with.
constexpr int kWaves = 1;
constexpr int kRowsPerWave = 2;

// The RMSNorm stage caps its large launches at 16 blocks per CU (the same
// LDS request as the packed kernels; uncapped, 32 blocks fit).  Measured on
// MI355X with cold caches: the in-place norm of the prefill q (2097152 rows,
// 1048576 one-wave blocks) 646.2 against 671.8 us, and the five-launch
// pipeline 770.0 against 795.3 us; at 1024 x 64 (32768 blocks) the cap was
// 3% slower (25.50 against 24.80 us).  The RoPE stage was slower with every
// cap tried (111-242 against 98.1 us at prefill).
constexpr int kNormCapBlocksPerCu = 16;
constexpr int64_t kNormCapMinBlocks = 131072;

template <int RS>
__global__ void __launch_bounds__(kWaves * 64) rms_norm_rows_kernel(
    const uint16_t* x, uint16_t* out, const uint16_t* __restrict__ weight,
    int64_t num_rows, float eps) {
  // x and out may be the same buffer: each lane reads and then writes only
  // its own 16 bytes.
  const int lane = lane_id();
  const int64_t first =
      (static_cast<int64_t>(blockIdx.x) * kWaves + wave_id()) * RS;
  if (first >= num_rows) return;
  u32x4_t v[RS];
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    const int64_t row = first + r < num_rows ? first + r : first;
    v[r] = load16<true>(x + row * 512 + lane * 8);
  }
  float w[8];
  unpack8(load16<false>(weight + lane * 8), w);
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    if (first + r >= num_rows) break;
    float f[8];
    unpack8(v[r], f);
    const float ss = wave64_sum(sum_sq8(f));
    const float rr = __builtin_amdgcn_rsqf(fmaf(ss, 1.0f / 512.0f, eps));
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = f[j] * rr * w[j];
    u32x4_t o = {pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]),
                 pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7])};
    store16<true>(out + (first + r) * 512 + lane * 8, o);
  }
}

__global__ void __launch_bounds__(kWaves * 64) rope_rows_kernel(
    uint16_t* __restrict__ x, const float* __restrict__ cos_sin,
    const int64_t* __restrict__ positions, int64_t num_rows,
    int32_t rows_per_token, int64_t max_position) {
  // 8 lanes per row: lane j of the group holds pairs 4j..4j+3 (dims
  // 448 + 8j .. 455 + 8j).
  const int lane = lane_id();
  const int64_t row =
      (static_cast<int64_t>(blockIdx.x) * kWaves + wave_id()) * 8 + (lane >> 3);
  if (row >= num_rows) return;
  const int j = lane & 7;
  uint16_t* p = x + row * 512 + 448 + j * 8;
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
  const int64_t t = row / rows_per_token;
  // An out-of-range position turns off the store (row 0's angles are read
  // instead), so no branch on the loaded position sits behind the row load.
  const int64_t pos_in = positions[t];
  // keep the row load in front of the wait for the position
  __builtin_amdgcn_sched_barrier(0);
  const bool ok = pos_in >= 0 && pos_in < max_position;
  const int64_t pos = ok ? pos_in : 0;
  const f32x4_t c = load16f(cos_sin + pos * 64 + j * 4);
  const f32x4_t s = load16f(cos_sin + pos * 64 + 32 + j * 4);
  float y[8];
  unpack8(v, y);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = y[2 * k], b = y[2 * k + 1];
    y[2 * k] = a * c[k] - b * s[k];
    y[2 * k + 1] = b * c[k] + a * s[k];
  }
  if (ok)
    *reinterpret_cast<u32x4_t*>(p) =
        u32x4_t{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]),
                pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7])};
}

__global__ void __launch_bounds__(kWaves * 64) kv_quant_insert_kernel(
    const uint16_t* __restrict__ kv, const int64_t* __restrict__ slot_mapping,
    uint8_t* __restrict__ kv_cache, uint8_t* __restrict__ kv_scale,
    int32_t num_tokens, int64_t num_cache_slots) {
  const int lane = lane_id();
  const int32_t t = static_cast<int32_t>(blockIdx.x) * kWaves + wave_id();
  if (t >= num_tokens) return;
  // The row load goes out with the slot load; a skipped slot turns off the
  // stores rather than returning in front of the row load.  The empty asm
  // statement takes both loaded values, so hipcc cannot sink the row load
  // below the test of the slot (it did, and the row then waited for it).
  u32x4_t raw = load16<true>(kv + static_cast<int64_t>(t) * 512 + lane * 8);
  int64_t slot = slot_mapping[t];
  __asm__ volatile("" : "+v"(raw), "+s"(slot));
  float y[8];
  unpack8(raw, y);
  if (slot >= 0 && slot < num_cache_slots)
    quantise_store_row(y, lane, kv_cache + slot * 576, kv_scale + slot * 8);
}

int to_status(hipError_t e) { return e == hipSuccess ? FP8KV_OK : FP8KV_ERR_LAUNCH; }

}  // namespace

int launch_rms_norm_rows(const uint16_t* x, uint16_t* out, const uint16_t* weight,
                         int64_t num_rows, float eps, hipStream_t stream) {
  const int64_t per_block = static_cast<int64_t>(kWaves) * kRowsPerWave;
  const int64_t blocks = (num_rows + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFF) return FP8KV_ERR_SHAPE;
  void* args[] = {&x, &out, &weight, &num_rows, &eps};
  const unsigned lds = blocks >= kNormCapMinBlocks
                           ? static_cast<unsigned>(lds_for_blocks_per_cu(kNormCapBlocksPerCu))
                           : 0u;
  return to_status(hipLaunchKernel(
      reinterpret_cast<const void*>(&rms_norm_rows_kernel<kRowsPerWave>),
      dim3(static_cast<uint32_t>(blocks)), dim3(kWaves * 64), args, lds, stream));
}

int launch_rope_rows(uint16_t* x, const float* cos_sin, const int64_t* positions,
                     int64_t num_tokens, int32_t rows_per_token,
                     int64_t max_position, hipStream_t stream) {
  int64_t num_rows = num_tokens * rows_per_token;
  const int64_t per_block = static_cast<int64_t>(kWaves) * 8;
  const int64_t blocks = (num_rows + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFF) return FP8KV_ERR_SHAPE;
  void* args[] = {&x, &cos_sin, &positions, &num_rows, &rows_per_token,
                  &max_position};
  return to_status(hipLaunchKernel(reinterpret_cast<const void*>(&rope_rows_kernel),
                                   dim3(static_cast<uint32_t>(blocks)),
                                   dim3(kWaves * 64), args, 0, stream));
}

int launch_kv_quant_insert(const uint16_t* kv, const int64_t* slot_mapping,
                           uint8_t* kv_cache, uint8_t* kv_scale, int32_t num_tokens,
                           int64_t num_cache_slots, hipStream_t stream) {
  const int64_t blocks = (static_cast<int64_t>(num_tokens) + kWaves - 1) / kWaves;
  void* args[] = {&kv, &slot_mapping, &kv_cache, &kv_scale, &num_tokens,
                  &num_cache_slots};
  return to_status(hipLaunchKernel(
      reinterpret_cast<const void*>(&kv_quant_insert_kernel),
      dim3(static_cast<uint32_t>(blocks)), dim3(kWaves * 64), args, 0, stream));
}

}  // namespace fp8kv
