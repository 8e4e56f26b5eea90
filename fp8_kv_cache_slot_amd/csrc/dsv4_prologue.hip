// Fused DeepSeek-V4 attention prologue for gfx950:
//   Q heads:  RMSNorm (q_weight) + interleaved RoPE on dims 448..511, in place
//   KV head:  RMSNorm (kv_weight) + RoPE, dims 0..447 quantised to FP8 E4M3 in
//             seven 64-dim blocks with UE8M0 exponents, dims 448..511 kept as
//             bf16, written to the paged cache row slot_mapping[t]
// (FlagGems PR #5449 / #5321, "Performance" and "What the optimisation does").
//
// Layout of the work.  A 512-element bf16 head is exactly one 16-byte vector
// per lane of a 64-lane wave, so every load and store is a fully coalesced
// 1 KiB wave access.  Blocks are uniformly KV or Q, as in the pages' tiled
// design (no divergence between the two paths):
//   blocks [0, kv_blocks)       one KV row per wave
//   blocks [kv_blocks, ...)     one wave = QS consecutive heads of one token
// Each Q wave issues its QS head loads before any arithmetic, so QS KiB are
// in flight per wave.  The q and kv streams are read and written with
// non-temporal loads and stores: none of it is reused, and keeping it out of
// the caches measured 9% faster on MI355X.  The q heads are stored with
// device scope as well ("nt sc1", store16_nt_sc1), 2.3-3.6% faster again.  The wave reads the token's
// position and cos/sin row once and reduces the sum of squares with DPP row
// steps plus four v_readlane of the row totals.  The rotary dims 448..511 sit
// in lanes 56..63, eight values (four interleaved pairs) per lane, so rotation
// never leaves the register file.  The KV quantisation block of dims
// 64b..64b+63 is the lane group 8b..8b+7:
// its absolute maximum is three DPP steps.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kv_quant.hpp"
#include "prologue_launch.hpp"
#include "wave_ops.hpp"

namespace fp8kv {
namespace {

constexpr int kRopeLane0 = 56;  // first lane holding a rotary dim (448 / 8)

// Normalise one head held as 8 bf16 per lane: y = x / rms(x) * w (fp32).
__device__ __forceinline__ void rms_normalise(u32x4_t x, const float* w,
                                              float eps, float* y) {
  float f[8];
  unpack8(x, f);
  const float ss = wave64_sum(sum_sq8(f));
  const float r = __builtin_amdgcn_rsqf(fmaf(ss, 1.0f / 512.0f, eps));
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = f[j] * r * w[j];
}

// Interleaved rotation of the four pairs a lane of 56..63 holds.
__device__ __forceinline__ void rotate4(float* y, f32x4_t c, f32x4_t s) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = y[2 * k], b = y[2 * k + 1];
    y[2 * k] = a * c[k] - b * s[k];
    y[2 * k + 1] = b * c[k] + a * s[k];
  }
}

// The row load goes out first and the slot and position loads overlap it.
// A skipped token (slot or position out of range) turns off the stores, not
// the loads: with an early return on a loaded index in front of them, hipcc
// moves the loads below the branch and the wave waits for the index, then
// for the row, one memory round trip after the other.  The cos/sin row index
// depends on the slot as well (a skipped token rotates with row 0, and stores
// nothing), so the slot load is issued with the position load instead of
// being sunk to the stores at the end.
template <bool SCALAR>
__device__ __forceinline__ void kv_row(
    int32_t t, const uint16_t* __restrict__ kv,
    const uint16_t* __restrict__ kv_weight, const float* __restrict__ cos_sin,
    const int64_t* __restrict__ positions,
    const int64_t* __restrict__ slot_mapping, uint8_t* __restrict__ kv_cache,
    uint8_t* __restrict__ kv_scale, const float* __restrict__ scalar_scale,
    int64_t num_cache_slots, int64_t max_position, float eps) {
  const int lane = lane_id();
  const u32x4_t x = load16<true>(kv + static_cast<int64_t>(t) * 512 + lane * 8);
  float w[8];
  unpack8(load16<false>(kv_weight + lane * 8), w);
  const int64_t slot = slot_mapping[t];
  const int64_t pos_in = positions[t];
  const bool write = pos_in >= 0 && pos_in < max_position && slot >= 0 &&
                     slot < num_cache_slots;
  const int64_t pos = write ? pos_in : 0;
  f32x4_t c = {1.f, 1.f, 1.f, 1.f}, s = {0.f, 0.f, 0.f, 0.f};
  if (lane >= kRopeLane0) {
    const float* row = cos_sin + pos * 64 + (lane - kRopeLane0) * 4;
    c = load16f(row);
    s = load16f(row + 32);
  }
  float y[8];
  rms_normalise(x, w, eps, y);
  if (lane >= kRopeLane0) rotate4(y, c, s);

  if constexpr (SCALAR) {
    // read only for a token that is written (the pointer may be NULL when
    // the cache has no pages, and then no token is written)
    if (write)
      quantise_store_row_scalar(y, lane, kv_cache + slot * 576, *scalar_scale);
  } else {
    if (write)
      quantise_store_row(y, lane, kv_cache + slot * 576, kv_scale + slot * 8);
  }
}

template <int WAVES, int QS, bool SCALAR>
__global__ void __launch_bounds__(WAVES * 64) dsv4_prologue_kernel(
    uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const uint16_t* __restrict__ q_weight,
    const uint16_t* __restrict__ kv_weight, const float* __restrict__ cos_sin,
    const int64_t* __restrict__ positions,
    const int64_t* __restrict__ slot_mapping, uint8_t* __restrict__ kv_cache,
    uint8_t* __restrict__ kv_scale, const float* __restrict__ scalar_scale,
    int32_t num_tokens, int32_t num_heads,
    int32_t waves_per_token, int32_t q_waves, int32_t kv_blocks,
    int64_t num_cache_slots, int64_t max_position, float eps) {
  const int lane = lane_id();
  const int wave = wave_id();
  int32_t b = blockIdx.x;
  if (b < kv_blocks) {
    const int32_t t = b * WAVES + wave;
    if (t < num_tokens)
      kv_row<SCALAR>(t, kv, kv_weight, cos_sin, positions, slot_mapping,
                     kv_cache, kv_scale, scalar_scale, num_cache_slots,
                     max_position, eps);
    return;
  }
  b -= kv_blocks;
  const int32_t qwave = b * WAVES + wave;
  if (qwave >= q_waves) return;

  // The streaming loads go out first; index arithmetic, the position load and
  // its range check overlap them.  When H is a multiple of QS the wave's heads
  // are the flat rows qwave*QS .. qwave*QS+QS-1 of q viewed as [T*H, 512], so
  // the address needs no token index at all.
  const bool dense = (num_heads % QS) == 0;
  int32_t t = 0, h0 = 0;
  int64_t row0;
  if (dense) {
    row0 = static_cast<int64_t>(qwave) * QS;
  } else {
    t = qwave / waves_per_token;
    h0 = (qwave - t * waves_per_token) * QS;
    row0 = static_cast<int64_t>(t) * num_heads + h0;
  }
  uint16_t* base = q + row0 * 512 + lane * 8;
  u32x4_t x[QS];
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    // heads past the last one re-read the wave's first head (in bounds) and
    // are not stored
    const bool ok = dense || h0 + s < num_heads;
    x[s] = load16<true>(base + (ok ? s * 512 : 0));
  }
  float w[8];
  unpack8(load16<false>(q_weight + lane * 8), w);
  if (dense) {
    t = qwave / waves_per_token;
    h0 = (qwave - t * waves_per_token) * QS;
  }
  // An out-of-range position turns off the token's stores, not an early
  // return, so that no branch on it sits in front of the loads above.
  const int64_t pos_in = positions[t];
  const bool pos_ok = pos_in >= 0 && pos_in < max_position;
  const int64_t pos = pos_ok ? pos_in : 0;
  f32x4_t c = {1.f, 1.f, 1.f, 1.f}, sn = {0.f, 0.f, 0.f, 0.f};
  if (lane >= kRopeLane0) {
    const float* row = cos_sin + pos * 64 + (lane - kRopeLane0) * 4;
    c = load16f(row);
    sn = load16f(row + 32);
  }

#pragma unroll
  for (int s = 0; s < QS; ++s) {
    if (h0 + s >= num_heads) break;
    float y[8];
    rms_normalise(x[s], w, eps, y);
    if (lane >= kRopeLane0) rotate4(y, c, sn);
    u32x4_t o = {pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]),
                 pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7])};
    if (pos_ok) store16_nt_sc1(base + s * 512, o);
  }
}

template <int WAVES, int QS, bool SCALAR>
int launch(const PrologueArgs& a, hipStream_t stream) {
  const int32_t waves_per_token = (a.num_heads + QS - 1) / QS;
  const int64_t kv_blocks = (static_cast<int64_t>(a.num_tokens) + WAVES - 1) / WAVES;
  const int64_t q_waves64 = static_cast<int64_t>(a.num_tokens) * waves_per_token;
  int32_t q_waves = static_cast<int32_t>(q_waves64);
  const int64_t q_blocks = (q_waves64 + WAVES - 1) / WAVES;
  const int64_t blocks = kv_blocks + q_blocks;
  if (blocks > 0x7FFFFFFF) return FP8KV_ERR_SHAPE;
  int32_t kvb = static_cast<int32_t>(kv_blocks);
  void* args[] = {
      const_cast<uint16_t**>(&a.q),          const_cast<const uint16_t**>(&a.kv),
      const_cast<const uint16_t**>(&a.q_weight),
      const_cast<const uint16_t**>(&a.kv_weight),
      const_cast<const float**>(&a.cos_sin),
      const_cast<const int64_t**>(&a.positions),
      const_cast<const int64_t**>(&a.slot_mapping),
      const_cast<uint8_t**>(&a.kv_cache),    const_cast<uint8_t**>(&a.kv_scale),
      const_cast<const float**>(&a.scalar_scale),
      const_cast<int32_t*>(&a.num_tokens),   const_cast<int32_t*>(&a.num_heads),
      const_cast<int32_t*>(&waves_per_token), &q_waves, &kvb,
      const_cast<int64_t*>(&a.num_cache_slots),
      const_cast<int64_t*>(&a.max_position), const_cast<float*>(&a.eps)};
  hipError_t err = hipLaunchKernel(
      reinterpret_cast<const void*>(&dsv4_prologue_kernel<WAVES, QS, SCALAR>),
      dim3(static_cast<uint32_t>(blocks)), dim3(WAVES * 64), args, 0, stream);
  return err == hipSuccess ? FP8KV_OK : FP8KV_ERR_LAUNCH;
}

}  // namespace

// Instantiated (waves per block, Q heads per wave) shapes.  (1, 1) is the
// small-batch kernel: one head per 64-lane block.
int launch_prologue(const PrologueArgs& a, int waves, int qs, hipStream_t stream) {
  // The scalar-scale cache convention is built in two shapes only: one head
  // per one-wave block (the small-batch and default tiled shape), and 4 waves
  // x 2 heads, which every other tiling selects.
  if (a.scalar) {
    if (waves == 1 && qs == 1) return launch<1, 1, true>(a, stream);
    return launch<4, 2, true>(a, stream);
  }
#define FP8KV_SHAPE(W, S)                                            \
  if (waves == W && qs == S) return launch<W, S, false>(a, stream);
  FP8KV_SHAPE(1, 1)
  FP8KV_SHAPE(1, 2)
  FP8KV_SHAPE(2, 1)
  FP8KV_SHAPE(2, 2)
  FP8KV_SHAPE(4, 1)
  FP8KV_SHAPE(4, 2)
  FP8KV_SHAPE(4, 4)
  FP8KV_SHAPE(8, 1)
  FP8KV_SHAPE(8, 2)
  FP8KV_SHAPE(8, 4)
  FP8KV_SHAPE(16, 1)
  FP8KV_SHAPE(16, 2)
#undef FP8KV_SHAPE
  return FP8KV_ERR_UNSUPPORTED;
}

bool prologue_shape_built(int waves, int qs) {
  static const int shapes[][2] = {{1, 1}, {1, 2}, {2, 1}, {2, 2}, {4, 1}, {4, 2},
                                  {4, 4}, {8, 1}, {8, 2}, {8, 4}, {16, 1}, {16, 2}};
  for (const auto& s : shapes)
    if (s[0] == waves && s[1] == qs) return true;
  return false;
}

}  // namespace fp8kv
