// The packed Q/K operator taken apart into separate launches, the baseline
// InfiniOps PR #1019 "Benchmark / Performance Impact" measures the fused call
// against: RmsNorm of the Q heads and of the K heads into preallocated
// outputs, then RotaryEmbedding of each (four launches).  Every stage reads
// and writes bf16 in HBM:
//
//   rms_norm_heads   out[t, h, :] = bf16(head / rms(head) * w), where head h
//                    of token t starts at x + t * x_token_stride + h * 128
//   rope_neox_heads  in place on x [T, H, 128]: NeoX pairs (i, i + 64)
//                    rotated by cos_sin_cache[positions[t]]
//
// The layouts follow the fused packed kernel: a 128-wide head is one 16-byte
// vector per lane of a 16-lane row, four heads per wave access; the NeoX
// partner of lane l sits in lane l +- 8 of the same row (DPP row_ror:8).  The
// baseline is built the way the fused kernel is (one wave per block, every
// load of a wave issued before its first wait, non-temporal streams, stores
// rather than an early return turned off by a bad index), so a fusion
// speedup measured against it is not inflated by a weaker comparison.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "prologue_launch.hpp"
#include "wave_ops.hpp"

namespace fp8kv {
namespace {

constexpr int kHeadElems = 128;

// U accesses (4U heads) per one-wave block.
template <int U>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(8, 8)))
rms_norm_heads_kernel(const uint16_t* __restrict__ x, int64_t x_token_stride,
                      uint16_t* __restrict__ out,
                      const uint16_t* __restrict__ weight, int32_t num_heads_total,
                      int32_t heads_per_token, float eps) {
  const int lane = lane_id();
  const int row = lane >> 4;
  const int l16 = lane & 15;
  // Head indices in 32-bit unsigned arithmetic: the last block's padding can
  // pass 2^31 - 1 when the heads in all come close to it.
  const uint32_t total = static_cast<uint32_t>(num_heads_total);
  const uint32_t g0 = blockIdx.x * 4u * U;  // < total
  u32x4_t v[U];
  uint32_t gh[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    gh[u] = g0 + 4u * u + row;
    // heads past the last re-read the block's first head and are not stored
    const uint32_t g = gh[u] < total ? gh[u] : g0;
    const uint32_t t = g / static_cast<uint32_t>(heads_per_token);
    const uint32_t h = g - t * static_cast<uint32_t>(heads_per_token);
    v[u] = load16<true>(x + static_cast<int64_t>(t) * x_token_stride +
                        static_cast<int64_t>(h) * kHeadElems + l16 * 8);
  }
  float w[8];
  unpack8(load16<false>(weight + l16 * 8), w);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float f[8];
    unpack8(v[u], f);
    const float ss = row16_sum(sum_sq8(f));
    const float r = __builtin_amdgcn_rsqf(fmaf(ss, 1.0f / kHeadElems, eps));
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = f[j] * r * w[j];
    if (gh[u] < total)
      store16<true>(out + static_cast<int64_t>(gh[u]) * kHeadElems + l16 * 8,
                    u32x4_t{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]),
                            pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7])});
  }
}

template <int U>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(8, 8)))
rope_neox_heads_kernel(uint16_t* __restrict__ x, const float* __restrict__ cos_sin,
                       const int64_t* __restrict__ positions,
                       int32_t num_heads_total, int32_t heads_per_token,
                       int64_t max_position) {
  const int lane = lane_id();
  const int row = lane >> 4;
  const int l16 = lane & 15;
  const uint32_t total = static_cast<uint32_t>(num_heads_total);
  const uint32_t g0 = blockIdx.x * 4u * U;  // < total
  u32x4_t v[U];
  uint32_t gh[U];
  uint32_t tok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    gh[u] = g0 + 4u * u + row;
    const uint32_t g = gh[u] < total ? gh[u] : g0;
    tok[u] = g / static_cast<uint32_t>(heads_per_token);
    v[u] = load16<true>(x + static_cast<int64_t>(g) * kHeadElems + l16 * 8);
  }
  // keep the head loads ahead of the position loads
  __builtin_amdgcn_sched_barrier(0);
  int64_t pos[U];
#pragma unroll
  for (int u = 0; u < U; ++u) pos[u] = positions[tok[u]];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // An out-of-range position turns off the store; its angles come from
    // row 0.  Lane l of a row: pair index i = 8 (l mod 8) + j; the first half
    // of the head takes n c - n' s, the second n c + n' s.
    const bool ok = pos[u] >= 0 && pos[u] < max_position;
    const float* rowp = cos_sin + (ok ? pos[u] : 0) * kHeadElems + (l16 & 7) * 8;
    const f32x4_t c0 = load16f(rowp), c1 = load16f(rowp + 4);
    f32x4_t s0 = load16f(rowp + 64), s1 = load16f(rowp + 68);
    if (l16 < 8) {
      s0 = -s0;
      s1 = -s1;
    }
    const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    const float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    float n[8], o[8];
    unpack8(v[u], n);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = dpp<kDppRowRor8>(n[j]);  // partner element i +- 64
      o[j] = n[j] * c[j] + p * s[j];
    }
    if (ok && gh[u] < total)
      store16<true>(x + static_cast<int64_t>(gh[u]) * kHeadElems + l16 * 8,
                    u32x4_t{pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]),
                            pack_bf16(o[4], o[5]), pack_bf16(o[6], o[7])});
  }
}

constexpr int kNormUnroll = 3;
constexpr int kRopeUnroll = 2;

int to_status(hipError_t e) { return e == hipSuccess ? FP8KV_OK : FP8KV_ERR_LAUNCH; }

}  // namespace

int launch_rms_norm_heads(const uint16_t* x, int64_t x_token_stride, uint16_t* out,
                          const uint16_t* weight, int32_t num_tokens,
                          int32_t num_heads, float eps, hipStream_t stream) {
  int32_t total = num_tokens * num_heads;  // checked to fit by the caller
  const int64_t per = 4 * kNormUnroll;
  const int64_t blocks = (static_cast<int64_t>(total) + per - 1) / per;
  void* args[] = {&x, &x_token_stride, &out, &weight, &total, &num_heads, &eps};
  return to_status(hipLaunchKernel(
      reinterpret_cast<const void*>(&rms_norm_heads_kernel<kNormUnroll>),
      dim3(static_cast<uint32_t>(blocks)), dim3(64), args, 0, stream));
}

int launch_rope_neox_heads(uint16_t* x, const float* cos_sin,
                           const int64_t* positions, int32_t num_tokens,
                           int32_t num_heads, int64_t max_position,
                           hipStream_t stream) {
  int32_t total = num_tokens * num_heads;
  const int64_t per = 4 * kRopeUnroll;
  const int64_t blocks = (static_cast<int64_t>(total) + per - 1) / per;
  void* args[] = {&x, &cos_sin, &positions, &total, &num_heads, &max_position};
  return to_status(hipLaunchKernel(
      reinterpret_cast<const void*>(&rope_neox_heads_kernel<kRopeUnroll>),
      dim3(static_cast<uint32_t>(blocks)), dim3(64), args, 0, stream));
}

}  // namespace fp8kv
