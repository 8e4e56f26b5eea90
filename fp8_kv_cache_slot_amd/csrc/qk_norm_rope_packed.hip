// Packed-QKV FusedQkNormRope for gfx950 (InfiniOps PR #1019 "FusedQkNormRope",
// "Summary"): in qkv[T, (Hq+Hk+Hv)*128], every Q head (q_weight) and K head
// (k_weight) is RMS-normalised and rotated with full-head NeoX RoPE in place;
// V heads are never read or written.
//
// Layout of the work.  A 128-element bf16 head is one 16-byte vector per lane
// of a 16-lane row, so one wave access covers four heads (rows 0..3 take heads
// g, g+4, g+8, ... of its range).  A token's Q and K heads are split over
// waves of U accesses (4U heads) each; a wave reads the token's position and
// requests its cos/sin row before it issues its U head loads.  Lane l of a
// row holds dims 8l..8l+7;
// its NeoX partner dims (i +- 64) sit in lane l +- 8 of the same row, which
// DPP row_ror:8 delivers in one register move, so the update is in place
// without any workspace and without a read/write hazard (each lane reads and
// writes only its own 16 bytes).  The row's sum of squares is four DPP steps.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "prologue_launch.hpp"
#include "wave_ops.hpp"

namespace fp8kv {
namespace {

// Eight waves per SIMD (at most 64 VGPRs): 8192 tokens of 16 + 8 heads then
// fit on the chip in one pass.
template <int WAVES, int U>
__global__ void __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(8, 8))) qk_norm_rope_packed_kernel(
    uint16_t* __restrict__ qkv, const uint16_t* __restrict__ q_weight,
    const uint16_t* __restrict__ k_weight, const float* __restrict__ cos_sin,
    const int64_t* __restrict__ position_ids, int32_t num_heads_q,
    int32_t num_heads_k, int32_t row_elems, int32_t waves_per_token,
    int32_t num_waves, int64_t max_position, float eps) {
  const int lane = lane_id();
  const int32_t wv = static_cast<int32_t>(blockIdx.x) * WAVES + wave_id();
  if (wv >= num_waves) return;
  const int32_t t = wv / waves_per_token;
  const int32_t h0 = (wv - t * waves_per_token) * 4 * U;  // first head of the wave
  const int g = lane >> 4;   // head slot within the row group
  const int l16 = lane & 15;
  const int32_t nh = num_heads_q + num_heads_k;

  // Load order: the position, its wait, the token's cos/sin row, then the U
  // head loads and both weight vectors.  The cos/sin requests then enter the
  // memory queues ahead of the wave's own head traffic instead of behind it
  // (with the heads first, hipcc also hoisted the first head's unpacking
  // above the cos/sin loads, so they waited for that head to arrive).
  // Measured on MI355X with cold caches, 16/8/8 heads of 128: 22.0 -> 21.0 us
  // at 8192 tokens, 13.4 -> 13.0 at 4096 and 69.8 -> 68.6 at 32768, outputs
  // identical.  A position out of range makes the stores, not an early
  // return, conditional; its cos/sin reads use row 0.  A weight of a group
  // without heads may be null, so that group borrows the other pointer
  // (Hq + Hk >= 1, so one is non-null).  Heads past the last one re-read
  // head 0 (in bounds) and are not stored.
  uint16_t* base = qkv + static_cast<int64_t>(t) * row_elems + l16 * 8;
  const int64_t pos_in = position_ids[t];
  const bool valid = pos_in >= 0 && pos_in < max_position;
  const int64_t pos = valid ? pos_in : 0;

  // cos_i, sin_i for the pair index i = 8 (l16 mod 8) + j of this lane.  The
  // first half of the head takes  n_i c - n_{i+64} s, the second half
  // n_{i+64} c + n_i s: fold the sign into the sine once.
  const float* row = cos_sin + pos * 128 + (l16 & 7) * 8;
  const f32x4_t c0 = load16f(row), c1 = load16f(row + 4);
  f32x4_t s0 = load16f(row + 64), s1 = load16f(row + 68);
  __builtin_amdgcn_sched_barrier(0);  // the head loads after these

  u32x4_t x[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int32_t h = h0 + 4 * u + g;
    x[u] = load16<true>(base + (h < nh ? h : 0) * 128);  // in bounds
  }
  const u32x4_t wqr = load16<false>((num_heads_q > 0 ? q_weight : k_weight) + l16 * 8);
  const u32x4_t wkr = load16<false>((num_heads_k > 0 ? k_weight : q_weight) + l16 * 8);
  __builtin_amdgcn_sched_barrier(0);
  if (l16 < 8) {
    s0 = -s0;
    s1 = -s1;
  }
  const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
  const float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};

#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int32_t h = h0 + 4 * u + g;
    float f[8], n[8];
    unpack8(x[u], f);
    const float ss = row16_sum(sum_sq8(f));
    const float r = __builtin_amdgcn_rsqf(fmaf(ss, 1.0f / 128.0f, eps));
    const bool is_q = h < num_heads_q;
    float w[8];
    unpack8(is_q ? wqr : wkr, w);
#pragma unroll
    for (int j = 0; j < 8; ++j) n[j] = f[j] * r * w[j];
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = dpp<kDppRowRor8>(n[j]);  // partner element, own weight
      o[j] = n[j] * c[j] + p * s[j];
    }
    if (valid && h < nh) {
      u32x4_t v = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]),
                   pack_bf16(o[4], o[5]), pack_bf16(o[6], o[7])};
      store16<true>(base + h * 128, v);
    }
  }
}

// 12 heads per wave, one wave per block: the 16 Q + 8 K heads of a token
// take two single-wave blocks.  Measured on MI355X with cold caches (16/8/8
// heads of 128) at 8192 tokens: 23.8 us with one wave per block, against 24.9
// with two, 25.3-25.5 with four, 26.0 with eight and 28.3 with sixteen; with
// one wave per block, 8 heads per wave took 25.6 us, 16 heads 25.9 us and all
// 24 heads in one wave 34.7 us (register-limited).  At 17 tokens 6.7 us
// against 7.0 us with four waves per block.  With four waves per block the
// position read before the head loads cost 1.5 us at 8192 tokens (27.5 us).
// The load order above took the kernel from 23.6 to 23.1 us at 8192 tokens.
// The build preloads the kernel arguments into SGPRs (user-SGPR kernarg
// preload), so the head loads are a wave's first memory instructions:
// 24.0 -> 22.9 us at 8192 tokens.
constexpr int kPackedWaves = 1;
constexpr int kPackedUnroll = 3;

}  // namespace

int launch_packed(const PackedArgs& a, hipStream_t stream) {
  constexpr int kHeadsPerWave = 4 * kPackedUnroll;
  const int32_t nh = a.num_heads_q + a.num_heads_k;
  int32_t waves_per_token = (nh + kHeadsPerWave - 1) / kHeadsPerWave;
  if (waves_per_token < 1) waves_per_token = 1;  // no Q/K heads: nothing stored
  const int64_t waves = static_cast<int64_t>(a.num_tokens) * waves_per_token;
  if (waves > 0x7FFFFFFF) return FP8KV_ERR_SHAPE;
  int32_t num_waves = static_cast<int32_t>(waves);
  const int64_t blocks = (waves + kPackedWaves - 1) / kPackedWaves;
  void* args[] = {const_cast<uint16_t**>(&a.qkv),
                  const_cast<const uint16_t**>(&a.q_weight),
                  const_cast<const uint16_t**>(&a.k_weight),
                  const_cast<const float**>(&a.cos_sin),
                  const_cast<const int64_t**>(&a.position_ids),
                  const_cast<int32_t*>(&a.num_heads_q),
                  const_cast<int32_t*>(&a.num_heads_k),
                  const_cast<int32_t*>(&a.row_elems),
                  &waves_per_token, &num_waves,
                  const_cast<int64_t*>(&a.max_position),
                  const_cast<float*>(&a.eps)};
  hipError_t err = hipLaunchKernel(
      reinterpret_cast<const void*>(
          &qk_norm_rope_packed_kernel<kPackedWaves, kPackedUnroll>),
      dim3(static_cast<uint32_t>(blocks)), dim3(kPackedWaves * 64), args, 0,
      stream);
  return err == hipSuccess ? FP8KV_OK : FP8KV_ERR_LAUNCH;
}

}  // namespace fp8kv
