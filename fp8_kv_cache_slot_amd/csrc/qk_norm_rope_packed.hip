// Packed-QKV FusedQkNormRope for gfx950 (InfiniOps PR #1019 "FusedQkNormRope",
// "Summary"): in qkv[T, (Hq+Hk+Hv)*128], every Q head (q_weight) and K head
// (k_weight) is RMS-normalised and rotated with full-head NeoX RoPE in place;
// V heads are never read or written.
//
// Layout of the work.  A 128-element bf16 head is one 16-byte vector per lane
// of a 16-lane row, so one wave access covers four heads (rows 0..3 take heads
// g, g+4, g+8, ... of its range).  A token's Q and K heads are split over
// waves of three accesses (12 heads) each, and a token's waves form one block
// (a token with more than kMaxBlockWaves waves takes several blocks).  The
// block's first wave reads the token's position and requests its cos/sin
// row before its own head loads, and hands the row to the other waves through
// LDS at the block's one barrier; the other waves go straight to their head
// loads.  Lane l of a row holds dims 8l..8l+7; its NeoX partner dims
// (i +- 64) sit in lane l +- 8 of the same row, which DPP row_ror:8 delivers
// in one register move, so the update is in place without any workspace and
// without a read/write hazard (each lane reads and writes only its own 16
// bytes).  The row's sum of squares is four DPP steps.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "occupancy.hpp"
#include "prologue_launch.hpp"
#include "wave_ops.hpp"

namespace fp8kv {
namespace {

constexpr int kUnroll = 3;         // accesses (of four heads) per wave
constexpr int kMaxBlockWaves = 8;  // waves of one token per block

// Measured on MI355X with cold caches, 16/8/8 heads of 128 (two waves per
// token, one block), against the same three accesses per wave in one-wave
// blocks that each read the position and cos/sin themselves: 6.80 / 7.20 us
// at 1024 tokens, 8.52 / 9.28 at 2048, 10.76 / 11.32 at 3072, 13.00 / 13.28
// at 4096, level from 8192 to 32768 tokens, outputs identical (an in-place
// streaming kernel over the same bytes: 6.32 / 8.08 / 9.88 / 11.72 us).  One
// access per wave in blocks of six waves was as fast at 1024 tokens but 8-12%
// slower from 4096 up; two accesses per wave fell between.  Without the
// barrier every wave waits for the position -> cos/sin round trip itself,
// and at these sizes the chip holds all the waves at once, so that round trip
// is the whole kernel's tail.  61 VGPRs: eight waves per SIMD.
//
// The build preloads the first 14 argument dwords into SGPRs (user-SGPR
// kernarg preload), so the arguments a wave needs before its first loads
// (addresses, head counts, the block shape) come first; q_weight lands in the
// preloaded dwords too, k_weight, max_position and eps are loaded while the
// heads are in flight.
__global__ void __launch_bounds__(kMaxBlockWaves * 64) qk_norm_rope_packed_kernel(
    uint16_t* __restrict__ qkv, const float* __restrict__ cos_sin,
    const int64_t* __restrict__ position_ids, int32_t num_heads_q,
    int32_t num_heads_k, int32_t row_elems, int32_t blocks_per_token,
    int32_t waves_per_block, const uint16_t* __restrict__ q_weight,
    const uint16_t* __restrict__ k_weight, int64_t max_position, float eps) {
  constexpr int U = kUnroll;
  __shared__ f32x4_t cs_lds[32];  // the token's row: 64 cosines, then 64 sines
  __shared__ int32_t valid_lds;
  const int lane = lane_id();
  const int wave = wave_id();
  // one block per token unless a token has more than kMaxBlockWaves waves
  // (no division on the usual path, in front of the position load)
  const int32_t t = blocks_per_token == 1
                        ? static_cast<int32_t>(blockIdx.x)
                        : static_cast<int32_t>(blockIdx.x) / blocks_per_token;
  const int32_t part = static_cast<int32_t>(blockIdx.x) - t * blocks_per_token;
  const int32_t h0 = (part * waves_per_block + wave) * 4 * U;  // first head of the wave
  const int g = lane >> 4;   // head slot within the row group
  const int l16 = lane & 15;
  const int32_t nh = num_heads_q + num_heads_k;
  uint16_t* base = qkv + static_cast<int64_t>(t) * row_elems + l16 * 8;

  // The block's first wave: the position, its wait, the cos/sin row (lanes
  // 0..31, 16 bytes each), ahead of its head loads.  A position out of range
  // turns off the token's stores, not an early return (every wave must reach
  // the barrier); its cos/sin reads use row 0.
  f32x4_t cs_v = {0.f, 0.f, 0.f, 0.f};
  bool valid0 = false;
  if (wave == 0) {
    const int64_t pos_in = position_ids[t];
    valid0 = pos_in >= 0 && pos_in < max_position;
    const int64_t pos = valid0 ? pos_in : 0;
    cs_v = load16f(cos_sin + pos * 128 + (lane & 31) * 4);
  }
  __builtin_amdgcn_sched_barrier(0);  // the head loads after these

  // Heads past the last one re-read head 0 (in bounds) and are not stored.
  // A weight of a group without heads may be null, so that group borrows the
  // other pointer (Hq + Hk >= 1, so one is non-null).
  u32x4_t x[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int32_t h = h0 + 4 * u + g;
    x[u] = load16<true>(base + (h < nh ? h : 0) * 128);
  }
  const u32x4_t wqr = load16<false>((num_heads_q > 0 ? q_weight : k_weight) + l16 * 8);
  const u32x4_t wkr = load16<false>((num_heads_k > 0 ? k_weight : q_weight) + l16 * 8);
  __builtin_amdgcn_sched_barrier(0);
  if (wave == 0) {
    if (lane < 32) cs_lds[lane] = cs_v;
    if (lane == 0) valid_lds = valid0 ? 1 : 0;
  }
  __syncthreads();
  const bool valid = valid_lds != 0;

  // cos_i, sin_i for the pair index i = 8 (l16 mod 8) + j of this lane.  The
  // first half of the head takes  n_i c - n_{i+64} s, the second half
  // n_{i+64} c + n_i s: fold the sign into the sine once.
  const int i0 = (l16 & 7) * 2;
  const f32x4_t c0 = cs_lds[i0], c1 = cs_lds[i0 + 1];
  f32x4_t s0 = cs_lds[16 + i0], s1 = cs_lds[16 + i0 + 1];
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
      store16_nt_sc1(base + h * 128, v);
    }
  }
}

// The kernel's LDS: the token's cos/sin row and its validity flag.
static_assert(32 * sizeof(f32x4_t) + sizeof(int32_t) + 16 <= kMaxStaticLds,
              "the occupancy cap assumes the kernel's own LDS fits kMaxStaticLds");

// Occupancy cap for large launches, by waves per block (index).  Measured on
// MI355X with cold caches against the same launch uncapped, outputs
// identical: at 16/8/8 heads (two-wave blocks) 7 blocks per CU takes 36.20 /
// 65.73 / 124.97 / 245.6 us at 16384 / 32768 / 65536 / 131072 tokens against
// 36.76 / 68.85 / 132.86 / 266.4 (8 blocks per CU: 36.70 / 67.85 / 130.14 /
// 262.6; 5 blocks: 273.9 at 131072), but 21.36 against 21.32 at 8192 tokens
// and 13.50 against 12.90 at 4096.  At about 65536 waves and more: 32/4/4
// heads (3 waves) with 5 blocks -2.6% / -3.9% at 8 / 16 chip fills of 8192
// waves, 40/8/8 (4 waves) with 4 blocks -1.7% / -4.3%, 48/8/8 (5 waves) with
// 4 blocks -1.7% / -2.5%; 8/2/2 (one wave) with 16 blocks -3.2% at 16 fills
// and level at 8.  Blocks of 6 to 8 waves gained nothing from any cap.
constexpr int kCapBlocksPerCu[kMaxBlockWaves + 1] = {0, 16, 7, 5, 4, 4, 0, 0, 0};
constexpr int64_t kCapMinWaves = 65536;     // blocks of 2-5 waves
constexpr int64_t kCapMinWaves1 = 131072;   // one-wave blocks

}  // namespace

int launch_packed(const PackedArgs& a, hipStream_t stream) {
  constexpr int kHeadsPerWave = 4 * kUnroll;
  const int32_t nh = a.num_heads_q + a.num_heads_k;
  int32_t waves_per_token = (nh + kHeadsPerWave - 1) / kHeadsPerWave;
  if (waves_per_token < 1) waves_per_token = 1;  // no Q/K heads: nothing stored
  int32_t blocks_per_token = (waves_per_token + kMaxBlockWaves - 1) / kMaxBlockWaves;
  int32_t waves_per_block = (waves_per_token + blocks_per_token - 1) / blocks_per_token;
  const int64_t blocks = static_cast<int64_t>(a.num_tokens) * blocks_per_token;
  if (blocks > 0x7FFFFFFF) return FP8KV_ERR_SHAPE;
  const int64_t waves = blocks * waves_per_block;
  const int cap = kCapBlocksPerCu[waves_per_block];
  const bool capped = cap > 0 && waves >= (waves_per_block == 1 ? kCapMinWaves1 : kCapMinWaves);
  const unsigned lds = capped ? static_cast<unsigned>(lds_for_blocks_per_cu(cap)) : 0u;
  void* args[] = {const_cast<uint16_t**>(&a.qkv),
                  const_cast<const float**>(&a.cos_sin),
                  const_cast<const int64_t**>(&a.position_ids),
                  const_cast<int32_t*>(&a.num_heads_q),
                  const_cast<int32_t*>(&a.num_heads_k),
                  const_cast<int32_t*>(&a.row_elems),
                  &blocks_per_token, &waves_per_block,
                  const_cast<const uint16_t**>(&a.q_weight),
                  const_cast<const uint16_t**>(&a.k_weight),
                  const_cast<int64_t*>(&a.max_position),
                  const_cast<float*>(&a.eps)};
  hipError_t err = hipLaunchKernel(
      reinterpret_cast<const void*>(&qk_norm_rope_packed_kernel),
      dim3(static_cast<uint32_t>(blocks)), dim3(waves_per_block * 64), args, lds,
      stream);
  return err == hipSuccess ? FP8KV_OK : FP8KV_ERR_LAUNCH;
}

}  // namespace fp8kv
