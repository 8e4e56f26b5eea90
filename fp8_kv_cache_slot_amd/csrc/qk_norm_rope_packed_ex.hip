// Packed-QKV Q/K RMSNorm + RoPE beyond the guarded fast path (InfiniOps PR
// #1019 "FusedQkNormRope", "Summary" and "Notes for Reviewers": the first
// implementation accepts only bf16, head_dim 128 and full-dimension NeoX
// rotation).  This kernel covers
//   head_dim D in {64, 128, 256}    (8, 16 or 32 lanes per head)
//   rotary_dim R, a multiple of 16, 0 <= R <= D (partial rotary: dims [R, D)
//                are normalised and weighted only)
//   NeoX pairs (i, i + R/2) or interleaved pairs (2i, 2i + 1)
//   bf16 or fp16 qkv and weights
// V heads are never read or written.
//
// Layout of the work.  A head is D/8 lanes of one 16-byte vector each, so a
// wave covers 512/D heads per access.  A token's Q and K heads are split over
// waves of U accesses each (U * 512/D heads).  Large launches put one wave in
// a block, and each wave issues its U loads before it reads the token's
// position, so it waits for one memory round trip, not one per batch of
// heads.  Launches that fit on the chip at once put a token's waves in one
// block, or four one-wave tokens in one block, whose first wave fetches the
// positions and rotary rows for all of them (the forms below); every form
// runs the same arithmetic.  The sum of
// squares is reduced over the head's lanes (DPP row steps, plus one lane
// shuffle across rows for D = 256).  Interleaved pairs sit inside a lane;
// a NeoX partner sits R/16 lanes away within the head and arrives through
// one ds_bpermute per value.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "prologue_launch.hpp"
#include "occupancy.hpp"
#include "wave_ops.hpp"

namespace fp8kv {
namespace {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <bool FP16>
__device__ __forceinline__ void unpack8_any(u32x4_t x, float* f) {
  if constexpr (FP16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // copy the element out first: hipcc (ROCm 7.2) evaluates a
      // __builtin_bit_cast of an ext_vector element as element 0
      const uint32_t word = x[i];
      const float2_t v =
          __builtin_convertvector(__builtin_bit_cast(f16x2_t, word), float2_t);
      f[2 * i] = v[0];
      f[2 * i + 1] = v[1];
    }
  } else {
    unpack8(x, f);
  }
}

template <bool FP16>
__device__ __forceinline__ uint32_t pack2_any(float a, float b) {
  if constexpr (FP16) {
    float2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
  } else {
    return pack_bf16(a, b);
  }
}

// Sum over each group of LPH consecutive lanes (LPH = 8, 16 or 32).
template <int LPH>
__device__ __forceinline__ float head_sum(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppRowHalfMirror>(v);
  if constexpr (LPH >= 16) v += dpp<kDppRowMirror>(v);
  if constexpr (LPH >= 32) v += __shfl_xor(v, 16, 64);
  return v;
}

// Rotation coefficients of one lane (lh: its lane within the head) from the
// token's cos/sin row (R/2 cosines, then R/2 sines), in global memory or in
// LDS: identity outside the rotary dims.  Returns the ds_bpermute byte
// address of the lane's NeoX partner (its own lane otherwise).  Every lane
// reads, at offset 0 outside the rotary dims, behind a test of
// rotary_dim > 0 only (uniform), and selects afterwards: a branch around the
// rotary lanes' reads added a wait for every outstanding load.
template <bool NEOX>
__device__ __forceinline__ int rotation_coefficients(const float* row, int rotary_dim,
                                                     int lh, int lane, float* c, float* s) {
  const int rot_lanes = rotary_dim / 8;
  const bool rotary = lh < rot_lanes;
  int partner = lane;
  const int half = rotary_dim / 2;
  if constexpr (NEOX) {
    // dims 8lh.. pair with dims 8lh +- R/2, R/16 lanes away; the first half
    // takes n c - n' s, the second half n c + n' s.  i0 <= R/2 - 8, so every
    // read stays inside the row (R >= 16 whenever R > 0).
    const bool first = lh < rot_lanes / 2;
    const int i0 = !rotary ? 0 : (first ? 8 * lh : 8 * lh - half);
    f32x4_t c0 = {1.f, 1.f, 1.f, 1.f}, c1 = c0, s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
    if (rotary_dim > 0) {
      c0 = load16f(row + i0); c1 = load16f(row + i0 + 4);
      s0 = load16f(row + half + i0); s1 = load16f(row + half + i0 + 4);
    }
    const float sg = first ? -1.0f : 1.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = rotary ? c0[j] : 1.0f;
      c[4 + j] = rotary ? c1[j] : 1.0f;
      s[j] = rotary ? sg * s0[j] : 0.0f;
      s[4 + j] = rotary ? sg * s1[j] : 0.0f;
    }
    if (rotary) partner = first ? lane + rot_lanes / 2 : lane - rot_lanes / 2;
  } else {
    // pairs 4lh .. 4lh+3 inside the lane
    const int i0 = rotary ? 4 * lh : 0;
    f32x4_t cc = {1.f, 1.f, 1.f, 1.f}, ss = {0.f, 0.f, 0.f, 0.f};
    if (rotary_dim > 0) {
      cc = load16f(row + i0); ss = load16f(row + half + i0);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c[2 * k] = c[2 * k + 1] = rotary ? cc[k] : 1.0f;
      s[2 * k] = rotary ? -ss[k] : 0.0f;
      s[2 * k + 1] = rotary ? ss[k] : 0.0f;
    }
  }
  return partner * 4;
}

// RMSNorm, weight and rotation of a wave's U accesses (heads h0 + u*HPW + g),
// stored in place where the token is valid and the head exists.
template <int D, bool FP16, bool NEOX, int U>
__device__ __forceinline__ void normalise_rotate_store(
    const u32x4_t* x, u32x4_t wqr, u32x4_t wkr, const float* c, const float* s,
    int partner_addr, uint16_t* base, int32_t h0, int g, int32_t num_heads_q,
    int32_t nh, bool valid, float eps) {
  constexpr int LPH = D / 8;
  constexpr int HPW = 64 / LPH;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int32_t h = h0 + u * HPW + g;
    float f[8], n[8], o[8];
    unpack8_any<FP16>(x[u], f);
    const float ss = head_sum<LPH>(sum_sq8(f));
    const float r = __builtin_amdgcn_rsqf(fmaf(ss, 1.0f / D, eps));
    const bool is_q = h < num_heads_q;
    float w[8];
    unpack8_any<FP16>(is_q ? wqr : wkr, w);
#pragma unroll
    for (int j = 0; j < 8; ++j) n[j] = f[j] * r * w[j];
    if constexpr (NEOX) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = __builtin_bit_cast(
            float, __builtin_amdgcn_ds_bpermute(partner_addr,
                                                __builtin_bit_cast(int, n[j])));
        o[j] = n[j] * c[j] + p * s[j];
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        o[2 * k] = n[2 * k] * c[2 * k] + n[2 * k + 1] * s[2 * k];
        o[2 * k + 1] = n[2 * k + 1] * c[2 * k + 1] + n[2 * k] * s[2 * k + 1];
      }
    }
    if (valid && h < nh) {
      u32x4_t v = {pack2_any<FP16>(o[0], o[1]), pack2_any<FP16>(o[2], o[3]),
                   pack2_any<FP16>(o[4], o[5]), pack2_any<FP16>(o[6], o[7])};
      store16_nt_sc1(base + static_cast<int64_t>(h) * D, v);
    }
  }
}

// One wave per block.  Load order: the U head loads, both weight vectors,
// then the position and (depending on it) the cos/sin row, with nothing
// between them that waits.  A weight of a group without heads may be null,
// so that group borrows the other pointer (Hq + Hk >= 1).  (A branch on the
// wave's first access holding a head, which it always does, let hipcc sink
// the head loads below the position's round trip.)  A position out of range
// makes the token's stores, not an early return, conditional; its cos/sin
// reads use row 0.  Heads past the last one re-read head 0 (in bounds) and
// are not stored.
template <int D, bool FP16, bool NEOX, int U>
__global__ void __launch_bounds__(64) qk_norm_rope_packed_ex_kernel(
    uint16_t* __restrict__ qkv, const uint16_t* __restrict__ q_weight,
    const uint16_t* __restrict__ k_weight, const float* __restrict__ cos_sin,
    const int64_t* __restrict__ position_ids, int32_t num_heads_q,
    int32_t num_heads_k, int32_t row_elems, int32_t rotary_dim,
    int32_t waves_per_token, int32_t num_waves, int64_t max_position,
    float eps) {
  constexpr int LPH = D / 8;   // lanes per head
  constexpr int HPW = 64 / LPH;  // heads per wave access
  const int lane = lane_id();
  const int32_t wv = static_cast<int32_t>(blockIdx.x);
  if (wv >= num_waves) return;
  const int32_t t = wv / waves_per_token;
  const int32_t h0 = (wv - t * waves_per_token) * U * HPW;  // first head of the wave
  const int g = lane / LPH;    // head slot within an access
  const int lh = lane % LPH;   // lane within the head: dims 8lh .. 8lh+7
  const int32_t nh = num_heads_q + num_heads_k;
  uint16_t* base = qkv + static_cast<int64_t>(t) * row_elems + lh * 8;

  u32x4_t x[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int32_t h = h0 + u * HPW + g;
    x[u] = load16<true>(base + static_cast<int64_t>(h < nh ? h : 0) * D);
  }
  const u32x4_t wqr = load16<false>((num_heads_q > 0 ? q_weight : k_weight) + lh * 8);
  const u32x4_t wkr = load16<false>((num_heads_k > 0 ? k_weight : q_weight) + lh * 8);
  __builtin_amdgcn_sched_barrier(0);  // keep the position load after these
  const int64_t pos_in = position_ids[t];
  // Without rotary dims no table row is read, so every token is stored.
  const bool in_range = pos_in >= 0 && pos_in < max_position;
  const bool valid = in_range || rotary_dim == 0;
  const int64_t pos = in_range ? pos_in : 0;
  float c[8], s[8];
  const int partner_addr =
      rotation_coefficients<NEOX>(cos_sin + pos * rotary_dim, rotary_dim, lh, lane, c, s);
  normalise_rotate_store<D, FP16, NEOX, U>(x, wqr, wkr, c, s, partner_addr, base, h0, g,
                                           num_heads_q, nh, valid, eps);
}

// A token's waves as one block (a token with more than kExMaxBlockWaves
// waves takes several blocks).  The block's first wave reads the position
// and requests the token's rotary row (R floats, up to 1 KiB) before its own
// head loads, writes it to LDS and the block meets at one barrier; the other
// waves go straight to their head loads.  No wave returns early.  The
// arguments a wave needs before its first loads come first, inside the
// argument dwords the build preloads into SGPRs.
template <int D, bool FP16, bool NEOX, int U>
__global__ void __launch_bounds__(512) qk_norm_rope_packed_ex_token_kernel(
    uint16_t* __restrict__ qkv, const float* __restrict__ cos_sin,
    const int64_t* __restrict__ position_ids, int32_t num_heads_q,
    int32_t num_heads_k, int32_t row_elems, int32_t rotary_dim,
    int32_t blocks_per_token, int32_t waves_per_block,
    const uint16_t* __restrict__ q_weight, const uint16_t* __restrict__ k_weight,
    int64_t max_position, float eps) {
  constexpr int LPH = D / 8;
  constexpr int HPW = 64 / LPH;
  __shared__ f32x4_t cs_lds[64];  // the token's row: R/2 cosines, R/2 sines
  __shared__ int32_t valid_lds;
  const int lane = lane_id();
  const int wave = wave_id();
  const int32_t t = blocks_per_token == 1
                        ? static_cast<int32_t>(blockIdx.x)
                        : static_cast<int32_t>(blockIdx.x) / blocks_per_token;
  const int32_t part = static_cast<int32_t>(blockIdx.x) - t * blocks_per_token;
  const int32_t h0 = (part * waves_per_block + wave) * U * HPW;
  const int g = lane / LPH;
  const int lh = lane % LPH;
  const int32_t nh = num_heads_q + num_heads_k;
  uint16_t* base = qkv + static_cast<int64_t>(t) * row_elems + lh * 8;

  f32x4_t row_v = {0.f, 0.f, 0.f, 0.f};
  bool valid0 = false;
  if (wave == 0) {
    const int64_t pos_in = position_ids[t];
    const bool in_range = pos_in >= 0 && pos_in < max_position;
    valid0 = in_range || rotary_dim == 0;
    const int64_t pos = in_range ? pos_in : 0;
    if (lane * 4 < rotary_dim) row_v = load16f(cos_sin + pos * rotary_dim + lane * 4);
  }
  __builtin_amdgcn_sched_barrier(0);  // the head loads after these

  u32x4_t x[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int32_t h = h0 + u * HPW + g;
    x[u] = load16<true>(base + static_cast<int64_t>(h < nh ? h : 0) * D);
  }
  const u32x4_t wqr = load16<false>((num_heads_q > 0 ? q_weight : k_weight) + lh * 8);
  const u32x4_t wkr = load16<false>((num_heads_k > 0 ? k_weight : q_weight) + lh * 8);
  __builtin_amdgcn_sched_barrier(0);
  if (wave == 0) {
    if (lane * 4 < rotary_dim) cs_lds[lane] = row_v;
    if (lane == 0) valid_lds = valid0 ? 1 : 0;
  }
  __syncthreads();
  const bool valid = valid_lds != 0;
  float c[8], s[8];
  const int partner_addr = rotation_coefficients<NEOX>(
      reinterpret_cast<const float*>(cs_lds), rotary_dim, lh, lane, c, s);
  normalise_rotate_store<D, FP16, NEOX, U>(x, wqr, wkr, c, s, partner_addr, base, h0, g,
                                           num_heads_q, nh, valid, eps);
}

// P tokens of one wave each per block (P = 2 or 4).  The block's first wave
// reads their positions and requests their rotary rows (up to 64 floats
// each, 64/P lanes of 16 bytes per token) before its own head loads, writes
// them to LDS, and the block meets at one barrier.  Tokens past the last one
// re-read the last token (in bounds) and store nothing.
constexpr int kExTokensMaxRotary = 64;  // floats per row

template <int D, bool FP16, bool NEOX, int U, int P>
__global__ void __launch_bounds__(P * 64) qk_norm_rope_packed_ex_tokens_kernel(
    uint16_t* __restrict__ qkv, const float* __restrict__ cos_sin,
    const int64_t* __restrict__ position_ids, int32_t num_heads_q,
    int32_t num_heads_k, int32_t row_elems, int32_t rotary_dim, int32_t num_tokens,
    const uint16_t* __restrict__ q_weight, const uint16_t* __restrict__ k_weight,
    int64_t max_position, float eps) {
  constexpr int LPH = D / 8;
  constexpr int HPW = 64 / LPH;
  constexpr int RL = 64 / P;  // lanes per token row
  static_assert(RL * 4 >= kExTokensMaxRotary, "a row must fit its lanes");
  __shared__ f32x4_t cs_lds[P][RL];
  __shared__ int32_t valid_lds[P];
  const int lane = lane_id();
  const int wave = wave_id();
  const int32_t t0 = static_cast<int32_t>(blockIdx.x) * P;
  const int32_t t = t0 + wave;
  const bool real = t < num_tokens;
  const int g = lane / LPH;
  const int lh = lane % LPH;
  const int32_t nh = num_heads_q + num_heads_k;
  uint16_t* base =
      qkv + static_cast<int64_t>(real ? t : num_tokens - 1) * row_elems + lh * 8;

  // the first wave: lanes RL*p .. RL*p + RL-1 fetch token t0 + p's row
  const int rp = lane / RL, rl = lane % RL;
  f32x4_t row_v = {0.f, 0.f, 0.f, 0.f};
  bool valid0 = false;
  if (wave == 0) {
    const int32_t tp = t0 + rp < num_tokens ? t0 + rp : num_tokens - 1;
    const int64_t pos_in = position_ids[tp];
    const bool in_range = pos_in >= 0 && pos_in < max_position;
    valid0 = in_range || rotary_dim == 0;
    const int64_t pos = in_range ? pos_in : 0;
    if (rl * 4 < rotary_dim) row_v = load16f(cos_sin + pos * rotary_dim + rl * 4);
  }
  __builtin_amdgcn_sched_barrier(0);  // the head loads after these

  u32x4_t x[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int32_t h = u * HPW + g;
    x[u] = load16<true>(base + static_cast<int64_t>(h < nh ? h : 0) * D);
  }
  const u32x4_t wqr = load16<false>((num_heads_q > 0 ? q_weight : k_weight) + lh * 8);
  const u32x4_t wkr = load16<false>((num_heads_k > 0 ? k_weight : q_weight) + lh * 8);
  __builtin_amdgcn_sched_barrier(0);
  if (wave == 0) {
    if (rl * 4 < rotary_dim) cs_lds[rp][rl] = row_v;
    if (rl == 0) valid_lds[rp] = valid0 ? 1 : 0;
  }
  __syncthreads();
  const bool valid = real && valid_lds[wave] != 0;
  float c[8], s[8];
  const int partner_addr = rotation_coefficients<NEOX>(
      reinterpret_cast<const float*>(cs_lds[wave]), rotary_dim, lh, lane, c, s);
  normalise_rotate_store<D, FP16, NEOX, U>(x, wqr, wkr, c, s, partner_addr, base, 0, g,
                                           num_heads_q, nh, valid, eps);
}

// One wave per block, three accesses (3 KiB) per wave, as for the guarded
// kernel.  Measured on MI355X with cold caches at 8192 tokens of 16/8/8
// heads: D=64 interleaved fp16 14.3 us, D=256 NeoX R=128 bf16 41.8 us, D=128
// interleaved bf16 23.3 us, against 15.7 / 44.1 / 26.1 us for one wave per
// token walking its heads in batches of four accesses (four waves per
// block).  Two accesses per wave: 17.5 / 43.2 / 25.8 us; four: 14.0 / 41.4 /
// 24.9 us; four waves per block: 14.4 / 41.2 / 24.2 us.  Those figures
// predate the load order above, which took the three forms from 14.2 / 41.8
// / 23.1 us to 13.6 / 37.7 / 22.2 us.
constexpr int kExUnroll = 3;

// Occupancy cap for large launches: at most 16 one-wave blocks per CU from
// 131072 waves (16 fills of the chip's 8192 wave slots) up.  Measured on
// MI355X with cold caches at 16/8/8 heads and 16 fills, against the same
// launch uncapped, outputs identical: D=64 interleaved fp16 130.3 against
// 134.8 us, D=256 NeoX R=128 127.6 against 132.0, D=128 NeoX R=64 131.3
// against 134.0, D=128 NeoX R=128 134.5 against 133.2 (level).  At 8 fills the
// cap was level to 1% faster, at 1 to 4 fills 1-8% slower.
constexpr int kExCapBlocksPerCu = 16;
constexpr int64_t kExCapMinWaves = 131072;

// Launches that fit on the chip at once (at most 8192 waves) share each
// token's position and rotary-row fetch within a block: a token's waves in
// one block when it spans two waves or more, four one-wave tokens per block
// with NeoX pairs (rotary rows of up to 64 floats).  Measured on MI355X with cold
// caches, against the one-wave form, outputs identical (us):
//   token blocks: 16/8/8 heads, D=256 NeoX R=128 at 1024 / 2048 tokens 9.24 /
//   8.56 and 13.88 / 12.58; D=128 interleaved at 3072 / 4096 tokens 11.16 /
//   10.44 and 13.56 / 12.32; 32/8/0 heads, D=128 NeoX R=64 fp16 at 1024 /
//   2048 tokens 9.16 / 8.42 and 12.60 / 11.08.  Never more than 1% slower
//   below the limit; beyond it 1-3% faster for some forms and up to 5% slower
//   for others (D=128 interleaved at 6144 / 8192 tokens 17.42 / 18.24 and
//   21.40 / 22.42).  A token of one wave alone in a block gained nothing
//   (2-5% slower at D=64 with 16/8/8 heads).
//   four tokens per block, NeoX pairs: 16/8/8 heads, D=64 R=32 at 4096 /
//   6144 / 8192 tokens 9.18 / 8.38, 11.42 / 10.10 and 13.80 / 11.72; D=64
//   R=64 fp16 at 5120 / 6144 tokens 10.00 / 9.48 and 11.50 / 10.28; 8/2/2
//   heads, D=128 R=64 at 4096 / 8192 tokens 8.76 / 8.20 and 12.60 / 11.24;
//   never more than 2% slower below the limit.
//   two tokens per block, interleaved pairs in bf16 (three runs each):
//   16/8/8 heads, D=64 R=64 at 2048 / 6144 / 8192 tokens 6.80-7.16 /
//   6.62-6.64, 10.92-11.00 / 10.14-10.36 and 13.18-13.30 / 12.60-12.72; D=64
//   R=32 at 6144 tokens 10.72-10.94 / 9.94-10.10; 8/2/2 heads, D=128 R=64 at
//   6144 tokens 10.18-10.44 / 9.52-9.56; never more than 0.6% slower.  Four
//   per block was better at 8192 tokens but up to 3% slower at 2048-4096.
//   With interleaved pairs in fp16 both were mixed (D=64 R=64: 4% slower to
//   5% faster), so those tokens keep one-wave blocks.
constexpr int kExMaxBlockWaves = 8;
constexpr int64_t kExTokenBlockMaxWaves = 8192;

static_assert(sizeof(f32x4_t) * 64 + sizeof(int32_t) <= 64 * 1024, "LDS row");

template <int D, bool FP16, bool NEOX>
int launch_ex(const PackedExArgs& a, hipStream_t stream) {
  constexpr int kHeadsPerWave = kExUnroll * (512 / D);
  const int32_t nh = a.num_heads_q + a.num_heads_k;
  int32_t waves_per_token = (nh + kHeadsPerWave - 1) / kHeadsPerWave;
  if (waves_per_token < 1) waves_per_token = 1;
  const int64_t waves = static_cast<int64_t>(a.num_tokens) * waves_per_token;
  if (waves > 0x7FFFFFFF) return FP8KV_ERR_SHAPE;
  hipError_t err;
  // one-wave tokens per block: four with NeoX pairs, two with interleaved
  // pairs in bf16, none with interleaved pairs in fp16
  constexpr int kTokensPerBlock = NEOX ? 4 : (FP16 ? 1 : 2);
  if constexpr (kTokensPerBlock > 1) {
    if (waves_per_token == 1 && waves <= kExTokenBlockMaxWaves &&
        a.rotary_dim <= kExTokensMaxRotary) {
      int32_t num_tokens = a.num_tokens;
      const int64_t blocks = (waves + kTokensPerBlock - 1) / kTokensPerBlock;
      void* args[] = {const_cast<uint16_t**>(&a.qkv),
                      const_cast<const float**>(&a.cos_sin),
                      const_cast<const int64_t**>(&a.position_ids),
                      const_cast<int32_t*>(&a.num_heads_q),
                      const_cast<int32_t*>(&a.num_heads_k),
                      const_cast<int32_t*>(&a.row_elems),
                      const_cast<int32_t*>(&a.rotary_dim), &num_tokens,
                      const_cast<const uint16_t**>(&a.q_weight),
                      const_cast<const uint16_t**>(&a.k_weight),
                      const_cast<int64_t*>(&a.max_position),
                      const_cast<float*>(&a.eps)};
      err = hipLaunchKernel(
          reinterpret_cast<const void*>(
              &qk_norm_rope_packed_ex_tokens_kernel<D, FP16, NEOX, kExUnroll, kTokensPerBlock>),
          dim3(static_cast<uint32_t>(blocks)), dim3(kTokensPerBlock * 64), args, 0, stream);
      return err == hipSuccess ? FP8KV_OK : FP8KV_ERR_LAUNCH;
    }
  }
  if (waves_per_token >= 2 && waves <= kExTokenBlockMaxWaves) {
    int32_t blocks_per_token = (waves_per_token + kExMaxBlockWaves - 1) / kExMaxBlockWaves;
    int32_t waves_per_block = (waves_per_token + blocks_per_token - 1) / blocks_per_token;
    const int64_t blocks = static_cast<int64_t>(a.num_tokens) * blocks_per_token;
    void* args[] = {const_cast<uint16_t**>(&a.qkv),
                    const_cast<const float**>(&a.cos_sin),
                    const_cast<const int64_t**>(&a.position_ids),
                    const_cast<int32_t*>(&a.num_heads_q),
                    const_cast<int32_t*>(&a.num_heads_k),
                    const_cast<int32_t*>(&a.row_elems),
                    const_cast<int32_t*>(&a.rotary_dim),
                    &blocks_per_token, &waves_per_block,
                    const_cast<const uint16_t**>(&a.q_weight),
                    const_cast<const uint16_t**>(&a.k_weight),
                    const_cast<int64_t*>(&a.max_position),
                    const_cast<float*>(&a.eps)};
    err = hipLaunchKernel(
        reinterpret_cast<const void*>(
            &qk_norm_rope_packed_ex_token_kernel<D, FP16, NEOX, kExUnroll>),
        dim3(static_cast<uint32_t>(blocks)), dim3(waves_per_block * 64), args, 0, stream);
  } else {
    int32_t num_waves = static_cast<int32_t>(waves);
    void* args[] = {const_cast<uint16_t**>(&a.qkv),
                    const_cast<const uint16_t**>(&a.q_weight),
                    const_cast<const uint16_t**>(&a.k_weight),
                    const_cast<const float**>(&a.cos_sin),
                    const_cast<const int64_t**>(&a.position_ids),
                    const_cast<int32_t*>(&a.num_heads_q),
                    const_cast<int32_t*>(&a.num_heads_k),
                    const_cast<int32_t*>(&a.row_elems),
                    const_cast<int32_t*>(&a.rotary_dim),
                    &waves_per_token, &num_waves,
                    const_cast<int64_t*>(&a.max_position),
                    const_cast<float*>(&a.eps)};
    err = hipLaunchKernel(
        reinterpret_cast<const void*>(&qk_norm_rope_packed_ex_kernel<D, FP16, NEOX, kExUnroll>),
        dim3(static_cast<uint32_t>(waves)), dim3(64), args,
        waves >= kExCapMinWaves
            ? static_cast<unsigned>(lds_for_blocks_per_cu(kExCapBlocksPerCu))
            : 0u,
        stream);
  }
  return err == hipSuccess ? FP8KV_OK : FP8KV_ERR_LAUNCH;
}

template <int D>
int launch_d(const PackedExArgs& a, hipStream_t stream) {
  if (a.is_fp16)
    return a.is_neox ? launch_ex<D, true, true>(a, stream)
                     : launch_ex<D, true, false>(a, stream);
  return a.is_neox ? launch_ex<D, false, true>(a, stream)
                   : launch_ex<D, false, false>(a, stream);
}

}  // namespace

int launch_packed_ex(const PackedExArgs& a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return launch_d<64>(a, stream);
    case 128: return launch_d<128>(a, stream);
    case 256: return launch_d<256>(a, stream);
    default: return FP8KV_ERR_UNSUPPORTED;
  }
}

}  // namespace fp8kv
