// Read side of the paged FP8/UE8M0 KV cache for gfx950: gather rows by slot
// and dequantise them to bf16, the inverse of the fused prologue's insert
// (the cache layout of FlagGems PR #5449 "Performance": FP8 codes with seven
// per-block power-of-two exponents per token).
//
//   out[i, d]       = E4M3(code[s, d]) * 2^(scale[s, d / 64] - 127), d < 448
//   out[i, 448 + j] = stored bf16 rotary value j
//
// Layout of the work.  A 64-lane wave writes one output row (1 KiB of bf16 =
// one 16-byte vector per lane, as in the prologue): lane l < 56 decodes the 8
// code bytes of dims 8l..8l+7 with v_cvt_pk_f32_fp8, scales them exactly by
// the block's power of two with v_ldexp and packs with v_cvt_pk_bf16_f32;
// lanes 56..63 pass the 128 stored rotary bytes through.  Rows come in groups
// of RS consecutive rows per wave (see the kernels).  The output is written
// non-temporally.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "prologue_launch.hpp"
#include "wave_ops.hpp"

namespace fp8kv {
namespace {

constexpr int kRopeLane0 = 56;

// One group of RS rows as loaded.  Every lane issues the same three loads per
// row, with no branch around them (so they stay in flight while other work
// runs): 8 code bytes at dims 8 min(l, 55).., the rotary vector of lane
// 56 + (l & 7), and the exponent byte of block l >> 3 (lanes 56..63 read the
// unused byte 7 of the 8-byte exponent row).  Each lane keeps what it needs.
// A row whose slot is invalid reads slot 0 (the cache has pages here) and is
// stored as zeros.
template <int RS>
struct Rows {
  u32x2_t codes[RS];
  u32x4_t rope[RS];
  uint32_t ebyte[RS];
};

__device__ __forceinline__ bool slot_valid(int64_t s, int64_t num_cache_slots) {
  return s >= 0 && s < num_cache_slots;
}

template <int RS, bool SCALAR>
__device__ __forceinline__ void load_rows(const uint8_t* __restrict__ kv_cache,
                                          const uint8_t* __restrict__ kv_scale,
                                          const int64_t* s, int64_t num_cache_slots,
                                          int lane, Rows<RS>& d) {
  const int cl = lane < kRopeLane0 ? lane : kRopeLane0 - 1;
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    const int64_t slot = slot_valid(s[r], num_cache_slots) ? s[r] : 0;
    const uint8_t* row = kv_cache + slot * 576;
    d.codes[r] = *reinterpret_cast<const u32x2_t*>(row + cl * 8);
    d.rope[r] = *reinterpret_cast<const u32x4_t*>(row + 448 + (lane & 7) * 16);
    if constexpr (SCALAR)
      d.ebyte[r] = 0u;
    else
      d.ebyte[r] = kv_scale[slot * 8 + (lane >> 3)];
  }
}

// Dequantise and store the RS rows of group grp (rows grp*RS ..); fs is the
// scalar scale (SCALAR) or unused.
template <int RS, bool SCALAR>
__device__ __forceinline__ void store_rows(const Rows<RS>& d, const int64_t* s,
                                           float fs, uint16_t* __restrict__ out,
                                           int32_t grp, int32_t num_rows,
                                           int64_t num_cache_slots, int lane) {
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    const int32_t i = grp * RS + r;
    if (i >= num_rows) break;
    const int e = static_cast<int>(d.ebyte[r]) - 127;
    const int lo = static_cast<int>(d.codes[r][0]);
    const int hi = static_cast<int>(d.codes[r][1]);
    const float2_t p[4] = {__builtin_amdgcn_cvt_pk_f32_fp8(lo, false),
                           __builtin_amdgcn_cvt_pk_f32_fp8(lo, true),
                           __builtin_amdgcn_cvt_pk_f32_fp8(hi, false),
                           __builtin_amdgcn_cvt_pk_f32_fp8(hi, true)};
    float v[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (SCALAR) {
        v[2 * k] = p[k][0] * fs;
        v[2 * k + 1] = p[k][1] * fs;
      } else {
        v[2 * k] = __builtin_ldexpf(p[k][0], e);
        v[2 * k + 1] = __builtin_ldexpf(p[k][1], e);
      }
    }
    const u32x4_t q = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]),
                       pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
    const u32x4_t z = {0u, 0u, 0u, 0u};
    const u32x4_t o = slot_valid(s[r], num_cache_slots)
                          ? (lane < kRopeLane0 ? q : d.rope[r])
                          : z;
    store16<true>(out + static_cast<int64_t>(i) * 512 + lane * 8, o);
  }
}

// SCALAR: the scalar-scale convention, out = E4M3(code) * scalar_scale[0]
// (rounded once to fp32, then to bf16) and no exponent bytes are read.
//
// The gather is a chain of two dependent loads: the slots, then the rows.
// Each one-wave block takes one group of RS consecutive rows: the RS slot
// indices are wave-uniform (one scalar load), then every lane issues the
// group's row loads with no branch in front of them, and the rows are
// dequantised and stored.  Many small one-shot blocks keep enough groups in
// flight to hide the two round trips.  Measured on MI355X over all 131072
// slots of a 2048-page cache in random order, caches cold and clean: 41.9 us
// with 4 rows per one-wave block, against 43.6 us with 2 rows, 42.8 with 8,
// 52.2 with 1, 42.3 with two waves of 4 rows and 44.1 with four waves of 2;
// and against 43.9 us for a persistent form in which each wave looped over
// its share of the groups with the next group's loads in flight.
template <int RS, bool SCALAR>
__global__ void __launch_bounds__(64) kv_cache_gather_dequant_kernel(
    const uint8_t* __restrict__ kv_cache, const uint8_t* __restrict__ kv_scale,
    const float* __restrict__ scalar_scale, const int64_t* __restrict__ slots,
    uint16_t* __restrict__ out, int32_t num_rows, int64_t num_cache_slots) {
  const int lane = lane_id();
  const int32_t grp = static_cast<int32_t>(blockIdx.x);
  if (grp * RS >= num_rows) return;
  if (num_cache_slots <= 0) {  // a cache without pages: every row is zero
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < RS; ++r) {
      const int32_t i = grp * RS + r;
      if (i < num_rows) store16<true>(out + static_cast<int64_t>(i) * 512 + lane * 8, z);
    }
    return;
  }
  // Rows past the last one re-read the last slot (in bounds) and are not
  // stored.
  int64_t s[RS];
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    int32_t i = grp * RS + r;
    if (i > num_rows - 1) i = num_rows - 1;
    s[r] = slots[i];
  }
  // with pages, the scalar scale pointer is a checked device pointer
  float fs = 1.0f;
  if constexpr (SCALAR) fs = *scalar_scale;
  Rows<RS> d;
  load_rows<RS, SCALAR>(kv_cache, kv_scale, s, num_cache_slots, lane, d);
  store_rows<RS, SCALAR>(d, s, fs, out, grp, num_rows, num_cache_slots, lane);
}

constexpr int kDequantRows = 4;

// The read side through block tables, as an attention consumer indexes the
// cache: token j of sequence s sits in slot
// block_table[s, j / 64] * 64 + j % 64 and its row goes to
// out[out_offsets[s] + j].  Grid: x = groups of PRS consecutive tokens of a
// sequence (covering max_blocks_per_seq pages), y = sequence.  PRS divides 64,
// so a wave's rows are consecutive slots of one page (PRS * 576 contiguous
// bytes).  The page id, length and output offset are three independent
// loads; every lane then issues its row loads with no branch in front of
// them (an invalid page reads slot 0 and stores zero rows, as in the slot-list
// kernel), and only the stores depend on the length and the output bounds.
//
// SCALAR: the scalar-scale convention, as in the slot-list kernel (no exponent
// bytes read; codes times scalar_scale[0], rounded to fp32, then to bf16).
template <int WAVES, int PRS, bool SCALAR>
__global__ void __launch_bounds__(WAVES * 64) kv_cache_gather_dequant_paged_kernel(
    const uint8_t* __restrict__ kv_cache, const uint8_t* __restrict__ kv_scale,
    const float* __restrict__ scalar_scale,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const int64_t* __restrict__ out_offsets, uint16_t* __restrict__ out,
    int32_t max_blocks_per_seq, int64_t num_pages, int64_t num_rows) {
  static_assert(64 % PRS == 0, "a group must not straddle a page");
  const int lane = lane_id();
  const int32_t seq = static_cast<int32_t>(blockIdx.y);
  // j0 < max_blocks_per_seq * 64: the grid covers exactly that many tokens
  const int32_t j0 = (static_cast<int32_t>(blockIdx.x) * WAVES + wave_id()) * PRS;
  const int64_t page =
      block_table[static_cast<int64_t>(seq) * max_blocks_per_seq + j0 / 64];
  const int32_t len = seq_lens[seq];
  const int64_t first = out_offsets[seq] + j0;
  if (j0 >= len) return;

  const u32x4_t z = {0u, 0u, 0u, 0u};
  if (num_pages <= 0) {  // a cache without pages: every row is zero
#pragma unroll
    for (int r = 0; r < PRS; ++r) {
      const int64_t i = first + r;
      if (j0 + r < len && i >= 0 && i < num_rows)
        store16<true>(out + i * 512 + lane * 8, z);
    }
    return;
  }
  const bool page_ok = page >= 0 && page < num_pages;
  const int64_t slot0 = (page_ok ? page : 0) * 64 + j0 % 64;
  int64_t sl[PRS];
#pragma unroll
  for (int r = 0; r < PRS; ++r) sl[r] = page_ok ? slot0 + r : -1;
  // with pages, the scalar scale pointer is a checked device pointer
  float fs = 1.0f;
  if constexpr (SCALAR) fs = *scalar_scale;
  Rows<PRS> d;
  load_rows<PRS, SCALAR>(kv_cache, kv_scale, sl, num_pages * 64, lane, d);
#pragma unroll
  for (int r = 0; r < PRS; ++r) {
    const int64_t i = first + r;
    if (j0 + r >= len || i < 0 || i >= num_rows) continue;
    const int e = static_cast<int>(d.ebyte[r]) - 127;
    const int lo = static_cast<int>(d.codes[r][0]);
    const int hi = static_cast<int>(d.codes[r][1]);
    const float2_t p[4] = {__builtin_amdgcn_cvt_pk_f32_fp8(lo, false),
                           __builtin_amdgcn_cvt_pk_f32_fp8(lo, true),
                           __builtin_amdgcn_cvt_pk_f32_fp8(hi, false),
                           __builtin_amdgcn_cvt_pk_f32_fp8(hi, true)};
    float v[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (SCALAR) {
        v[2 * k] = p[k][0] * fs;
        v[2 * k + 1] = p[k][1] * fs;
      } else {
        v[2 * k] = __builtin_ldexpf(p[k][0], e);
        v[2 * k + 1] = __builtin_ldexpf(p[k][1], e);
      }
    }
    const u32x4_t q = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]),
                       pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
    const u32x4_t o = page_ok ? (lane < kRopeLane0 ? q : d.rope[r]) : z;
    store16<true>(out + i * 512 + lane * 8, o);
  }
}

// 2 waves of 8 rows (4.6 KiB of contiguous cache rows per wave).  Measured
// on MI355X over all 2048 pages of a cache in a random page order, caches
// cold and clean: 42.5 us for 32 x 4096 and for 256 x 512 tokens, against
// 43.5-44.7 us for 4 x 4, 43.5-43.9 for 4 x 8, 44.5-45.5 for 8 x 4 and
// 46-49 us for 4 x 2 and 4 x 16 (waves x rows per wave).
constexpr int kPagedWaves = 2;
constexpr int kPagedRows = 8;

}  // namespace

int launch_gather_dequant_paged(const PagedDequantArgs& a, hipStream_t stream) {
  constexpr int64_t kTokensPerBlock = int64_t{kPagedWaves} * kPagedRows;
  const int64_t blocks_x = int64_t{a.max_blocks_per_seq} * 64 / kTokensPerBlock;
  if (blocks_x > 0x7FFFFFFF || a.num_seqs > 65535) return FP8KV_ERR_SHAPE;
  void* args[] = {const_cast<const uint8_t**>(&a.kv_cache),
                  const_cast<const uint8_t**>(&a.kv_scale),
                  const_cast<const float**>(&a.scalar_scale),
                  const_cast<const int32_t**>(&a.block_table),
                  const_cast<const int32_t**>(&a.seq_lens),
                  const_cast<const int64_t**>(&a.out_offsets),
                  const_cast<uint16_t**>(&a.out),
                  const_cast<int32_t*>(&a.max_blocks_per_seq),
                  const_cast<int64_t*>(&a.num_pages),
                  const_cast<int64_t*>(&a.num_rows)};
  const void* fn =
      a.scalar ? reinterpret_cast<const void*>(
                     &kv_cache_gather_dequant_paged_kernel<kPagedWaves, kPagedRows, true>)
               : reinterpret_cast<const void*>(
                     &kv_cache_gather_dequant_paged_kernel<kPagedWaves, kPagedRows, false>);
  hipError_t err = hipLaunchKernel(
      fn,
      dim3(static_cast<uint32_t>(blocks_x), static_cast<uint32_t>(a.num_seqs)),
      dim3(kPagedWaves * 64), args, 0, stream);
  return err == hipSuccess ? FP8KV_OK : FP8KV_ERR_LAUNCH;
}

int launch_gather_dequant(const DequantArgs& a, hipStream_t stream) {
  // row indices (and grp * RS + RS - 1) fit int32
  if (a.num_rows > 0x7FFFFFFF - kDequantRows) return FP8KV_ERR_SHAPE;
  const int64_t blocks = (static_cast<int64_t>(a.num_rows) + kDequantRows - 1) /
                         kDequantRows;
  void* args[] = {const_cast<const uint8_t**>(&a.kv_cache),
                  const_cast<const uint8_t**>(&a.kv_scale),
                  const_cast<const float**>(&a.scalar_scale),
                  const_cast<const int64_t**>(&a.slots),
                  const_cast<uint16_t**>(&a.out),
                  const_cast<int32_t*>(&a.num_rows),
                  const_cast<int64_t*>(&a.num_cache_slots)};
  const void* fn =
      a.scalar
          ? reinterpret_cast<const void*>(
                &kv_cache_gather_dequant_kernel<kDequantRows, true>)
          : reinterpret_cast<const void*>(
                &kv_cache_gather_dequant_kernel<kDequantRows, false>);
  hipError_t err = hipLaunchKernel(fn, dim3(static_cast<uint32_t>(blocks)),
                                   dim3(64), args, 0, stream);
  return err == hipSuccess ? FP8KV_OK : FP8KV_ERR_LAUNCH;
}

}  // namespace fp8kv
