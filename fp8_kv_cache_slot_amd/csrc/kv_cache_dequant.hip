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

// One group of RS rows as loaded.  Each lane issues one 16-byte load per
// row: lane l < 56 reads bytes 8l..8l+15 of the row and keeps the low 8 (its
// codes; lane 55 ends at byte 455, inside the 576-byte row), lanes 56..63
// read the rotary vector 448 + 16 (l - 56).  The row's 8 exponent bytes are
// one wave-uniform (scalar) load.  A row whose slot is invalid reads slot 0
// (the cache has pages here) and is stored as zeros.
//
// All of a group's loads are issued before anything waits on them or
// branches: the empty asm statements below take the loaded registers as
// operands, so hipcc cannot sink a row's loads below the per-row store
// conditions (it did, and then each row waited for its own round trip).
template <int RS>
struct Rows {
  u32x4_t v[RS];
  uint64_t ev[RS];
};

__device__ __forceinline__ bool slot_valid(int64_t s, int64_t num_cache_slots) {
  return s >= 0 && s < num_cache_slots;
}

__device__ __forceinline__ int row_offset(int lane) {
  return lane < kRopeLane0 ? lane * 8 : 448 + (lane - kRopeLane0) * 16;
}

// Rows at slots s[0..RS), each already in [0, num_cache_slots).
template <int RS, bool SCALAR>
__device__ __forceinline__ void load_rows(const uint8_t* __restrict__ kv_cache,
                                          const uint8_t* __restrict__ kv_scale,
                                          const int64_t* slot, int lane,
                                          Rows<RS>& d) {
  const int off = row_offset(lane);
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    // lane l < 56 reads bytes 8l..8l+15 of the row: 8-byte aligned only
    d.v[r] = *reinterpret_cast<const u32x4_a8_t*>(kv_cache + slot[r] * 576 + off);
    d.ev[r] = SCALAR ? 0u : *reinterpret_cast<const uint64_t*>(kv_scale + slot[r] * 8);
  }
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    if constexpr (SCALAR)
      __asm__ volatile("" : "+v"(d.v[r]));
    else
      __asm__ volatile("" : "+v"(d.v[r]), "+s"(d.ev[r]));
  }
}

// Output vector of row r for this lane: decoded codes (lanes < 56) or the
// stored rotary vector; fs is the scalar scale (SCALAR) or unused.
template <bool SCALAR>
__device__ __forceinline__ u32x4_t dequant_vector(u32x4_t v, uint64_t ev, float fs,
                                                  int lane) {
  const int sh = (lane >> 3) * 8;  // exponent byte of block l >> 3
  const uint32_t w = sh < 32 ? static_cast<uint32_t>(ev) : static_cast<uint32_t>(ev >> 32);
  const int e = static_cast<int>((w >> (sh & 31)) & 0xFFu) - 127;
  const int lo = static_cast<int>(v[0]);
  const int hi = static_cast<int>(v[1]);
  const float2_t p[4] = {__builtin_amdgcn_cvt_pk_f32_fp8(lo, false),
                         __builtin_amdgcn_cvt_pk_f32_fp8(lo, true),
                         __builtin_amdgcn_cvt_pk_f32_fp8(hi, false),
                         __builtin_amdgcn_cvt_pk_f32_fp8(hi, true)};
  float f[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (SCALAR) {
      f[2 * k] = p[k][0] * fs;
      f[2 * k + 1] = p[k][1] * fs;
    } else {
      f[2 * k] = __builtin_ldexpf(p[k][0], e);
      f[2 * k + 1] = __builtin_ldexpf(p[k][1], e);
    }
  }
  const u32x4_t q = {pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]),
                     pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7])};
  return lane < kRopeLane0 ? q : v;
}

// SCALAR: the scalar-scale convention, out = E4M3(code) * scalar_scale[0]
// (rounded once to fp32, then to bf16) and no exponent bytes are read.
//
// The gather is a chain of two dependent loads: the slots, then the rows.
// Each one-wave block takes one group of RS consecutive rows: the RS slot
// indices are wave-uniform (scalar loads), then every lane issues the group's
// row loads, and the rows are dequantised and stored.  Many small one-shot
// blocks keep enough groups in flight to hide the two round trips.  Measured
// on MI355X over all 131072 slots of a 2048-page cache in random order,
// caches cold and clean: 40.0 us with 2 rows per one-wave block, against
// 41.0 with 4 and 41.7 with 8; a plain streaming kernel with the same bytes
// per row (576 read, 1024 written, contiguous rows, no arithmetic) takes
// 40.1 us.  The form before (three loads per row: codes, rotary vector and
// exponent byte, some sunk below the store conditions) took 42.0 us, and a
// persistent form with the next group's loads in flight 43.9 us.
template <int RS, bool SCALAR>
__global__ void __launch_bounds__(64) kv_cache_gather_dequant_kernel(
    const uint8_t* __restrict__ kv_cache, const uint8_t* __restrict__ kv_scale,
    const float* __restrict__ scalar_scale, const int64_t* __restrict__ slots,
    uint16_t* __restrict__ out, int32_t num_rows, int64_t num_cache_slots) {
  const int lane = lane_id();
  const int32_t grp = static_cast<int32_t>(blockIdx.x);
  if (grp * RS >= num_rows) return;
  const u32x4_t z = {0u, 0u, 0u, 0u};
  if (num_cache_slots <= 0) {  // a cache without pages: every row is zero
#pragma unroll
    for (int r = 0; r < RS; ++r) {
      const int32_t i = grp * RS + r;
      if (i < num_rows) store16_nt_sc1(out + static_cast<int64_t>(i) * 512 + lane * 8, z);
    }
    return;
  }
  // Rows past the last one re-read the last slot (in bounds) and are not
  // stored.
  int64_t s[RS], slot[RS];
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    int32_t i = grp * RS + r;
    if (i > num_rows - 1) i = num_rows - 1;
    s[r] = slots[i];
  }
  // all slot loads in flight together
#pragma unroll
  for (int r = 0; r < RS; ++r) __asm__ volatile("" : "+s"(s[r]));
#pragma unroll
  for (int r = 0; r < RS; ++r) slot[r] = slot_valid(s[r], num_cache_slots) ? s[r] : 0;
  // with pages, the scalar scale pointer is a checked device pointer
  float fs = 1.0f;
  if constexpr (SCALAR) fs = *scalar_scale;
  Rows<RS> d;
  load_rows<RS, SCALAR>(kv_cache, kv_scale, slot, lane, d);
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    const int32_t i = grp * RS + r;
    if (i >= num_rows) break;
    const u32x4_t o = slot_valid(s[r], num_cache_slots)
                          ? dequant_vector<SCALAR>(d.v[r], d.ev[r], fs, lane)
                          : z;
    store16_nt_sc1(out + static_cast<int64_t>(i) * 512 + lane * 8, o);
  }
}

constexpr int kDequantRows = 2;

// The read side through block tables, as an attention consumer indexes the
// cache: token j of sequence s sits in slot
// block_table[s, j / 64] * 64 + j % 64 and its row goes to
// out[out_offsets[s] + j].  Grid: x = groups of PRS consecutive tokens of a
// sequence (covering max_blocks_per_seq pages), y = sequence.  PRS divides 64,
// so a wave's rows are consecutive slots of one page (PRS * 576 contiguous
// bytes, and PRS * 8 contiguous exponent bytes).  The page id, length and
// output offset are three independent scalar loads, all issued before the
// wave branches on the length; the row loads follow (an invalid page reads
// slots 0.. and stores zero rows, as in the slot-list kernel), and only the
// stores depend on the length and the output bounds.
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
  int32_t page = block_table[static_cast<int64_t>(seq) * max_blocks_per_seq + j0 / 64];
  int32_t len = seq_lens[seq];
  int64_t first = out_offsets[seq];
  // all three loads in flight together (hipcc otherwise waits for the length
  // and branches before it asks for the other two)
  __asm__ volatile("" : "+s"(page), "+s"(len), "+s"(first));
  first += j0;
  if (j0 >= len) return;

  const u32x4_t z = {0u, 0u, 0u, 0u};
  if (num_pages <= 0) {  // a cache without pages: every row is zero
#pragma unroll
    for (int r = 0; r < PRS; ++r) {
      const int64_t i = first + r;
      if (j0 + r < len && i >= 0 && i < num_rows)
        store16_nt_sc1(out + i * 512 + lane * 8, z);
    }
    return;
  }
  const bool page_ok = page >= 0 && page < num_pages;
  const int64_t slot0 = page_ok ? static_cast<int64_t>(page) * 64 + j0 % 64 : 0;
  int64_t slot[PRS];
#pragma unroll
  for (int r = 0; r < PRS; ++r) slot[r] = slot0 + r;
  // with pages, the scalar scale pointer is a checked device pointer
  float fs = 1.0f;
  if constexpr (SCALAR) fs = *scalar_scale;
  Rows<PRS> d;
  load_rows<PRS, SCALAR>(kv_cache, kv_scale, slot, lane, d);
#pragma unroll
  for (int r = 0; r < PRS; ++r) {
    const int64_t i = first + r;
    if (j0 + r >= len || i < 0 || i >= num_rows) continue;
    const u32x4_t o = page_ok ? dequant_vector<SCALAR>(d.v[r], d.ev[r], fs, lane) : z;
    store16_nt_sc1(out + i * 512 + lane * 8, o);
  }
}

// One wave of 2 rows per block.  Measured on MI355X over all 2048 pages of a
// cache in a random page order, caches cold and clean: 40.3 us for 32 x 4096
// and 39.9 us for 256 x 512 tokens, against 40.6 for 1 x 4 and 2 x 4, 40.5-
// 40.7 for 4 x 4, 41.0-41.2 for 1 x 8 and 2 x 8 (waves x rows per wave); the
// form before (three loads per row, the length waited for before the page id
// was asked for) took 42.4 and 42.9 us.
constexpr int kPagedWaves = 1;
constexpr int kPagedRows = 2;

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
