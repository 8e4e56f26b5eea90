// Wave64 building blocks for gfx950 (CDNA4): cross-lane reductions on DPP and
// v_readlane, bf16 unpack/pack and 16-byte memory access.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fp8kv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// Four dwords at an address that is only known to be 8-byte aligned (gfx950
// global loads do not need the vector's natural 16-byte alignment).
typedef uint32_t u32x4_a8_t __attribute__((ext_vector_type(4), aligned(8)));

// DPP lane patterns (GCN/CDNA encoding).  All reductions below run with every
// lane of the wave active.
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i within 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i within 16 lanes
constexpr int kDppRowRor8 = 0x128;        // lane i <- (i+8) mod 16 within a row

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                         0xF, 0xF, false));
}

// Sum over each 16-lane row; every lane of the row receives the row's sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppRowHalfMirror>(v);
  v += dpp<kDppRowMirror>(v);
  return v;
}

// Sum over the whole wave; every lane receives the same (wave-uniform)
// value.  After the row sums, the four row totals are read from lanes 0, 16,
// 32 and 48.  (The gfx950 permlane swaps would do this in VALU registers, but
// hipcc of ROCm 7.2 folds the second result of v_permlane16/32_swap into the
// first when both operands are the same value, so they are not used.)
__device__ __forceinline__ float wave64_sum(float v) {
  v = row16_sum(v);
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

// Maximum over each group of 8 consecutive lanes.
__device__ __forceinline__ float group8_max(float v) {
  v = fmaxf(v, dpp<kDppQuadXor1>(v));
  v = fmaxf(v, dpp<kDppQuadXor2>(v));
  v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
  return v;
}

// bf16 pair (low half = element 0) to two floats, exactly.
__device__ __forceinline__ float bf16_lo(uint32_t u) {
  return __builtin_bit_cast(float, u << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t u) {
  return __builtin_bit_cast(float, u & 0xFFFF0000u);
}

// Two floats to a bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  float2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Sum of squares of 8 values (fp32 fused multiply-adds).
__device__ __forceinline__ float sum_sq8(const float* f) {
  float acc = f[0] * f[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) acc = fmaf(f[j], f[j], acc);
  return acc;
}

__device__ __forceinline__ void unpack8(u32x4_t x, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(x[i]);
    f[2 * i + 1] = bf16_hi(x[i]);
  }
}

template <bool NT>
__device__ __forceinline__ u32x4_t load16(const void* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  else
    return *static_cast<const u32x4_t*>(p);
}

template <bool NT>
__device__ __forceinline__ void store16(void* p, u32x4_t v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, static_cast<u32x4_t*>(p));
  else
    *static_cast<u32x4_t*>(p) = v;
}

// Non-temporal 16-byte store with device scope (gfx950 cache policy "nt sc1"),
// for the streams that write each line once.  The compiler's non-temporal
// store builtin sets only "nt", and no builtin reaches the scope bits of a
// global store, hence the asm (a vector store: no result, so nothing waits
// on it; the "memory" clobber keeps its place among the other memory
// operations).  The hardware reads a 16-byte store's data registers after
// the store issues, so a VALU write to them must come some wait states later.
// The compiler inserts those after its own stores (two, here), but it cannot
// see a store inside an asm statement: without the s_nop a kernel with
// several stores per wave overwrote a store's data before it was read (a
// seeded packed case stored wrong values).  The s_nop 4 gives five wait
// states in the same statement.  Measured on MI355X against "nt" alone, each
// launch after a cache-flushing read, two runs: the prologue 673.3 -> 657.3-
// 658.4 us at 32768 x 64 and 2703 -> 2635 us at 131072 x 64 (2.3-3.6% faster
// from 1024 tokens up), the read sides 1-2%, the packed op 0.3-1.3% and its
// variants 1.3-5% faster, the in-place RMW and copy references 1.1-1.2%
// faster; "nt sc0 sc1" measured the same as "nt sc1", "nt sc0" the same as
// "nt", and "sc1" without "nt" was mixed.  The prologue's KV row stores (8-byte codes, 16-byte rotary
// part) measured 0.5-1% slower with it and keep "nt"; so do the separate-
// launch baselines, which were 2-5% slower with it.
__device__ __forceinline__ void store16_nt_sc1(void* p, u32x4_t v) {
  __asm__ volatile("global_store_dwordx4 %0, %1, off nt sc1\n\ts_nop 4"
                   : : "v"(p), "v"(v) : "memory");
}

__device__ __forceinline__ f32x4_t load16f(const float* p) {
  return *reinterpret_cast<const f32x4_t*>(p);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

}  // namespace fp8kv
