// Quantise one normalised, rotated KV head held as 8 fp32 values per lane of
// a 64-lane wave (lane l holds dims 8l..8l+7) and write its paged-cache row:
// seven UE8M0 power-of-two block exponents over dims 0..447 (block b = lanes
// 8b..8b+7), FP8 E4M3 codes of y * 2^-e, and dims 448..511 as bf16 (the cache
// layout of FlagGems PR #5449 "Performance": an exponent for each of a
// token's seven blocks).  Shared by the fused prologue and the stand-alone quantise+insert.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "wave_ops.hpp"

namespace fp8kv {

// Smallest e with amax <= 448 * 2^e, clamped to [-127, 127]; 0 -> -127.
// Exact: amax = m 2^k with m in [0.5, 1) and 448 = 0.875 2^9.
__device__ __forceinline__ int ue8m0_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  const int k = __builtin_amdgcn_frexp_expf(amax);
  const float m = __builtin_amdgcn_frexp_mantf(amax);
  int e = k - 9 + (m > 0.875f ? 1 : 0);
  e = e < -127 ? -127 : e;
  return e > 127 ? 127 : e;
}

// Every lane of the wave must be active (the block maximum is a DPP step).
// row = the 576-byte cache row, scale = its 8-byte exponent row (byte 7 is
// left untouched).
__device__ __forceinline__ void quantise_store_row(const float* y, int lane,
                                                   uint8_t* row, uint8_t* scale) {
  constexpr int kRopeLane0 = 56;  // first lane holding a rotary dim
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(y[j]));
  amax = group8_max(amax);
  const int e = ue8m0_exponent(amax);
  if (lane < kRopeLane0) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_ldexpf(y[j], -e);  // exact
    uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo, true);
    uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], hi, true);
    __builtin_nontemporal_store(u32x2_t{lo, hi},
                                reinterpret_cast<u32x2_t*>(row + lane * 8));
    if ((lane & 7) == 0) scale[lane >> 3] = static_cast<uint8_t>(e + 127);
  } else {
    u32x4_t o = {pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]),
                 pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7])};
    store16<true>(row + 448 + (lane - kRopeLane0) * 16, o);
  }
}

// The scalar-scale convention (one kv_cache_scale float for the whole cache,
// FlagGems PR #5449 "Performance"): codes of y / scale, saturated to the
// E4M3 range; dims 448..511 as bf16; no exponent bytes.  No cross-lane work.
__device__ __forceinline__ void quantise_store_row_scalar(const float* y, int lane,
                                                          uint8_t* row,
                                                          float scale) {
  constexpr int kRopeLane0 = 56;
  if (lane < kRopeLane0) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = fminf(fmaxf(y[j] / scale, -448.0f), 448.0f);
    uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo, true);
    uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], hi, true);
    __builtin_nontemporal_store(u32x2_t{lo, hi},
                                reinterpret_cast<u32x2_t*>(row + lane * 8));
  } else {
    u32x4_t o = {pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]),
                 pack_bf16(y[4], y[5]), pack_bf16(y[6], y[7])};
    store16<true>(row + 448 + (lane - kRopeLane0) * 16, o);
  }
}

}  // namespace fp8kv
