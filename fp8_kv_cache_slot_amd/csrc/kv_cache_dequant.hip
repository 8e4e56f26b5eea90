// Read side of the paged FP8/UE8M0 KV cache for gfx950: gather rows by slot
// and dequantise them to bf16, the inverse of the fused prologue's insert
// (the cache layout of FlagGems PR #5449 "Performance": FP8 codes with seven
// per-block power-of-two exponents per token).
//
//   out[i, d]       = E4M3(code[s, d]) * 2^(scale[s, d / 64] - 127), d < 448
//   out[i, 448 + j] = stored bf16 rotary value j
//
// Layout of the work.  One 64-lane wave per output row (1 KiB of bf16 = one
// 16-byte vector per lane, as in the prologue).  Lane l < 56 reads the 8 code
// bytes of dims 8l..8l+7 (one 8-byte load) and the row's 8-byte scale word
// (one address for the whole wave), decodes with v_cvt_pk_f32_fp8, scales
// exactly with v_ldexp and packs with v_cvt_pk_bf16_f32; lanes 56..63 move the
// 128 stored rotary bytes unchanged.  Each wave gathers RS rows and issues all
// of their loads before any arithmetic.  The output is written non-temporally.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "prologue_launch.hpp"
#include "wave_ops.hpp"

namespace fp8kv {
namespace {

constexpr int kRopeLane0 = 56;

// SCALAR: the scalar-scale convention, out = E4M3(code) * scalar_scale[0]
// (rounded once to fp32, then to bf16) and no exponent bytes are read.
template <int WAVES, int RS, bool SCALAR>
__global__ void __launch_bounds__(WAVES * 64) kv_cache_gather_dequant_kernel(
    const uint8_t* __restrict__ kv_cache, const uint8_t* __restrict__ kv_scale,
    const float* __restrict__ scalar_scale, const int64_t* __restrict__ slots,
    uint16_t* __restrict__ out, int32_t num_rows, int64_t num_cache_slots) {
  const int lane = lane_id();
  const int32_t first = (static_cast<int32_t>(blockIdx.x) * WAVES + wave_id()) * RS;
  if (first >= num_rows) return;

  int64_t slot[RS];
  bool ok[RS];
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    const int32_t i = first + r < num_rows ? first + r : num_rows - 1;
    slot[r] = slots[i];
    ok[r] = first + r < num_rows && slot[r] >= 0 && slot[r] < num_cache_slots;
  }
  u32x2_t codes[RS], sc[RS];
  u32x4_t rope[RS];
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    codes[r] = u32x2_t{0u, 0u};
    sc[r] = u32x2_t{0u, 0u};
    rope[r] = u32x4_t{0u, 0u, 0u, 0u};
    if (ok[r]) {
      const uint8_t* row = kv_cache + slot[r] * 576;
      if constexpr (!SCALAR)
        sc[r] = *reinterpret_cast<const u32x2_t*>(kv_scale + slot[r] * 8);
      if (lane < kRopeLane0)
        codes[r] = *reinterpret_cast<const u32x2_t*>(row + lane * 8);
      else
        rope[r] = *reinterpret_cast<const u32x4_t*>(row + 448 + (lane - kRopeLane0) * 16);
    }
  }

  const int b = lane >> 3;  // quantisation block of this lane's dims
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    if (first + r >= num_rows) break;
    uint16_t* dst = out + static_cast<int64_t>(first + r) * 512 + lane * 8;
    u32x4_t o = {0u, 0u, 0u, 0u};
    if (ok[r]) {
      if (lane < kRopeLane0) {
        // a valid slot exists only when the cache has pages, and then the
        // scalar scale pointer is a checked device pointer
        float fs = 1.0f;
        if constexpr (SCALAR) fs = *scalar_scale;
        const uint32_t word = b < 4 ? sc[r][0] : sc[r][1];
        const int e = static_cast<int>((word >> (8 * (b & 3))) & 0xFFu) - 127;
        const int lo = static_cast<int>(codes[r][0]);
        const int hi = static_cast<int>(codes[r][1]);
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
        o = u32x4_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]),
                    pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
      } else {
        o = rope[r];
      }
    }
    store16<true>(dst, o);
  }
}

constexpr int kDequantWaves = 4;
constexpr int kDequantRows = 2;

}  // namespace

int launch_gather_dequant(const DequantArgs& a, hipStream_t stream) {
  const int64_t rows_per_block = static_cast<int64_t>(kDequantWaves) * kDequantRows;
  const int64_t blocks = (static_cast<int64_t>(a.num_rows) + rows_per_block - 1) /
                         rows_per_block;
  if (blocks > 0x7FFFFFFF) return FP8KV_ERR_SHAPE;
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
                &kv_cache_gather_dequant_kernel<kDequantWaves, kDequantRows, true>)
          : reinterpret_cast<const void*>(
                &kv_cache_gather_dequant_kernel<kDequantWaves, kDequantRows, false>);
  hipError_t err = hipLaunchKernel(fn,
      dim3(static_cast<uint32_t>(blocks)), dim3(kDequantWaves * 64), args, 0,
      stream);
  return err == hipSuccess ? FP8KV_OK : FP8KV_ERR_LAUNCH;
}

}  // namespace fp8kv
