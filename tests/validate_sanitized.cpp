// Host-only driver for the argument checks, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (no HIP, no GPU): every check is called with
// extreme arguments (the int32 and int64 limits, negatives, zero, misaligned
// and null pointers) and must return the expected status without undefined
// behaviour (signed overflow, division by zero, shifts).  Prints "ok" and
// exits 0, or names the failing case and exits 1.
#include <cstdint>
#include <cstdio>
#include <limits>
#include <vector>

#include "validate.hpp"

namespace {

int failures = 0;

void expect(int got, int want, const char* what, long long a, long long b) {
  if (got != want) {
    std::printf("FAIL %s (%lld, %lld): got %d want %d\n", what, a, b, got, want);
    ++failures;
  }
}

}  // namespace

int main() {
  using namespace fp8kv;
  constexpr int32_t kI32Max = std::numeric_limits<int32_t>::max();
  constexpr int32_t kI32Min = std::numeric_limits<int32_t>::min();
  constexpr int64_t kI64Max = std::numeric_limits<int64_t>::max();
  constexpr int64_t kI64Min = std::numeric_limits<int64_t>::min();
  void* p = reinterpret_cast<void*>(uintptr_t{1} << 20);  // aligned, never dereferenced
  void* odd = reinterpret_cast<void*>((uintptr_t{1} << 20) + 2);
  const float* fp = static_cast<const float*>(p);
  const int64_t* ip = static_cast<const int64_t*>(p);
  const int32_t* i32p = static_cast<const int32_t*>(p);
  const uint8_t* bp = static_cast<const uint8_t*>(p);
  uint8_t* wbp = static_cast<uint8_t*>(p);

  const std::vector<int64_t> i64s = {kI64Min, -1, 0, 1, 7, 1 << 20, kI32Max, int64_t{1} << 40,
                                     kI64Max};
  const std::vector<int32_t> i32s = {kI32Min, -1, 0, 1, 12, 64, 1 << 20, kI32Max};

  // Every check on every combination of extreme sizes: any undefined
  // behaviour aborts the process under the sanitizers.
  for (int64_t t : i64s) {
    for (int32_t h : i32s) {
      (void)validate_prologue(p, p, p, p, fp, ip, ip, bp, bp, t, h, 512, 64, t, t, 64);
      (void)validate_packed(p, t, h, h, h, 128, p, p, fp, 1, ip, -1, t);
      (void)validate_packed(p, t, h, kI32Max, kI32Max, 128, p, p, fp, 1, ip, -1, t);
      (void)validate_packed_ex(p, t, h, h, h, 256, p, p, fp, 1, ip, 256, 0, t);
      (void)validate_packed_ex(p, t, kI32Max, h, kI32Max, 64, p, p, fp, 0, ip, 64, 1, t);
      (void)validate_gather_dequant(bp, bp, t, 64, ip, t, p);
      (void)validate_gather_dequant_paged(bp, bp, t, 64, i32p, h, h, i32p, ip, t, p);
      (void)validate_rms_norm_rows(p, p, p, t, 512);
      (void)validate_rope_rows(p, fp, ip, t, h, 512, 64, t);
      (void)validate_heads(t, h, 128);
      (void)validate_rms_norm_heads(p, t, p, p, t, h, 128);
      (void)validate_rms_norm_heads(p, kI64Max, p, p, t, h, 128);
      (void)validate_rope_neox_heads(p, fp, ip, t, h, 128, t);
      (void)validate_kv_quant_insert(p, ip, bp, bp, t, t, 64);
    }
  }

  // Expected statuses at the limits.
  expect(validate_packed(p, 1, kI32Max, kI32Max, 0, 128, p, p, fp, 1, ip, -1, 8),
         FP8KV_ERR_SHAPE, "packed: Hq + Hk overflows int32", kI32Max, kI32Max);
  expect(validate_packed(p, 1, kI32Max, 1, 0, 128, p, p, fp, 1, ip, -1, 8),
         FP8KV_ERR_SHAPE, "packed: heads past 2^20", kI32Max, 1);
  expect(validate_packed(p, 1, 0, 0, 0, 128, p, p, fp, 1, ip, -1, 8), FP8KV_ERR_SHAPE,
         "packed: no Q/K head", 0, 0);
  expect(validate_packed(p, kI64Max, 1, 1, 0, 128, p, p, fp, 1, ip, -1, 8), FP8KV_ERR_SHAPE,
         "packed: tokens x heads past 2^31", kI64Max, 2);
  expect(validate_packed(p, 4, 2, 2, 0, 128, p, p, fp, 1, ip, -1, 8), FP8KV_OK,
         "packed: plain call", 4, 4);
  expect(validate_packed_ex(p, 1, kI32Max, kI32Max, 0, 64, p, p, fp, 1, ip, 64, 0, 8),
         FP8KV_ERR_SHAPE, "packed_ex: Hq + Hk overflows int32", kI32Max, kI32Max);
  expect(validate_packed_ex(p, 1, 1 << 21, 1 << 21, 1 << 21, 256, p, p, fp, 1, ip, 256, 0, 8),
         FP8KV_ERR_SHAPE, "packed_ex: row past 2^30 elements", 3 << 21, 256);
  expect(validate_packed_ex(p, 1, 1 << 20, 1 << 20, 1 << 20, 256, p, p, fp, 1, ip, 256, 0, 8),
         FP8KV_OK, "packed_ex: row of 3 * 2^28 elements", 3 << 20, 256);
  expect(validate_packed_ex(p, 3, 2, 2, 1, 64, p, p, nullptr, 0, ip, 0, 1, 0), FP8KV_OK,
         "packed_ex: no rotary dims, empty table", 3, 0);
  expect(validate_prologue(p, p, p, p, fp, ip, ip, bp, bp, kI64Max, kI32Max, 512, 64, 8, 8, 64),
         FP8KV_ERR_SHAPE, "prologue: tokens x (heads + 1) past 2^31", kI64Max, kI32Max);
  expect(validate_prologue(odd, p, p, p, fp, ip, ip, bp, bp, 1, 1, 512, 64, 8, 8, 64),
         FP8KV_ERR_ALIGN, "prologue: misaligned q", 1, 1);
  expect(validate_prologue(p, p, p, p, fp, ip, ip, nullptr, nullptr, 1, 1, 512, 64, 8, 0, 64),
         FP8KV_OK, "prologue: cache without pages", 1, 0);
  expect(validate_rope_rows(p, fp, ip, kI64Max, 1, 512, 64, 8), FP8KV_ERR_SHAPE,
         "rope_rows: tokens past 2^40", kI64Max, 1);
  expect(validate_heads(kI64Max, kI32Max, 128), FP8KV_ERR_SHAPE, "heads: product", kI64Max,
         kI32Max);
  expect(validate_rms_norm_heads(p, kI64Max, p, p, 2, 2, 128), FP8KV_ERR_SHAPE,
         "rms_norm_heads: stride past 2^40", kI64Max, 2);
  expect(validate_gather_dequant_paged(bp, bp, 4, 64, i32p, 65536, 1, i32p, ip, 1, p),
         FP8KV_ERR_SHAPE, "paged: sequences past 65535", 65536, 1);
  expect(validate_kv_quant_insert(p, ip, wbp, wbp, int64_t{1} << 31, 1, 64), FP8KV_ERR_SHAPE,
         "kv_quant_insert: tokens past 2^31 - 1", int64_t{1} << 31, 1);
  expect(valid_eps(std::numeric_limits<float>::quiet_NaN()) ? 1 : 0, 0, "eps NaN", 0, 0);
  expect(valid_eps(std::numeric_limits<float>::infinity()) ? 1 : 0, 0, "eps inf", 0, 0);
  expect(valid_eps(0.0f) ? 1 : 0, 1, "eps 0", 0, 0);

  if (failures) return 1;
  std::printf("ok\n");
  return 0;
}
