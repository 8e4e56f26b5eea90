// Host-only driver for the CPU oracle, built with AddressSanitizer and
// UndefinedBehaviorSanitizer together with oracle/oracle.cpp: every entry is
// called on small random inputs held in buffers of exactly the documented
// size (so a read or write past an end is caught), with the edge cases the
// entries document (skipped and out-of-range slots, invalid pages, lengths
// past the table, rows past the output, partial rotary, zero rotary, both
// pairings, both dtypes), and every number-format routine over its whole
// input range.  Prints "ok" and exits 0; undefined behaviour aborts.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "oracle.h"

namespace {

std::mt19937_64 rng(12345);

uint16_t rand_bf16() {
  std::normal_distribution<double> n(0.0, 2.0);
  return oracle_bf16_rne(n(rng));
}

std::vector<uint16_t> bf16s(size_t n) {
  std::vector<uint16_t> v(n);
  for (auto& x : v) x = rand_bf16();
  return v;
}

std::vector<uint16_t> weights(size_t n, bool fp16 = false) {
  std::uniform_real_distribution<double> u(0.5, 1.5);
  std::vector<uint16_t> v(n);
  for (auto& x : v) x = fp16 ? oracle_fp16_rne(u(rng)) : oracle_bf16_rne(u(rng));
  return v;
}

std::vector<float> cos_sin(int64_t rows, int r) {
  std::vector<float> v(static_cast<size_t>(rows) * r);
  for (int64_t p = 0; p < rows; ++p)
    for (int i = 0; i < r / 2; ++i) {
      const double a = p * std::pow(10000.0, -2.0 * i / r);
      v[p * r + i] = static_cast<float>(std::cos(a));
      v[p * r + r / 2 + i] = static_cast<float>(std::sin(a));
    }
  return v;
}

int failures = 0;
void check(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAIL %s\n", what);
    ++failures;
  }
}

}  // namespace

int main() {
  // number formats over their whole input ranges
  for (uint32_t b = 0; b < 65536; ++b) {
    const double v = oracle_bf16_to_double(static_cast<uint16_t>(b));
    if (std::isfinite(v)) check(oracle_bf16_rne(v) == b || v == 0.0, "bf16 round trip");
    const double h = oracle_fp16_to_double(static_cast<uint16_t>(b));
    if (std::isfinite(h)) check(oracle_fp16_rne(h) == b || h == 0.0, "fp16 round trip");
  }
  for (uint32_t c = 0; c < 256; ++c) {
    const double v = oracle_e4m3_decode(static_cast<uint8_t>(c));
    if (!std::isnan(v)) check(oracle_e4m3_encode(v) == c, "e4m3 round trip");
  }
  for (double v : {0.0, -0.0, 1e-300, -1e-300, 1e-45, 448.0, 449.0, 464.0, -1e300, 1e300})
    (void)oracle_e4m3_encode(v);
  for (double a : {0.0, 1e-320, 1e-300, 4.9e-324, 448.0 * std::ldexp(1.0, -127), 1.0, 448.0,
                   1e38, 1e300}) {
    const int32_t e = oracle_ue8m0_exponent(a);
    check(e >= -127 && e <= 127, "ue8m0 range");
  }

  // the prologue: 5 tokens, 3 heads, one page; slots valid, -1 and past the page
  {
    const int64_t T = 5, pages = 1, P = 16;
    const int32_t H = 3;
    auto q = bf16s(T * H * 512), kv = bf16s(T * 512), qw = weights(512), kw = weights(512);
    auto cs = cos_sin(P, 64);
    std::vector<int64_t> pos = {0, 3, 15, 7, 1}, slot = {0, 63, -1, 64, 5};
    std::vector<uint8_t> cache(pages * 64 * 576, 0xA5), scale(pages * 64 * 8, 0x5A);
    oracle_qnorm_rope_kv_quant_insert(q.data(), kv.data(), qw.data(), kw.data(), cs.data(),
                                      pos.data(), slot.data(), cache.data(), scale.data(), T,
                                      H, pages, 1e-6);
    oracle_qnorm_rope_kv_quant_insert_scalar(q.data(), kv.data(), qw.data(), kw.data(),
                                             cs.data(), pos.data(), slot.data(), cache.data(),
                                             0.03125f, T, H, pages, 1e-6);
    std::vector<double> y(T * 512);
    oracle_kv_normalised(kv.data(), kw.data(), cs.data(), pos.data(), T, 1e-6, y.data());
    // no pages at all: nothing is written
    oracle_qnorm_rope_kv_quant_insert(q.data(), kv.data(), qw.data(), kw.data(), cs.data(),
                                      pos.data(), slot.data(), nullptr, nullptr, T, H, 0, 0.0);
    // the separate stages
    std::vector<uint16_t> rows(T * H * 512);
    oracle_rms_norm_rows(q.data(), qw.data(), rows.data(), T * H, 1e-6);
    oracle_rope_rows(rows.data(), cs.data(), pos.data(), T, H);
    std::vector<uint16_t> kvr(T * 512);
    oracle_rms_norm_rows(kv.data(), kw.data(), kvr.data(), T, 1e-6);
    oracle_kv_quant_insert(kvr.data(), slot.data(), cache.data(), scale.data(), T, pages);
    // read side by slot list and through block tables
    std::vector<int64_t> slots = {0, 63, -5, 64, 1 << 20, 5};
    std::vector<uint16_t> out(slots.size() * 512);
    oracle_kv_cache_gather_dequant(cache.data(), scale.data(), slots.data(),
                                   static_cast<int64_t>(slots.size()), pages, out.data());
    oracle_kv_cache_gather_dequant_scalar(cache.data(), 0.5f, slots.data(),
                                          static_cast<int64_t>(slots.size()), pages,
                                          out.data());
    const int32_t S = 3, MB = 2;
    std::vector<int32_t> table = {0, -1, 7, 0, 0, 0}, lens = {70, 200, 5};
    std::vector<int64_t> offs = {0, 60, -3};
    const int64_t NR = 150;
    std::vector<uint16_t> pout(NR * 512);
    oracle_kv_cache_gather_dequant_paged(cache.data(), scale.data(), pages, table.data(), S, MB,
                                         lens.data(), offs.data(), NR, pout.data());
    oracle_kv_cache_gather_dequant_paged_scalar(cache.data(), 2.0f, pages, table.data(), S, MB,
                                                lens.data(), offs.data(), NR, pout.data());
  }

  // the packed operator and its separate stages
  for (int D : {64, 128, 256}) {
    for (int R : {0, 16, D / 2, D}) {
      for (int neox = 0; neox < 2; ++neox) {
        for (int fp16 = 0; fp16 < 2; ++fp16) {
          const int64_t T = 7;
          const int32_t hq = 3, hk = 2, hv = 1;
          std::vector<uint16_t> qkv(T * (hq + hk + hv) * D);
          for (auto& x : qkv) x = fp16 ? oracle_fp16_rne(oracle_bf16_to_double(rand_bf16()))
                                       : rand_bf16();
          auto qw = weights(D, fp16), kw = weights(D, fp16);
          auto cs = cos_sin(9, R > 0 ? R : 2);
          std::vector<int64_t> pos = {0, 8, 3, 3, 1, 7, 2};
          oracle_qk_norm_rope_packed_ex(qkv.data(), T, hq, hk, hv, D, R, neox, fp16, 1e-6,
                                        qw.data(), kw.data(), R > 0 ? cs.data() : nullptr,
                                        pos.data());
          if (D == 128 && R == 128 && neox && !fp16)
            oracle_qk_norm_rope_packed(qkv.data(), T, hq, hk, hv, D, 1e-6, qw.data(),
                                       kw.data(), cs.data(), pos.data());
          if (R == D && neox && !fp16) {
            std::vector<uint16_t> heads(T * hk * D);
            oracle_rms_norm_heads(qkv.data() + hq * D, (hq + hk + hv) * D, kw.data(),
                                  heads.data(), T, hk, D, 1e-6);
            oracle_rope_neox_heads(heads.data(), cs.data(), pos.data(), T, hk, D);
          }
        }
      }
    }
  }
  if (failures) return 1;
  std::printf("ok\n");
  return 0;
}
