// CPU oracle: TEST INFRASTRUCTURE ONLY (see oracle.h for the sources cited
// as [P1], [P2], [P3] and for who may load this library).
//
// Everything is computed in double; the only roundings are the ones that
// produce a stored output (bf16 for q and for the rotary part of the cache,
// E4M3 for the cache codes, an exact integer for the block exponent), and the
// rounding of each quantised element to fp32 on which the quantiser's two
// integer decisions (block exponent and code) are taken.
// No blocking, fusion or reordering: each token, then each head, then each
// element, in the order the operator is described.

#include "oracle.h"

#include <cfenv>
#include <cmath>
#include <cstring>

namespace {

// Geometry of the DeepSeek-V4 prologue.  The head width is fixed by [P1]
// "Correctness" (16744448 q elements at 511 tokens and 64 heads = 512 per
// head) and [P2] "What the optimisation does" (64 threads for 512 elements).
// Rotary width, block width and page size are readings: 64 rotary dims at the
// end of the head, seven 64-dim quantisation blocks over the first 448 dims
// ([P1] "Performance": one exponent per block, seven per token), 64-slot pages.
constexpr int kHeadDim = 512;
constexpr int kRopeDim = 64;
constexpr int kRopeStart = kHeadDim - kRopeDim;  // 448
constexpr int kQuantBlock = 64;
constexpr int kNumBlocks = kRopeStart / kQuantBlock;  // 7
constexpr int kPageSize = 64;
constexpr int kRowBytes = kRopeStart + 2 * kRopeDim;  // 576
constexpr int kScaleBytes = 8;                        // 7 used + 1 reserved
constexpr double kE4M3Max = 448.0;

// Round a double to the nearest multiple of `quantum` (a power of two), ties
// to even.  nearbyint honours the current rounding mode, which is forced to
// round-to-nearest-even around every use.
double round_to_quantum(double v, double quantum) {
  return std::nearbyint(v / quantum) * quantum;
}

struct NearestEven {
  int saved;
  NearestEven() : saved(std::fegetround()) { std::fesetround(FE_TONEAREST); }
  ~NearestEven() { std::fesetround(saved); }
};

// Nearest fp32 value of v, ties to even.
double to_fp32(double v) {
  NearestEven mode;
  return static_cast<double>(static_cast<float>(v));
}

// RMSNorm of one row of n bf16 values with a bf16 weight, all in double:
//   y_d = x_d / sqrt(mean(x^2) + eps) * w_d
// Reading: the mean runs over every element of the head (the rotary dims
// included), eps sits inside the square root and the weight multiplies plainly
// and before any rotation ([P3] "Summary": the paired element enters the
// rotation with its own norm weight).
void rms_norm(const uint16_t* x, const uint16_t* w, int n, double eps,
              double* y) {
  double sum_sq = 0.0;
  for (int d = 0; d < n; ++d) {
    double v = oracle_bf16_to_double(x[d]);
    sum_sq += v * v;
  }
  double mean_sq = sum_sq / n;
  double inv_rms = 1.0 / std::sqrt(mean_sq + eps);
  for (int d = 0; d < n; ++d)
    y[d] = oracle_bf16_to_double(x[d]) * inv_rms * oracle_bf16_to_double(w[d]);
}

// Rotation of one pair (a, b) by an angle with cosine c and sine s:
// a' = a c - b s, b' = b c + a s  (multiplication of a + ib by c + is).
void rotate_pair(double* a, double* b, double c, double s) {
  double a0 = *a, b0 = *b;
  *a = a0 * c - b0 * s;
  *b = b0 * c + a0 * s;
}

// The KV head of one token, normalised with kv_weight and rotated like a Q
// head (reading: the norm applies to KV as well as to Q).
void kv_head(const uint16_t* x, const uint16_t* w, const float* cosv,
             const float* sinv, double eps, double* y) {
  rms_norm(x, w, kHeadDim, eps, y);
  for (int i = 0; i < kRopeDim / 2; ++i)
    rotate_pair(&y[kRopeStart + 2 * i], &y[kRopeStart + 2 * i + 1], cosv[i],
                sinv[i]);
}

// Quantise one normalised, rotated KV head y and write its cache row and
// exponent bytes.  Seven UE8M0 power-of-two block scales per token ([P1]
// "Performance": a single scalar scale could not hold one exponent per
// block), each the smallest power of two that brings the block's largest
// magnitude within the E4M3 range; the rotary dims are kept
// as bf16 after the codes (reading).  The exponent and the codes are integers
// that floating-point values decide; both are decided on each element's
// nearest fp32 value, the precision the operator computes in ([P2] "The four
// test and benchmark fixes": the reference takes q to fp32), so that a block
// maximum a hair above a power-of-two boundary in double, but on it in fp32,
// gets the fp32 answer.
void quantise_insert(const double* y, uint8_t* dst, uint8_t* scale) {
  double yf[kRopeStart];
  for (int d = 0; d < kRopeStart; ++d) yf[d] = to_fp32(y[d]);
  for (int b = 0; b < kNumBlocks; ++b) {
    double amax = 0.0;
    for (int d = b * kQuantBlock; d < (b + 1) * kQuantBlock; ++d)
      amax = std::fmax(amax, std::fabs(yf[d]));
    int32_t e = oracle_ue8m0_exponent(amax);
    scale[b] = static_cast<uint8_t>(e + 127);
    for (int d = b * kQuantBlock; d < (b + 1) * kQuantBlock; ++d)
      dst[d] = oracle_e4m3_encode(std::ldexp(yf[d], -e));  // exact scaling
  }
  for (int j = 0; j < kRopeDim; ++j) {
    uint16_t bits = oracle_bf16_rne(y[kRopeStart + j]);
    dst[kRopeStart + 2 * j] = static_cast<uint8_t>(bits & 0xFF);
    dst[kRopeStart + 2 * j + 1] = static_cast<uint8_t>(bits >> 8);
  }
}

// The walk of the read side through block tables: token j of sequence s is
// slot block_table[s][j / 64] * 64 + j % 64 (or -1 for a page id outside the
// cache) and goes to output row out_offsets[s] + j; tokens past the table's
// width and rows outside [0, num_rows) are skipped.  Calls row_fn(slot, row)
// for every row written.
template <class RowFn>
void for_each_table_row(int64_t num_pages, const int32_t* block_table,
                        int32_t num_seqs, int32_t max_blocks_per_seq,
                        const int32_t* seq_lens, const int64_t* out_offsets,
                        int64_t num_rows, RowFn row_fn) {
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t len = seq_lens[s];
    for (int64_t j = 0; j < len && j < int64_t{max_blocks_per_seq} * kPageSize; ++j) {
      const int64_t row = out_offsets[s] + j;
      if (row < 0 || row >= num_rows) continue;
      const int64_t page = block_table[int64_t{s} * max_blocks_per_seq + j / kPageSize];
      const int64_t slot = page < 0 || page >= num_pages ? -1 : page * kPageSize + j % kPageSize;
      row_fn(slot, row);
    }
  }
}

}  // namespace

extern "C" {

double oracle_bf16_to_double(uint16_t bits) {
  uint32_t u = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return static_cast<double>(f);
}

uint16_t oracle_bf16_rne(double v) {
  // bf16 keeps 8 significant bits (1 implicit + 7 stored) with the exponent
  // range of binary32: normals from 2^-126, subnormal spacing 2^-133.
  if (std::isnan(v)) return 0x7FC0;
  NearestEven mode;
  double a = std::fabs(v);
  double r;
  if (a == 0.0) {
    r = 0.0;
  } else {
    int k;
    std::frexp(a, &k);  // a = m * 2^k, m in [0.5, 1): top bit has weight 2^(k-1)
    int lsb_exp = (k - 1) - 7;
    if (lsb_exp < -133) lsb_exp = -133;
    r = round_to_quantum(a, std::ldexp(1.0, lsb_exp));
  }
  uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  if (r >= std::ldexp(1.0, 128)) return sign | 0x7F80;  // overflow to inf
  float f = static_cast<float>(r);  // exact: r has at most 8 significant bits
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  return sign | static_cast<uint16_t>(u >> 16);
}

double oracle_fp16_to_double(uint16_t bits) {
  // IEEE binary16: sign, 5 exponent bits (bias 15), 10 mantissa bits.
  const int sign = bits >> 15;
  const int exp_field = (bits >> 10) & 0x1F;
  const int mant = bits & 0x3FF;
  double mag;
  if (exp_field == 0x1F)
    mag = mant ? std::nan("") : HUGE_VAL;
  else if (exp_field == 0)
    mag = std::ldexp(static_cast<double>(mant), -24);
  else
    mag = std::ldexp(1.0 + mant / 1024.0, exp_field - 15);
  return sign ? -mag : mag;
}

uint16_t oracle_fp16_rne(double v) {
  if (std::isnan(v)) return 0x7E00;
  NearestEven mode;
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  const double a = std::fabs(v);
  double r = 0.0;
  if (a != 0.0) {
    int k;
    std::frexp(a, &k);
    const int top = k - 1;
    const int lsb_exp = (top < -14 ? -14 : top) - 10;  // subnormal spacing 2^-24
    r = round_to_quantum(a, std::ldexp(1.0, lsb_exp));
  }
  if (r > 65504.0) return sign | 0x7C00;  // rounds past the largest finite
  if (r < std::ldexp(1.0, -14))
    return sign | static_cast<uint16_t>(std::ldexp(r, 24));
  int k;
  const double m = std::frexp(r, &k);
  const int exp_field = (k - 1) + 15;
  const int mant = static_cast<int>((2.0 * m - 1.0) * 1024.0);
  return sign | static_cast<uint16_t>((exp_field << 10) | mant);
}

double oracle_e4m3_decode(uint8_t code) {
  // OCP 8-bit floating point, E4M3: sign, 4 exponent bits (bias 7), 3
  // mantissa bits; exponent field 0 is subnormal; S.1111.111 is NaN.
  int sign = code >> 7;
  int exp_field = (code >> 3) & 0xF;
  int mant = code & 0x7;
  if (exp_field == 0xF && mant == 0x7) return std::nan("");
  double mag = exp_field == 0 ? std::ldexp(static_cast<double>(mant), -9)
                              : std::ldexp(1.0 + mant / 8.0, exp_field - 7);
  return sign ? -mag : mag;
}

uint8_t oracle_e4m3_encode(double v) {
  NearestEven mode;
  uint8_t sign = std::signbit(v) ? 0x80 : 0x00;
  double a = std::fabs(v);
  if (std::isnan(v)) return 0x7F;
  // Quantum: 2^(E-3) for a normal value in [2^E, 2^(E+1)), E >= -6; the
  // subnormal range below 2^-6 has the fixed spacing 2^-9.
  double r;
  if (a == 0.0) {
    r = 0.0;
  } else {
    int k;
    std::frexp(a, &k);
    int top = k - 1;
    int lsb_exp = (top < -6 ? -6 : top) - 3;
    r = round_to_quantum(a, std::ldexp(1.0, lsb_exp));
  }
  if (r > kE4M3Max) r = kE4M3Max;  // saturate: no infinities in E4M3
  // Encode the representable magnitude r.
  uint8_t bits;
  if (r < std::ldexp(1.0, -6)) {
    bits = static_cast<uint8_t>(std::ldexp(r, 9));  // subnormal (or zero)
  } else {
    int k;
    double m = std::frexp(r, &k);  // r = m 2^k, m in [0.5, 1)
    int exp_field = (k - 1) + 7;
    int mant = static_cast<int>((2.0 * m - 1.0) * 8.0);
    bits = static_cast<uint8_t>((exp_field << 3) | mant);
  }
  return sign | bits;
}

int32_t oracle_ue8m0_exponent(double amax) {
  // Smallest integer e with amax <= 448 * 2^e.  Write amax = m 2^k with
  // m in [0.5, 1) and 448 = 0.875 * 2^9: then amax <= 448 * 2^e exactly when
  // e >= k - 9 for m <= 0.875 and when e >= k - 8 for m > 0.875.
  if (amax == 0.0) return -127;
  int k;
  double m = std::frexp(amax, &k);
  int e = k - 9 + (m > 0.875 ? 1 : 0);
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

void oracle_qnorm_rope_kv_quant_insert(
    uint16_t* q, const uint16_t* kv, const uint16_t* q_weight,
    const uint16_t* kv_weight, const float* cos_sin_cache,
    const int64_t* positions, const int64_t* slot_mapping, uint8_t* kv_cache,
    uint8_t* kv_scale, int64_t num_tokens, int32_t num_heads,
    int64_t num_pages, double eps) {
  const int64_t num_slots = num_pages * kPageSize;
  double y[kHeadDim];
  for (int64_t t = 0; t < num_tokens; ++t) {
    // Interleaved rotary angles of this token's position: pair i rotates
    // dims (448 + 2i, 449 + 2i) by cos[i], sin[i] (reading: interleaved pairs
    // on the last 64 dims, cosines before sines in the cache row).
    const float* row = cos_sin_cache + positions[t] * kRopeDim;
    const float* cosv = row;
    const float* sinv = row + kRopeDim / 2;

    // Q: every head is normalised with q_weight, rotated and written back as
    // bf16 ([P2] "What the optimisation does": a Q slot is normalise and
    // rotate; [P1] "Correctness": q compared in bf16 ULP).
    for (int32_t h = 0; h < num_heads; ++h) {
      uint16_t* qh = q + (t * num_heads + h) * kHeadDim;
      rms_norm(qh, q_weight, kHeadDim, eps, y);
      for (int i = 0; i < kRopeDim / 2; ++i)
        rotate_pair(&y[kRopeStart + 2 * i], &y[kRopeStart + 2 * i + 1],
                    cosv[i], sinv[i]);
      for (int d = 0; d < kHeadDim; ++d) qh[d] = oracle_bf16_rne(y[d]);
    }

    // KV: the single latent head.
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) continue;  // skipped token
    kv_head(kv + t * kHeadDim, kv_weight, cosv, sinv, eps, y);

    quantise_insert(y, kv_cache + slot * kRowBytes, kv_scale + slot * kScaleBytes);
  }
}

void oracle_qnorm_rope_kv_quant_insert_scalar(
    uint16_t* q, const uint16_t* kv, const uint16_t* q_weight,
    const uint16_t* kv_weight, const float* cos_sin_cache,
    const int64_t* positions, const int64_t* slot_mapping, uint8_t* kv_cache,
    float kv_cache_scale, int64_t num_tokens, int32_t num_heads,
    int64_t num_pages, double eps) {
  const int64_t num_slots = num_pages * kPageSize;
  double y[kHeadDim];
  for (int64_t t = 0; t < num_tokens; ++t) {
    const float* row = cos_sin_cache + positions[t] * kRopeDim;
    const float* cosv = row;
    const float* sinv = row + kRopeDim / 2;
    for (int32_t h = 0; h < num_heads; ++h) {
      uint16_t* qh = q + (t * num_heads + h) * kHeadDim;
      rms_norm(qh, q_weight, kHeadDim, eps, y);
      for (int i = 0; i < kRopeDim / 2; ++i)
        rotate_pair(&y[kRopeStart + 2 * i], &y[kRopeStart + 2 * i + 1],
                    cosv[i], sinv[i]);
      for (int d = 0; d < kHeadDim; ++d) qh[d] = oracle_bf16_rne(y[d]);
    }
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) continue;
    kv_head(kv + t * kHeadDim, kv_weight, cosv, sinv, eps, y);
    uint8_t* dst = kv_cache + slot * kRowBytes;
    // one scale for everything: codes of y / s, saturating at the E4M3 range.
    // The code is decided in fp32 like the blockwise one: the element's fp32
    // value divided by the fp32 scale, the quotient rounded to fp32 (a double
    // quotient of two fp32 values rounds to the correctly rounded fp32 one).
    for (int d = 0; d < kRopeStart; ++d)
      dst[d] = oracle_e4m3_encode(
          to_fp32(to_fp32(y[d]) / static_cast<double>(kv_cache_scale)));
    for (int j = 0; j < kRopeDim; ++j) {
      uint16_t bits = oracle_bf16_rne(y[kRopeStart + j]);
      dst[kRopeStart + 2 * j] = static_cast<uint8_t>(bits & 0xFF);
      dst[kRopeStart + 2 * j + 1] = static_cast<uint8_t>(bits >> 8);
    }
  }
}

void oracle_kv_normalised(const uint16_t* kv, const uint16_t* kv_weight,
                          const float* cos_sin_cache, const int64_t* positions,
                          int64_t num_tokens, double eps, double* y_out) {
  for (int64_t t = 0; t < num_tokens; ++t) {
    const float* row = cos_sin_cache + positions[t] * kRopeDim;
    kv_head(kv + t * kHeadDim, kv_weight, row, row + kRopeDim / 2, eps,
            y_out + t * kHeadDim);
  }
}

void oracle_kv_cache_gather_dequant_scalar(const uint8_t* kv_cache,
                                           float kv_cache_scale,
                                           const int64_t* slots,
                                           int64_t num_rows, int64_t num_pages,
                                           uint16_t* out) {
  const int64_t num_slots = num_pages * kPageSize;
  for (int64_t i = 0; i < num_rows; ++i) {
    uint16_t* dst = out + i * kHeadDim;
    const int64_t slot = slots[i];
    if (slot < 0 || slot >= num_slots) {
      for (int d = 0; d < kHeadDim; ++d) dst[d] = 0;
      continue;
    }
    const uint8_t* row = kv_cache + slot * kRowBytes;
    for (int d = 0; d < kRopeStart; ++d)
      dst[d] = oracle_bf16_rne(oracle_e4m3_decode(row[d]) *
                               static_cast<double>(kv_cache_scale));
    for (int j = 0; j < kRopeDim; ++j)
      dst[kRopeStart + j] = static_cast<uint16_t>(
          row[kRopeStart + 2 * j] | (row[kRopeStart + 2 * j + 1] << 8));
  }
}

void oracle_rms_norm_rows(const uint16_t* x, const uint16_t* weight,
                          uint16_t* out, int64_t num_rows, double eps) {
  double y[kHeadDim];
  for (int64_t r = 0; r < num_rows; ++r) {
    rms_norm(x + r * kHeadDim, weight, kHeadDim, eps, y);
    for (int d = 0; d < kHeadDim; ++d) out[r * kHeadDim + d] = oracle_bf16_rne(y[d]);
  }
}

void oracle_rope_rows(uint16_t* x, const float* cos_sin_cache,
                      const int64_t* positions, int64_t num_tokens,
                      int32_t rows_per_token) {
  for (int64_t t = 0; t < num_tokens; ++t) {
    const float* row = cos_sin_cache + positions[t] * kRopeDim;
    for (int32_t h = 0; h < rows_per_token; ++h) {
      uint16_t* xr = x + (t * rows_per_token + h) * kHeadDim;
      for (int i = 0; i < kRopeDim / 2; ++i) {
        double a = oracle_bf16_to_double(xr[kRopeStart + 2 * i]);
        double b = oracle_bf16_to_double(xr[kRopeStart + 2 * i + 1]);
        rotate_pair(&a, &b, row[i], row[kRopeDim / 2 + i]);
        xr[kRopeStart + 2 * i] = oracle_bf16_rne(a);
        xr[kRopeStart + 2 * i + 1] = oracle_bf16_rne(b);
      }
    }
  }
}

void oracle_kv_quant_insert(const uint16_t* kv, const int64_t* slot_mapping,
                            uint8_t* kv_cache, uint8_t* kv_scale,
                            int64_t num_tokens, int64_t num_pages) {
  const int64_t num_slots = num_pages * kPageSize;
  double y[kHeadDim];
  for (int64_t t = 0; t < num_tokens; ++t) {
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) continue;
    for (int d = 0; d < kHeadDim; ++d) y[d] = oracle_bf16_to_double(kv[t * kHeadDim + d]);
    quantise_insert(y, kv_cache + slot * kRowBytes, kv_scale + slot * kScaleBytes);
  }
}

// One cache row dequantised (blockwise exponents), or a zero row for a slot
// outside [0, num_slots).
static void dequant_row(const uint8_t* kv_cache, const uint8_t* kv_scale,
                        int64_t slot, int64_t num_slots, uint16_t* dst) {
  if (slot < 0 || slot >= num_slots) {
    for (int d = 0; d < kHeadDim; ++d) dst[d] = 0;
    return;
  }
  const uint8_t* row = kv_cache + slot * kRowBytes;
  const uint8_t* scale = kv_scale + slot * kScaleBytes;
  for (int d = 0; d < kRopeStart; ++d) {
    const int e = static_cast<int>(scale[d / kQuantBlock]) - 127;
    dst[d] = oracle_bf16_rne(std::ldexp(oracle_e4m3_decode(row[d]), e));
  }
  for (int j = 0; j < kRopeDim; ++j)
    dst[kRopeStart + j] = static_cast<uint16_t>(
        row[kRopeStart + 2 * j] | (row[kRopeStart + 2 * j + 1] << 8));
}

void oracle_kv_cache_gather_dequant(const uint8_t* kv_cache,
                                    const uint8_t* kv_scale,
                                    const int64_t* slots, int64_t num_rows,
                                    int64_t num_pages, uint16_t* out) {
  const int64_t num_slots = num_pages * kPageSize;
  for (int64_t i = 0; i < num_rows; ++i)
    dequant_row(kv_cache, kv_scale, slots[i], num_slots, out + i * kHeadDim);
}

void oracle_kv_cache_gather_dequant_paged(
    const uint8_t* kv_cache, const uint8_t* kv_scale, int64_t num_pages,
    const int32_t* block_table, int32_t num_seqs, int32_t max_blocks_per_seq,
    const int32_t* seq_lens, const int64_t* out_offsets, int64_t num_rows,
    uint16_t* out) {
  const int64_t num_slots = num_pages * kPageSize;
  for_each_table_row(num_pages, block_table, num_seqs, max_blocks_per_seq,
                     seq_lens, out_offsets, num_rows,
                     [&](int64_t slot, int64_t row) {
                       dequant_row(kv_cache, kv_scale, slot, num_slots,
                                   out + row * kHeadDim);
                     });
}

void oracle_kv_cache_gather_dequant_paged_scalar(
    const uint8_t* kv_cache, float kv_cache_scale, int64_t num_pages,
    const int32_t* block_table, int32_t num_seqs, int32_t max_blocks_per_seq,
    const int32_t* seq_lens, const int64_t* out_offsets, int64_t num_rows,
    uint16_t* out) {
  for_each_table_row(num_pages, block_table, num_seqs, max_blocks_per_seq,
                     seq_lens, out_offsets, num_rows,
                     [&](int64_t slot, int64_t row) {
                       oracle_kv_cache_gather_dequant_scalar(
                           kv_cache, kv_cache_scale, &slot, 1, num_pages,
                           out + row * kHeadDim);
                     });
}

void oracle_qk_norm_rope_packed(
    uint16_t* qkv, int64_t num_tokens, int32_t num_heads_q,
    int32_t num_heads_k, int32_t num_heads_v, int32_t head_dim, double eps,
    const uint16_t* q_weight, const uint16_t* k_weight,
    const float* cos_sin_cache, const int64_t* position_ids) {
  const int64_t row_elems =
      static_cast<int64_t>(num_heads_q + num_heads_k + num_heads_v) * head_dim;
  const int half = head_dim / 2;
  double* y = new double[head_dim];
  for (int64_t t = 0; t < num_tokens; ++t) {
    const float* row = cos_sin_cache + position_ids[t] * head_dim;
    const float* cosv = row;
    const float* sinv = row + half;
    // Heads are packed [Q heads | K heads | V heads]; Q heads take q_weight
    // and K heads k_weight; V heads are not touched ([P3] "Summary").
    for (int32_t h = 0; h < num_heads_q + num_heads_k; ++h) {
      uint16_t* xh = qkv + t * row_elems + static_cast<int64_t>(h) * head_dim;
      const uint16_t* w = h < num_heads_q ? q_weight : k_weight;
      rms_norm(xh, w, head_dim, eps, y);
      // NeoX pairs (i, i + D/2) over the whole head; each element carries its
      // own weight into the rotation ([P3] "Summary", paired-weight rule).
      for (int i = 0; i < half; ++i) rotate_pair(&y[i], &y[i + half], cosv[i], sinv[i]);
      for (int d = 0; d < head_dim; ++d) xh[d] = oracle_bf16_rne(y[d]);
    }
  }
  delete[] y;
}

// The packed operator's separate-launch baseline ([P3] "Benchmark /
// Performance Impact": two RmsNorm calls into preallocated Q and K outputs,
// then two RotaryEmbedding calls).  Each stage rounds its output to bf16.
void oracle_rms_norm_heads(const uint16_t* x, int64_t x_token_stride,
                           const uint16_t* weight, uint16_t* out,
                           int64_t num_tokens, int32_t num_heads,
                           int32_t head_dim, double eps) {
  double* y = new double[head_dim];
  for (int64_t t = 0; t < num_tokens; ++t)
    for (int32_t h = 0; h < num_heads; ++h) {
      rms_norm(x + t * x_token_stride + static_cast<int64_t>(h) * head_dim,
               weight, head_dim, eps, y);
      uint16_t* dst = out + (t * num_heads + h) * static_cast<int64_t>(head_dim);
      for (int d = 0; d < head_dim; ++d) dst[d] = oracle_bf16_rne(y[d]);
    }
  delete[] y;
}

void oracle_rope_neox_heads(uint16_t* x, const float* cos_sin_cache,
                            const int64_t* positions, int64_t num_tokens,
                            int32_t num_heads, int32_t head_dim) {
  const int half = head_dim / 2;
  for (int64_t t = 0; t < num_tokens; ++t) {
    const float* row = cos_sin_cache + positions[t] * head_dim;
    for (int32_t h = 0; h < num_heads; ++h) {
      uint16_t* xh = x + (t * num_heads + h) * static_cast<int64_t>(head_dim);
      for (int i = 0; i < half; ++i) {
        double a = oracle_bf16_to_double(xh[i]);
        double b = oracle_bf16_to_double(xh[i + half]);
        rotate_pair(&a, &b, row[i], row[half + i]);
        xh[i] = oracle_bf16_rne(a);
        xh[i + half] = oracle_bf16_rne(b);
      }
    }
  }
}

void oracle_qk_norm_rope_packed_ex(
    uint16_t* qkv, int64_t num_tokens, int32_t num_heads_q,
    int32_t num_heads_k, int32_t num_heads_v, int32_t head_dim,
    int32_t rotary_dim, int32_t is_neox, int32_t is_fp16, double eps,
    const uint16_t* q_weight, const uint16_t* k_weight,
    const float* cos_sin_cache, const int64_t* position_ids) {
  const int64_t row_elems =
      static_cast<int64_t>(num_heads_q + num_heads_k + num_heads_v) * head_dim;
  const int half = rotary_dim / 2;
  auto decode = [is_fp16](uint16_t b) {
    return is_fp16 ? oracle_fp16_to_double(b) : oracle_bf16_to_double(b);
  };
  auto encode = [is_fp16](double v) {
    return is_fp16 ? oracle_fp16_rne(v) : oracle_bf16_rne(v);
  };
  double* y = new double[head_dim];
  for (int64_t t = 0; t < num_tokens; ++t) {
    const float* row = cos_sin_cache + position_ids[t] * rotary_dim;
    for (int32_t h = 0; h < num_heads_q + num_heads_k; ++h) {
      uint16_t* xh = qkv + t * row_elems + static_cast<int64_t>(h) * head_dim;
      const uint16_t* w = h < num_heads_q ? q_weight : k_weight;
      // RMSNorm over the whole head with its own weight per element
      double sum_sq = 0.0;
      for (int d = 0; d < head_dim; ++d) sum_sq += decode(xh[d]) * decode(xh[d]);
      const double inv_rms = 1.0 / std::sqrt(sum_sq / head_dim + eps);
      for (int d = 0; d < head_dim; ++d) y[d] = decode(xh[d]) * inv_rms * decode(w[d]);
      // rotation of the first rotary_dim dims only
      for (int i = 0; i < half; ++i) {
        if (is_neox)
          rotate_pair(&y[i], &y[i + half], row[i], row[half + i]);
        else
          rotate_pair(&y[2 * i], &y[2 * i + 1], row[i], row[half + i]);
      }
      for (int d = 0; d < head_dim; ++d) xh[d] = encode(y[d]);
    }
  }
  delete[] y;
}

}  // extern "C"
