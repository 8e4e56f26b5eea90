/*
 * fp8kv — fused attention prologue for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libfp8kv.so.  Two operators, both single-launch, stream-ordered and
 * asynchronous, both bandwidth-bound (no matrix cores):
 *
 *   qnorm_rope_kv_quant_insert — the DeepSeek-V4 attention prologue that the
 *     pages call fused_deepseek_v4_qnorm_rope_kv_rope_quant_insert
 *     (FlagGems PR #5449 "[KMCompiler][Hygon] Token-tiled
 *     fused_deepseek_v4_qnorm_rope_kv_rope_quant_insert", and FlagGems PR #5321
 *     "… plus test and benchmark fixes", sections "Performance" and "What the
 *     optimisation does"): per token, every Q head is RMS-normalised and
 *     rotated in place; the single latent KV head is normalised, rotated,
 *     quantised to FP8 E4M3 with seven UE8M0 (power-of-two) block exponents
 *     and inserted into a paged cache through slot_mapping.
 *
 *   qk_norm_rope_packed — the packed-QKV FusedQkNormRope (InfiniOps PR #1019
 *     "FusedQkNormRope", section "Summary"): per-head Q and K RMSNorm followed
 *     by full-head NeoX RoPE, in place in qkv[T, (Hq+Hk+Hv)*D]; V untouched.
 *     Argument order follows that page's "Open-Source Alignment" list.
 *
 * Conventions shared by every call:
 *   - Every buffer pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees or synchronises, and keeps no state
 *     besides the two tuning knobs below.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it; the call returns before the kernel runs.
 *   - Return value: FP8KV_OK (0) or a positive fp8kv_status.  On any argument
 *     error nothing is launched and no buffer is touched.  num_tokens == 0
 *     returns FP8KV_OK without touching the device.  A launch failure returns
 *     FP8KV_ERR_LAUNCH.  A fault inside a kernel surfaces, as with any HIP
 *     kernel, at the caller's next synchronising call.
 *   - Tensors are dense and row-major (contiguous).  bf16 data is passed as
 *     void*; the library reads and writes it as 16-bit bf16 patterns.
 *   - Calls that write overlapping buffers race unless stream-ordered.
 */
#ifndef FP8KV_H
#define FP8KV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8KV_ABI_VERSION 2

enum fp8kv_status {
  FP8KV_OK = 0,
  FP8KV_ERR_NULL = 1,        /* a required pointer is NULL                     */
  FP8KV_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be,
                                or too large for the kernels' index range      */
  FP8KV_ERR_UNSUPPORTED = 3, /* a layout parameter other than the supported one */
  FP8KV_ERR_ALIGN = 4,       /* a pointer is not aligned as documented          */
  FP8KV_ERR_DEVICE = 5,      /* no current HIP device, or it is not gfx950      */
  FP8KV_ERR_LAUNCH = 6,      /* the kernel launch itself failed                 */
  FP8KV_ERR_VALUE = 7        /* eps is negative, infinite or NaN                */
};

/*
 * Fused DeepSeek-V4 attention prologue.
 *
 * Shapes: T = num_tokens, H = num_heads, D = head_dim = 512 (the pages count
 * 16744448 q elements at 511 tokens and 64 heads: FlagGems PR #5449,
 * "Correctness"), R = rope_dim = 64, page_size = 64.
 *
 *   q              bf16 [T, H, 512], read and rewritten in place.  16-byte
 *                  aligned.
 *   kv             bf16 [T, 512], the one latent KV head per token (the
 *                  program count is num_tokens * (num_heads + 1): FlagGems
 *                  PR #5449, "Dispatch threshold").  Read only.  16-byte
 *                  aligned.
 *   q_weight       bf16 [512], RMSNorm weight of every Q head.  16-B aligned.
 *   kv_weight      bf16 [512], RMSNorm weight of the KV head.  16-B aligned.
 *   cos_sin_cache  fp32 [max_position, 64]; row p holds cos(p f_i) for
 *                  i = 0..31 followed by sin(p f_i).  16-byte aligned.
 *   positions      int64 [T].  A token whose position is outside
 *                  [0, max_position) is skipped entirely: its q heads and its
 *                  cache slot are left as they were (no read out of bounds).
 *   slot_mapping   int64 [T].  Flat cache slot (page * page_size + offset) of
 *                  each token's KV row.  A negative slot, or one >=
 *                  num_pages * page_size, skips the cache write of that token;
 *                  its q heads are still processed.  Slots of distinct tokens
 *                  must differ (precondition, not checked).
 *   kv_cache       uint8 [num_pages, page_size, 576], 16-byte aligned.  Row of
 *                  a written slot: bytes 0..447 = FP8 E4M3 (OCP, finite-only)
 *                  codes of dims 0..447; bytes 448..575 = dims 448..511 as 64
 *                  little-endian bf16.  Rows of other slots are not touched.
 *   kv_scale       uint8 [num_pages, page_size, 8].  Bytes 0..6 of a written
 *                  slot = e_b + 127, where 2^e_b is the UE8M0 scale of the
 *                  64-dim block b (dims 64b..64b+63) and e_b is the smallest
 *                  integer with amax_b <= 448 * 2^e_b, clamped to [-127, 127]
 *                  (amax 0 gives -127).  Byte 7 is never written.  One
 *                  exponent for each of a token's seven blocks: FlagGems
 *                  PR #5449, "Performance".
 *   eps            added to the mean square inside the square root; finite
 *                  and >= 0 (FP8KV_ERR_VALUE otherwise).  With eps = 0 an
 *                  all-zero head is 0/0 and its outputs are NaN.
 * The elements of q, kv, the weights and the table rows are finite
 * (precondition, not checked).  A NaN or an infinity in q or kv makes the
 * outputs of its own head unspecified (NaN, or zero where an infinite mean
 * square scales finite elements to 0), and in the KV head also its exponents
 * and codes; no other head or token is affected.  One in a weight or a table
 * row does the same to every head that uses it.
 *
 * Per token t, for each Q head and then for the KV head x (with its weight w):
 *   y_d = x_d / sqrt(mean_d(x_d^2) + eps) * w_d            (fp32)
 *   pairs (448 + 2i, 449 + 2i), i < 32, rotate by row positions[t]:
 *     y_a' = y_a cos_i - y_b sin_i,  y_b' = y_b cos_i + y_a sin_i
 *   Q: q[t, h, :] = bf16_rne(y).
 *   KV: codes_d = e4m3_rne(y_d * 2^-e_b) for d < 448; dims 448.. as bf16_rne.
 *
 * Errors: NULL pointer -> FP8KV_ERR_NULL; num_tokens < 0, num_heads < 1,
 * max_position < 1, num_pages < 0 or num_tokens * (num_heads + 1) >= 2^31 ->
 * FP8KV_ERR_SHAPE; head_dim != 512, rope_dim != 64, page_size != 64 ->
 * FP8KV_ERR_UNSUPPORTED; misaligned pointer -> FP8KV_ERR_ALIGN.
 */
int qnorm_rope_kv_quant_insert(
    void* q, const void* kv, const void* q_weight, const void* kv_weight,
    const float* cos_sin_cache, const int64_t* positions,
    const int64_t* slot_mapping, uint8_t* kv_cache, uint8_t* kv_scale,
    int64_t num_tokens, int32_t num_heads, int32_t head_dim, int32_t rope_dim,
    int64_t max_position, int64_t num_pages, int32_t page_size, float eps,
    void* stream);

/*
 * The same prologue writing the scalar-scale FP8 cache convention that the
 * pages set against the blockwise one (FlagGems PR #5449 "Performance": a
 * single kv_cache_scale float for the whole cache, with no room for a
 * power-of-two exponent per block).  Arguments as qnorm_rope_kv_quant_insert, except:
 *   kv_cache_scale  DEVICE pointer to one fp32 scale s > 0 (4-byte aligned),
 *                   required when num_pages > 0.  The value is a precondition
 *                   (not checked: a non-positive or non-finite s gives
 *                   saturated or undefined codes, never a fault).
 * q is processed exactly as by qnorm_rope_kv_quant_insert.  A written cache
 * row holds E4M3(y_d / s) for d < 448 (nearest even, saturating at +-448) and
 * dims 448..511 as bf16; there is no exponent tensor.
 */
int qnorm_rope_kv_quant_insert_scalar_scale(
    void* q, const void* kv, const void* q_weight, const void* kv_weight,
    const float* cos_sin_cache, const int64_t* positions,
    const int64_t* slot_mapping, uint8_t* kv_cache, const float* kv_cache_scale,
    int64_t num_tokens, int32_t num_heads, int32_t head_dim, int32_t rope_dim,
    int64_t max_position, int64_t num_pages, int32_t page_size, float eps,
    void* stream);

/*
 * Packed-QKV FusedQkNormRope (InfiniOps PR #1019, "Summary").
 *
 *   qkv           bf16 [T, (Hq + Hk + Hv) * D], heads packed as
 *                 [Q heads | K heads | V heads].  Q and K heads are rewritten
 *                 in place; the V heads are neither read nor written.  16-B
 *                 aligned.
 *   num_heads_q/k/v  Hq >= 0, Hk >= 0, Hv >= 0, Hq + Hk >= 1.
 *   head_dim      D = 128 (the page's guarded fast path; others ->
 *                 FP8KV_ERR_UNSUPPORTED).
 *   eps           added inside the square root; finite and >= 0
 *                 (FP8KV_ERR_VALUE otherwise).
 *   q_weight      bf16 [D] for Q heads; k_weight bf16 [D] for K heads;
 *                 separate one-dimensional tensors as on the page.  16-B
 *                 aligned.
 *   cos_sin_cache fp32 [max_position, D]; row p = D/2 cosines then D/2 sines.
 *                 16-byte aligned.
 *   is_neox       must be 1 (NeoX pairs (i, i + D/2)); else UNSUPPORTED.
 *   position_ids  int64 [T]; a token whose position is outside
 *                 [0, max_position) is left untouched.
 *   forced_token_heads_per_warp  must be -1 (automatic scheduling, as on the
 *                 page); anything else -> FP8KV_ERR_UNSUPPORTED.
 *
 * Per Q or K head x with weight w:
 *   n_d = x_d / sqrt(mean(x^2) + eps) * w_d
 *   out_i = n_i cos_i - n_{i+D/2} sin_i,  out_{i+D/2} = n_{i+D/2} cos_i + n_i sin_i
 * so the partner element enters the rotation with its own weight (the page's
 * paired-weight rule).  Outputs are rounded to bf16 (nearest even).  Inputs
 * are finite (precondition, as for the prologue: a non-finite element of qkv
 * makes only its own head's outputs unspecified; V elements are never read,
 * whatever their values).
 */
int qk_norm_rope_packed(
    void* qkv, int64_t num_tokens, int32_t num_heads_q, int32_t num_heads_k,
    int32_t num_heads_v, int32_t head_dim, float eps, const void* q_weight,
    const void* k_weight, const float* cos_sin_cache, int32_t is_neox,
    const int64_t* position_ids, int32_t forced_token_heads_per_warp,
    int64_t max_position, void* stream);

/* Element types of qk_norm_rope_packed_ex. */
enum fp8kv_dtype { FP8KV_DTYPE_BF16 = 0, FP8KV_DTYPE_FP16 = 1 };

/*
 * Packed-QKV Q/K RMSNorm + RoPE beyond the guarded fast path that InfiniOps
 * PR #1019 ships ("Notes for Reviewers": bf16, head_dim 128, full-dimension
 * NeoX only).  Same arguments and semantics as qk_norm_rope_packed, plus:
 *   head_dim     64, 128 or 256
 *   rotary_dim   R, a multiple of 16 with 0 <= R <= head_dim: only dims
 *                [0, R) of a head rotate; dims [R, head_dim) are normalised
 *                and weighted only (partial rotary); R = 0 is RMSNorm alone:
 *                no table row is read, so position_ids are not used (every
 *                token is written, whatever its position) and max_position
 *                may be 0
 *   is_neox      1: pairs (i, i + R/2); 0: interleaved pairs (2i, 2i + 1);
 *                i < R/2, rotated by cos_sin_cache row positions[t] =
 *                [R/2 cosines | R/2 sines] (fp32 [max_position, R]; may be
 *                NULL when R = 0)
 *   dtype        FP8KV_DTYPE_BF16 or FP8KV_DTYPE_FP16: the type of qkv and of
 *                both weights; outputs round to nearest even in that type
 * Anything else -> FP8KV_ERR_UNSUPPORTED.  There is no scheduling knob.
 */
int qk_norm_rope_packed_ex(
    void* qkv, int64_t num_tokens, int32_t num_heads_q, int32_t num_heads_k,
    int32_t num_heads_v, int32_t head_dim, float eps, const void* q_weight,
    const void* k_weight, const float* cos_sin_cache, int32_t is_neox,
    const int64_t* position_ids, int32_t rotary_dim, int32_t dtype,
    int64_t max_position, void* stream);

/*
 * Read side of the paged cache written by qnorm_rope_kv_quant_insert: gather
 * rows by slot and dequantise them to bf16 (the inverse the cache layout of
 * FlagGems PR #5449 "Performance" implies: FP8 codes plus one power-of-two
 * exponent for each of a token's seven blocks).
 *
 *   kv_cache   uint8 [num_pages, page_size, 576], layout as above.  16-B aligned.
 *   kv_scale   uint8 [num_pages, page_size, 8].  8-byte aligned.
 *   page_size  must be 64 (else FP8KV_ERR_UNSUPPORTED).
 *   slots      int64 [num_rows]: the flat slot of each output row.  A negative
 *              slot or one >= num_pages * page_size yields a row of +0.
 *   out        bf16 [num_rows, 512], written (16-byte aligned):
 *                out[i, d]       = E4M3(code[s, d]) * 2^(scale[s, d/64] - 127)
 *                                  for d < 448, rounded to bf16 (exact unless
 *                                  the exponent leaves bf16's range)
 *                out[i, 448 + j] = the stored bf16 rotary value j.
 * Errors: num_rows < 0 or >= 2^31, num_pages < 0 -> FP8KV_ERR_SHAPE; NULL
 * slots/out, or NULL cache/scale with num_pages > 0 -> FP8KV_ERR_NULL;
 * misalignment -> FP8KV_ERR_ALIGN.  num_rows == 0 returns FP8KV_OK.
 */
int kv_cache_gather_dequant(const uint8_t* kv_cache, const uint8_t* kv_scale,
                            int64_t num_pages, int32_t page_size,
                            const int64_t* slots, int64_t num_rows, void* out,
                            void* stream);

/*
 * The prologue taken apart into separate launches: the unfused baseline the
 * fused call is measured against (FlagGems PR #5449 "Performance": one fused
 * launch against the baseline's two; InfiniOps PR #1019 "Benchmark /
 * Performance Impact": separate RmsNorm and RotaryEmbedding calls).  Every
 * stage reads and writes bf16, so the composition rounds to bf16 between
 * stages where qnorm_rope_kv_quant_insert does not.
 *
 * rms_norm_rows: out[r, :] = bf16(x[r, :] / sqrt(mean(x[r, :]^2) + eps) * w)
 *   for num_rows rows of row_dim = 512 bf16 (x, out, weight 16-B aligned).
 *   out may equal x (in place); otherwise they must not overlap.
 * rope_rows: in place on x bf16 [num_tokens, rows_per_token, 512]: the pairs
 *   (448 + 2i, 449 + 2i), i < rope_dim / 2 = 32, of every row of token t
 *   rotate by cos_sin_cache[positions[t]] (layout as for the fused call) and
 *   are rounded to bf16; dims 0..447 are not touched.  A token whose position
 *   is outside [0, max_position) is left as it was.
 * kv_quant_insert: kv bf16 [num_tokens, 512] holds KV rows that are already
 *   normalised and rotated; each row whose slot_mapping entry is valid is
 *   quantised and written to kv_cache / kv_scale exactly as the fused call
 *   writes them (the exponent of a block is taken from the bf16 values).
 * Errors as for the fused call; row_dim != 512, rope_dim != 64 or
 * page_size != 64 -> FP8KV_ERR_UNSUPPORTED.  Zero rows/tokens return FP8KV_OK.
 */
int rms_norm_rows(const void* x, void* out, const void* weight,
                  int64_t num_rows, int32_t row_dim, float eps, void* stream);
int rope_rows(void* x, const float* cos_sin_cache, const int64_t* positions,
              int64_t num_tokens, int32_t rows_per_token, int32_t row_dim,
              int32_t rope_dim, int64_t max_position, void* stream);
int kv_quant_insert(const void* kv, const int64_t* slot_mapping,
                    uint8_t* kv_cache, uint8_t* kv_scale, int64_t num_tokens,
                    int64_t num_pages, int32_t page_size, void* stream);

/*
 * The packed Q/K operator taken apart into the four launches InfiniOps PR
 * #1019 "Benchmark / Performance Impact" measures the fused call against: an
 * RmsNorm of the Q heads and one of the K heads, each into its own
 * preallocated output, then a RotaryEmbedding of each.  Every stage reads
 * and writes bf16, so the composition rounds to bf16 between the norm and
 * the rotation where qk_norm_rope_packed does not.
 *
 * rms_norm_heads: head h < num_heads of token t < num_tokens is the
 *   head_dim = 128 bf16 values at x + t * x_token_stride + h * 128 (elements;
 *   for the Q heads of packed qkv: x = qkv, stride (Hq + Hk + Hv) * 128; for
 *   the K heads: x = qkv + Hq * 128).  out bf16 [num_tokens, num_heads, 128]
 *   (contiguous) = bf16(head / sqrt(mean(head^2) + eps) * weight).
 *   x_token_stride >= num_heads * 128 and a multiple of 8; x, out, weight
 *   16-B aligned.  out must not overlap x unless it equals x with
 *   x_token_stride = num_heads * 128 (in place).
 * rope_neox_heads: in place on x bf16 [num_tokens, num_heads, 128]: the
 *   NeoX pairs (i, i + 64), i < 64, of every head of token t rotate by
 *   cos_sin_cache[positions[t]] (fp32 [max_position, 128] = 64 cosines then
 *   64 sines; 16-B aligned) and are rounded to bf16.  A token whose position
 *   is outside [0, max_position) is left as it was.
 * Errors: head_dim != 128 -> FP8KV_ERR_UNSUPPORTED; negative counts, more
 *   than 2^31 - 1 heads in all, a short stride or max_position < 1 ->
 *   FP8KV_ERR_SHAPE; eps as for the fused calls.  Zero tokens or heads return
 *   FP8KV_OK without a launch.
 */
int rms_norm_heads(const void* x, int64_t x_token_stride, void* out,
                   const void* weight, int64_t num_tokens, int32_t num_heads,
                   int32_t head_dim, float eps, void* stream);
int rope_neox_heads(void* x, const float* cos_sin_cache, const int64_t* positions,
                    int64_t num_tokens, int32_t num_heads, int32_t head_dim,
                    int64_t max_position, void* stream);

/*
 * The read side through block tables, as an attention consumer indexes the
 * paged cache (the layout of FlagGems PR #5449 "Performance": pages of 64
 * token rows of 576 bytes plus seven exponents each).  Sequence s holds
 * seq_lens[s] tokens, 64 to a page, in the pages
 * block_table[s * max_blocks_per_seq + 0, 1, ...] in order; its token j is
 * slot block_table[s * max_blocks_per_seq + j / 64] * 64 + j % 64, and that
 * row, dequantised exactly as by kv_cache_gather_dequant, is written to
 * out[out_offsets[s] + j].  A page id outside [0, num_pages) gives a zero row.
 *
 *   block_table  int32 [num_seqs, max_blocks_per_seq] (4-byte aligned)
 *   seq_lens     int32 [num_seqs] (4-byte aligned); tokens past
 *                max_blocks_per_seq * 64 are not written
 *   out_offsets  int64 [num_seqs] (8-byte aligned): first output row of s
 *   out          bf16 [num_rows, 512], device, 16-byte aligned; rows outside
 *                [0, num_rows) are never written, nor are rows that no
 *                sequence covers
 * num_seqs <= 65535 and max_blocks_per_seq <= 2^24 (FP8KV_ERR_SHAPE
 * otherwise); page_size must be 64.  num_seqs, max_blocks_per_seq or
 * num_rows == 0 launches nothing.  kv_cache / kv_scale may be NULL only when
 * num_pages == 0 (every row written is then zero).  Sequences whose output
 * ranges overlap race (precondition: disjoint).
 */
int kv_cache_gather_dequant_paged(const uint8_t* kv_cache, const uint8_t* kv_scale,
                                  int64_t num_pages, int32_t page_size,
                                  const int32_t* block_table, int32_t num_seqs,
                                  int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                  const int64_t* out_offsets, int64_t num_rows,
                                  void* out, void* stream);

/*
 * Read side of the scalar-scale convention: as kv_cache_gather_dequant, with
 * out[i, d] = bf16(E4M3(code[s, d]) * kv_cache_scale[0]) for d < 448 (the
 * product rounded to fp32, then to bf16) and no exponent tensor.
 * kv_cache_scale is a device pointer, required when num_pages > 0.
 */
int kv_cache_gather_dequant_scalar_scale(const uint8_t* kv_cache,
                                         const float* kv_cache_scale,
                                         int64_t num_pages, int32_t page_size,
                                         const int64_t* slots, int64_t num_rows,
                                         void* out, void* stream);

/*
 * The scalar-scale read side through block tables: the rows, walk, bounds and
 * errors of kv_cache_gather_dequant_paged, each row dequantised as by
 * kv_cache_gather_dequant_scalar_scale.  kv_cache_scale is a device pointer
 * (4-byte aligned), required when num_pages > 0 and then read once per wave.
 */
int kv_cache_gather_dequant_paged_scalar_scale(
    const uint8_t* kv_cache, const float* kv_cache_scale, int64_t num_pages,
    int32_t page_size, const int32_t* block_table, int32_t num_seqs,
    int32_t max_blocks_per_seq, const int32_t* seq_lens,
    const int64_t* out_offsets, int64_t num_rows, void* out, void* stream);

/* Static text for a status code (never NULL). */
const char* fp8kv_status_string(int status);

/* Library ABI version (FP8KV_ABI_VERSION of the build). */
int fp8kv_abi_version(void);

/*
 * Dispatch threshold of the fused prologue, in programs = num_tokens *
 * (num_heads + 1) (the quantity FlagGems PR #5449 "Dispatch threshold" finds
 * both head counts agree on).  Calls below it use the small-batch kernel
 * (one (token, head) slot per 64-lane block); calls at or above it the tiled
 * kernel.  programs < 0 restores the built-in default; 0 sends everything to
 * the tiled kernel; INT64_MAX everything to the small-batch kernel.  MI355X
 * has no crossover: the small-batch shape is the fastest at every size
 * measured, so it is also the tiled kernel's default shape, and the built-in
 * default threshold is 0.
 * Process-wide; returns FP8KV_OK.  When the library is loaded, the threshold
 * starts at the value of the environment variable FP8KV_DISPATCH_THRESHOLD if
 * that is a non-negative decimal integer, else at the built-in default.
 */
int fp8kv_set_dispatch_threshold(int64_t programs);
int64_t fp8kv_get_dispatch_threshold(void);

/*
 * Tiling of the tiled prologue kernel: waves (of 64 lanes) per block and
 * Q slots per wave.  The built-in default (1, 1) is the measured best on
 * MI355X and equals the small-batch shape; the other instantiated shapes
 * exist for measurement (the scalar-scale prologue is built in two shapes:
 * (1, 1), and (4, 2), which it runs under any other tiling).  (0, 0) restores
 * the default.  Returns FP8KV_ERR_UNSUPPORTED, and changes nothing, for a shape
 * that is not built.  Process-wide.
 */
int fp8kv_set_tiling(int32_t waves_per_block, int32_t slots_per_wave);
void fp8kv_get_tiling(int32_t* waves_per_block, int32_t* slots_per_wave);

/*
 * Measurement aids: the hand-written streaming kernels the prologue's HBM
 * bandwidth is compared with (a bandwidth-bound operator is measured against
 * the rate of a plain copy on the same device; FlagGems PR #5449
 * "Performance" reports its kernel as a share of a measured copy peak).
 * Both move one 16-byte vector per lane, one 64-lane wave per block, with
 * non-temporal loads and stores (the stores with device scope, as the
 * prologue's q stores); neither is part of the prologue.  From
 * 128 MiB up the read-modify-write runs at most 25 blocks per CU (a request
 * for LDS it never uses), which measured 1-2.5% faster on MI355X; the copy
 * is never capped.
 *
 *   fp8kv_stream_copy  dst[0:bytes) = src[0:bytes)
 *   fp8kv_stream_rmw   buf[i] ^= mask for every 32-bit word i, in place
 *                      (mask 0 leaves the bytes unchanged; the pattern of
 *                      the prologue's in-place Q heads)
 *
 * bytes: a multiple of 16, >= 0 (FP8KV_ERR_SHAPE otherwise); 0 launches
 * nothing.  Pointers: device, 16-byte aligned (FP8KV_ERR_ALIGN), non-NULL
 * when bytes > 0 (FP8KV_ERR_NULL).  dst and src must not overlap.
 */
int fp8kv_stream_copy(void* dst, const void* src, int64_t bytes, void* stream);
int fp8kv_stream_rmw(void* buf, int64_t bytes, uint32_t mask, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8KV_H */
