/*
 * CPU oracle for the fused attention prologue and the packed Q/K norm+RoPE.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is a plain, slow, single-threaded
 * statement of what the two operators compute, evaluated in double precision
 * with exactly one rounding at every stored output, except that the FP8
 * quantiser takes its integer decisions (block exponent, code) on each
 * element's fp32 value, the precision the operator computes in.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it.  It shares
 * no code, header, table or helper with the GPU library and never calls it.
 *
 * Sources (cited by page title and section):
 *   [P1] FlagGems PR #5449 "[KMCompiler][Hygon] Token-tiled
 *        fused_deepseek_v4_qnorm_rope_kv_rope_quant_insert"
 *   [P2] FlagGems PR #5321 "[KMCompiler][MetaX][Hygon] Token-tiled
 *        fused_deepseek_v4_qnorm_rope_kv_rope_quant_insert, plus test and
 *        benchmark fixes"
 *   [P3] InfiniOps PR #1019 "FusedQkNormRope"
 *
 * The pages name the operator, its inputs and its outputs but never write it
 * down as formulas; every step below that the pages leave open is marked
 * "reading" and takes the plainest interpretation consistent with them.
 *
 * Every pointer is a host pointer owned by the caller.  bf16 values travel as
 * their raw 16-bit patterns (uint16_t).  No function allocates, and none
 * checks its preconditions beyond what is stated.
 *
 * Parity pins: every function here is pinned by the CPU test suite against
 * closed forms, library conversions or brute force; none is "parity unpinned"
 * except the exact bf16 values of random inputs beyond those properties.
 */
#ifndef FP8KV_ORACLE_H
#define FP8KV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats ---------------------------------------------------- */

/* Exact value of a bf16 bit pattern. */
double oracle_bf16_to_double(uint16_t bits);

/* bf16 bit pattern nearest to v, ties to even (one rounding from double). */
uint16_t oracle_bf16_rne(double v);

/* Exact value of an IEEE binary16 (fp16) bit pattern. */
double oracle_fp16_to_double(uint16_t bits);

/* fp16 bit pattern nearest to v, ties to even; overflow gives +-inf. */
uint16_t oracle_fp16_rne(double v);

/* Value of an OCP FP8 E4M3 ("fn": no infinities, 0x7F/0xFF are NaN) code.
 * NaN codes decode to NaN. */
double oracle_e4m3_decode(uint8_t code);

/* OCP E4M3 code nearest to v, ties to even, saturating at +-448, sign kept
 * (a negative value that rounds to zero gives 0x80).  This is the cache's
 * Triton fp8e4nv format that [P2] "The four test and benchmark fixes" names. */
uint8_t oracle_e4m3_encode(double v);

/* UE8M0 block exponent: the smallest integer e with amax <= 448 * 2^e, i.e.
 * e = ceil(log2(amax / 448)), clamped to [-127, 127]; amax == 0 gives -127
 * (reading: the closed form is undefined at zero and no epsilon is added).
 * amax must be >= 0 and finite.  The stored byte is e + 127. */
int32_t oracle_ue8m0_exponent(double amax);

/* ---- entry 1: fused DeepSeek-V4 attention prologue ----------------------- */
/*
 * fused_deepseek_v4_qnorm_rope_kv_rope_quant_insert ([P1], [P2]).
 *
 *   q             bf16 [T, H, 512], rewritten in place
 *   kv            bf16 [T, 512], the single latent KV head of each token
 *   q_weight      bf16 [512];  kv_weight bf16 [512]
 *   cos_sin_cache fp32 [max_position, 64]: row p = 32 cosines then 32 sines
 *   positions     int64 [T], 0 <= positions[t] < max_position (precondition)
 *   slot_mapping  int64 [T]; a negative slot, or one >= num_pages*64, skips
 *                 the cache write of that token (q is still rewritten)
 *   kv_cache      uint8 [num_pages, 64, 576]: 448 E4M3 codes of dims 0..447
 *                 then dims 448..511 as 64 little-endian bf16
 *   kv_scale      uint8 [num_pages, 64, 8]: bytes 0..6 = e_b + 127 for the
 *                 seven 64-dim quantisation blocks; byte 7 is never written
 *   eps           added to the mean square inside the square root
 * e_b and the codes E4M3(y_d 2^-e_b) are decided on fp32(y_d), each element
 * of the normalised, rotated KV row rounded to the nearest fp32 value.
 */
void oracle_qnorm_rope_kv_quant_insert(
    uint16_t* q, const uint16_t* kv, const uint16_t* q_weight,
    const uint16_t* kv_weight, const float* cos_sin_cache,
    const int64_t* positions, const int64_t* slot_mapping, uint8_t* kv_cache,
    uint8_t* kv_scale, int64_t num_tokens, int32_t num_heads,
    int64_t num_pages, double eps);

/*
 * The same prologue with the scalar-scale FP8 cache convention the pages set
 * against the blockwise one ([P1] "Performance": a single kv_cache_scale
 * float for the whole cache, with no room for an exponent per block).  q is
 * processed exactly as above; the KV row's dims 0..447 become
 * E4M3(fp32(fp32(y_d) / kv_cache_scale)) (nearest even, saturating at
 * +-448; the code decided in fp32 as in entry 1) and dims
 * 448..511 are stored as bf16 as before; no exponent bytes exist.
 * kv_cache_scale must be positive and finite.
 */
void oracle_qnorm_rope_kv_quant_insert_scalar(
    uint16_t* q, const uint16_t* kv, const uint16_t* q_weight,
    const uint16_t* kv_weight, const float* cos_sin_cache,
    const int64_t* positions, const int64_t* slot_mapping, uint8_t* kv_cache,
    float kv_cache_scale, int64_t num_tokens, int32_t num_heads,
    int64_t num_pages, double eps);

/* The KV head of each token after RMSNorm and rotation, before any rounding
 * (double [T, 512]): the values entry 1 quantises.  Exposed so that tests can
 * tell how close a block maximum sits to a power-of-two exponent boundary. */
void oracle_kv_normalised(const uint16_t* kv, const uint16_t* kv_weight,
                          const float* cos_sin_cache, const int64_t* positions,
                          int64_t num_tokens, double eps, double* y_out);

/* ---- the prologue as separate stages (an unfused pipeline) ---------------- */
/*
 * The same operator taken apart into the launches an unfused implementation
 * would make ([P1] "Performance": the baseline's two launches against one
 * fused launch; [P3] "Benchmark / Performance Impact": separate RmsNorm and
 * RotaryEmbedding calls).  Each stage reads and writes bf16, so the pipeline
 * rounds to bf16 between stages where the fused operator does not.
 *
 * oracle_rms_norm_rows: out[r, :] = bf16(x[r, :] / sqrt(mean(x^2) + eps) * w)
 *   for rows of 512; out may equal x.
 * oracle_rope_rows: in place on x [T, rows_per_token, 512]; the pairs
 *   (448 + 2i, 449 + 2i) of every row of token t rotate by cos_sin_cache row
 *   positions[t], result rounded to bf16; the other dims are not touched.
 * oracle_kv_quant_insert: kv [T, 512] holds bf16 values that are already
 *   normalised and rotated; quantise and insert them exactly as entry 1 does
 *   with its unrounded values (seven UE8M0 blocks over dims 0..447, dims
 *   448..511 copied as bf16).
 */
void oracle_rms_norm_rows(const uint16_t* x, const uint16_t* weight,
                          uint16_t* out, int64_t num_rows, double eps);
void oracle_rope_rows(uint16_t* x, const float* cos_sin_cache,
                      const int64_t* positions, int64_t num_tokens,
                      int32_t rows_per_token);
void oracle_kv_quant_insert(const uint16_t* kv, const int64_t* slot_mapping,
                            uint8_t* kv_cache, uint8_t* kv_scale,
                            int64_t num_tokens, int64_t num_pages);

/*
 * The packed Q/K operator taken apart as [P3] "Benchmark / Performance
 * Impact" measures it: RmsNorm of the Q heads and of the K heads into
 * separate, preallocated outputs, then RotaryEmbedding of each.
 *
 * oracle_rms_norm_heads: head h of token t starts at
 *   x + t * x_token_stride + h * head_dim (elements);
 *   out[t, h, :] = bf16(head / sqrt(mean(head^2) + eps) * weight), out
 *   contiguous [num_tokens, num_heads, head_dim].
 * oracle_rope_neox_heads: in place on x [num_tokens, num_heads, head_dim]:
 *   the NeoX pairs (i, i + head_dim/2) of every head of token t rotate by
 *   cos_sin_cache row positions[t] (fp32 [max_position, head_dim] = head_dim/2
 *   cosines then head_dim/2 sines), each result rounded to bf16.
 */
void oracle_rms_norm_heads(const uint16_t* x, int64_t x_token_stride,
                           const uint16_t* weight, uint16_t* out,
                           int64_t num_tokens, int32_t num_heads,
                           int32_t head_dim, double eps);
void oracle_rope_neox_heads(uint16_t* x, const float* cos_sin_cache,
                            const int64_t* positions, int64_t num_tokens,
                            int32_t num_heads, int32_t head_dim);

/* ---- read side of the cache ------------------------------------------------ */
/*
 * Gather rows of the paged FP8/UE8M0 cache by slot and dequantise them:
 *   out[i, d]       = E4M3(kv_cache[s, d]) * 2^(kv_scale[s, d / 64] - 127), d < 448
 *   out[i, 448 + j] = the stored bf16 rotary value j
 * with s = slots[i]; a negative slot or one >= num_pages * 64 gives a row of
 * +0.  out is bf16 [N, 512] (uint16 patterns), rounded to nearest even from
 * the exact double product (exact in practice: an E4M3 value has 4 significant
 * bits).  This is the inverse the fused prologue's cache layout implies
 * ([P1] "Performance": a power-of-two exponent for each of a token's seven
 * blocks).
 */
void oracle_kv_cache_gather_dequant(const uint8_t* kv_cache,
                                    const uint8_t* kv_scale,
                                    const int64_t* slots, int64_t num_rows,
                                    int64_t num_pages, uint16_t* out);

/*
 * The read side through block tables, as an attention consumer indexes the
 * cache: sequence s holds seq_lens[s] tokens, 64 to a page, in the pages
 * block_table[s * max_blocks_per_seq + 0, 1, ...] in order, so its token j
 * is slot block_table[s * max_blocks_per_seq + j / 64] * 64 + j % 64.  That
 * row, dequantised as by oracle_kv_cache_gather_dequant (a page id outside
 * [0, num_pages) gives a zero row), is written to out[out_offsets[s] + j].
 * Tokens j >= max_blocks_per_seq * 64 and rows outside [0, num_rows) are not
 * written; nor is any row of out no sequence covers.
 */
void oracle_kv_cache_gather_dequant_paged(
    const uint8_t* kv_cache, const uint8_t* kv_scale, int64_t num_pages,
    const int32_t* block_table, int32_t num_seqs, int32_t max_blocks_per_seq,
    const int32_t* seq_lens, const int64_t* out_offsets, int64_t num_rows,
    uint16_t* out);

/* Read side of the scalar-scale convention: out[i, d] =
 * bf16(E4M3(code[s, d]) * kv_cache_scale) for d < 448, rotary part copied,
 * invalid slots give +0 rows.  The product is rounded once from double. */
void oracle_kv_cache_gather_dequant_scalar(const uint8_t* kv_cache,
                                           float kv_cache_scale,
                                           const int64_t* slots,
                                           int64_t num_rows, int64_t num_pages,
                                           uint16_t* out);

/* The scalar-scale read side through block tables: the rows of
 * oracle_kv_cache_gather_dequant_paged (same walk over sequences, pages and
 * output rows), each dequantised as by oracle_kv_cache_gather_dequant_scalar. */
void oracle_kv_cache_gather_dequant_paged_scalar(
    const uint8_t* kv_cache, float kv_cache_scale, int64_t num_pages,
    const int32_t* block_table, int32_t num_seqs, int32_t max_blocks_per_seq,
    const int32_t* seq_lens, const int64_t* out_offsets, int64_t num_rows,
    uint16_t* out);

/* ---- entry 2: packed-QKV FusedQkNormRope ([P3] "Summary") ---------------- */
/*
 *   qkv           bf16 [T, (Hq + Hk + Hv) * D], Q and K heads rewritten in
 *                 place, the V heads neither read nor written
 *   q_weight      bf16 [D] applied to Q heads; k_weight bf16 [D] to K heads
 *   cos_sin_cache fp32 [max_position, D]: row p = D/2 cosines then D/2 sines
 *   position_ids  int64 [T], in range (precondition)
 * Per head: RMSNorm over D with its own weight per element, then NeoX RoPE
 * over the full head (pairs i, i + D/2), each element entering the rotation
 * with its own weight already applied.
 */
void oracle_qk_norm_rope_packed(
    uint16_t* qkv, int64_t num_tokens, int32_t num_heads_q,
    int32_t num_heads_k, int32_t num_heads_v, int32_t head_dim, double eps,
    const uint16_t* q_weight, const uint16_t* k_weight,
    const float* cos_sin_cache, const int64_t* position_ids);

/*
 * The packed operator beyond the page's guarded fast path ([P3] "Summary" and
 * "Notes for Reviewers": the first implementation is restricted to bf16,
 * head_dim 128, full-dimension NeoX RoPE).  Here:
 *   head_dim      any even D
 *   rotary_dim    R, even, R <= D: only dims [0, R) of a head rotate (partial
 *                 rotary); dims [R, D) are normalised and weighted only
 *   is_neox       1: pairs (i, i + R/2); 0: interleaved pairs (2i, 2i + 1);
 *                 i < R/2 in both, rotated by cos_i, sin_i
 *   is_fp16       0: qkv and both weights are bf16; 1: all three are fp16
 *   cos_sin_cache fp32 [max_position, R] = R/2 cosines then R/2 sines
 * With D = R = 128, is_neox = 1, is_fp16 = 0 this is oracle_qk_norm_rope_packed.
 */
void oracle_qk_norm_rope_packed_ex(
    uint16_t* qkv, int64_t num_tokens, int32_t num_heads_q,
    int32_t num_heads_k, int32_t num_heads_v, int32_t head_dim,
    int32_t rotary_dim, int32_t is_neox, int32_t is_fp16, double eps,
    const uint16_t* q_weight, const uint16_t* k_weight,
    const float* cos_sin_cache, const int64_t* position_ids);

#ifdef __cplusplus
}
#endif

#endif /* FP8KV_ORACLE_H */
