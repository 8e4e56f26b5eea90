"""The oracle's pins catch plausible mistakes: each case below plants one
mistake in a copy of oracle/oracle.cpp (a dropped term, a wrong sign, index,
bias or rounding, a transposed operand, an off-by-one bound), builds that copy
into a library of its own, and runs every oracle pin test
(tests/test_oracle_*.py) against it in a fresh process.  A mutant is killed
when the pins report a test failure; a mutant that passes them, or that
crashes instead of failing, fails this test.  The unmutated source built the
same way must pass.  Runs on the CPU only; the oracle source in the tree is
never modified."""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.cpp")
# test_oracle_sanitized.py builds the tree's own oracle source, not a mutant,
# so it is not one of the pins run against each mutant.
PIN_FILES = sorted(os.path.relpath(p, ROOT) for p in
                   glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py"))
                   if not p.endswith(("test_oracle_mutations.py",
                                      "test_oracle_sanitized.py")))

# (name, text in oracle.cpp, replacement); each text occurs exactly once.
MUTATIONS = [
    # number formats
    ("bf16_precision", "int lsb_exp = (k - 1) - 7;", "int lsb_exp = (k - 1) - 8;"),
    ("bf16_truncates",
     "    r = round_to_quantum(a, std::ldexp(1.0, lsb_exp));\n  }\n"
     "  uint16_t sign = std::signbit(v) ? 0x8000 : 0;",
     "    r = std::floor(a / std::ldexp(1.0, lsb_exp)) * std::ldexp(1.0, lsb_exp);\n"
     "  }\n  uint16_t sign = std::signbit(v) ? 0x8000 : 0;"),
    ("fp16_precision", "const int lsb_exp = (top < -14 ? -14 : top) - 10;",
     "const int lsb_exp = (top < -14 ? -14 : top) - 11;"),
    ("e4m3_subnormal_quantum", "int lsb_exp = (top < -6 ? -6 : top) - 3;",
     "int lsb_exp = (top < -7 ? -7 : top) - 3;"),
    ("e4m3_saturates_late", "if (r > kE4M3Max) r = kE4M3Max;",
     "if (r > 480.0) r = 480.0;"),
    ("e4m3_sign_of_zero", "uint8_t sign = std::signbit(v) ? 0x80 : 0x00;",
     "uint8_t sign = v < 0.0 ? 0x80 : 0x00;"),
    ("e4m3_decode_subnormal", "? std::ldexp(static_cast<double>(mant), -9)",
     "? std::ldexp(static_cast<double>(mant), -10)"),
    ("ue8m0_boundary", "int e = k - 9 + (m > 0.875 ? 1 : 0);",
     "int e = k - 9 + (m >= 0.875 ? 1 : 0);"),
    ("ue8m0_offset", "int e = k - 9 + (m > 0.875 ? 1 : 0);",
     "int e = k - 8 + (m > 0.875 ? 1 : 0);"),
    ("ue8m0_no_low_clamp", "if (e < -127) e = -127;", ""),
    ("ue8m0_clamp_one_high", "if (e < -127) e = -127;",
     "if (e < -126) e = -126;"),
    ("fp32_decision_flushes_subnormals",
     "  return static_cast<double>(static_cast<float>(v));",
     "  const float f = static_cast<float>(v);\n"
     "  return std::fpclassify(f) == FP_SUBNORMAL ? 0.0 : static_cast<double>(f);"),
    # RMSNorm
    ("rms_eps_outside_root", "double inv_rms = 1.0 / std::sqrt(mean_sq + eps);",
     "double inv_rms = 1.0 / (std::sqrt(mean_sq) + eps);"),
    ("rms_mean_over_448", "double mean_sq = sum_sq / n;",
     "double mean_sq = sum_sq / (n - n / 8);"),
    ("rms_no_weight",
     "y[d] = oracle_bf16_to_double(x[d]) * inv_rms * oracle_bf16_to_double(w[d]);",
     "y[d] = oracle_bf16_to_double(x[d]) * inv_rms;"),
    # rotation
    ("rope_sign", "*a = a0 * c - b0 * s;", "*a = a0 * c + b0 * s;"),
    ("rope_cos_sin_swapped",
     "    const float* cosv = row;\n    const float* sinv = row + kRopeDim / 2;\n\n    // Q:",
     "    const float* cosv = row + kRopeDim / 2;\n    const float* sinv = row;\n\n    // Q:"),
    ("rope_neox_instead_of_interleaved",
     "        rotate_pair(&y[kRopeStart + 2 * i], &y[kRopeStart + 2 * i + 1],\n"
     "                    cosv[i], sinv[i]);\n"
     "      for (int d = 0; d < kHeadDim; ++d) qh[d] = oracle_bf16_rne(y[d]);\n"
     "    }\n\n    // KV",
     "        rotate_pair(&y[kRopeStart + i], &y[kRopeStart + i + kRopeDim / 2],\n"
     "                    cosv[i], sinv[i]);\n"
     "      for (int d = 0; d < kHeadDim; ++d) qh[d] = oracle_bf16_rne(y[d]);\n"
     "    }\n\n    // KV"),
    ("rope_position_row",
     "    const float* row = cos_sin_cache + positions[t] * kRopeDim;\n"
     "    const float* cosv = row;\n    const float* sinv = row + kRopeDim / 2;\n\n    // Q:",
     "    const float* row = cos_sin_cache + positions[t] * (kRopeDim / 2);\n"
     "    const float* cosv = row;\n    const float* sinv = row + kRopeDim / 2;\n\n    // Q:"),
    ("q_uses_kv_weight",
     "      rms_norm(qh, q_weight, kHeadDim, eps, y);\n"
     "      for (int i = 0; i < kRopeDim / 2; ++i)\n"
     "        rotate_pair(&y[kRopeStart + 2 * i], &y[kRopeStart + 2 * i + 1],\n"
     "                    cosv[i], sinv[i]);\n"
     "      for (int d = 0; d < kHeadDim; ++d) qh[d] = oracle_bf16_rne(y[d]);\n"
     "    }\n\n    // KV",
     "      rms_norm(qh, kv_weight, kHeadDim, eps, y);\n"
     "      for (int i = 0; i < kRopeDim / 2; ++i)\n"
     "        rotate_pair(&y[kRopeStart + 2 * i], &y[kRopeStart + 2 * i + 1],\n"
     "                    cosv[i], sinv[i]);\n"
     "      for (int d = 0; d < kHeadDim; ++d) qh[d] = oracle_bf16_rne(y[d]);\n"
     "    }\n\n    // KV"),
    ("kv_not_rotated",
     "  rms_norm(x, w, kHeadDim, eps, y);\n  for (int i = 0; i < kRopeDim / 2; ++i)",
     "  rms_norm(x, w, kHeadDim, eps, y);\n  for (int i = 0; i < 0; ++i)"),
    # quantise + insert
    ("quant_half_block_amax",
     "    for (int d = b * kQuantBlock; d < (b + 1) * kQuantBlock; ++d)\n"
     "      amax = std::fmax(amax, std::fabs(yf[d]));",
     "    for (int d = b * kQuantBlock; d < b * kQuantBlock + kQuantBlock / 2; ++d)\n"
     "      amax = std::fmax(amax, std::fabs(yf[d]));"),
    ("quant_byte_bias", "scale[b] = static_cast<uint8_t>(e + 127);",
     "scale[b] = static_cast<uint8_t>(e + 128);"),
    ("quant_scale_direction", "dst[d] = oracle_e4m3_encode(std::ldexp(yf[d], -e));",
     "dst[d] = oracle_e4m3_encode(std::ldexp(yf[d], e));"),
    ("quant_decides_in_double", "yf[d] = to_fp32(y[d]);", "yf[d] = y[d];"),
    ("rope_bytes_big_endian",
     "    uint16_t bits = oracle_bf16_rne(y[kRopeStart + j]);\n"
     "    dst[kRopeStart + 2 * j] = static_cast<uint8_t>(bits & 0xFF);\n"
     "    dst[kRopeStart + 2 * j + 1] = static_cast<uint8_t>(bits >> 8);\n"
     "  }\n}\n\n// The walk of the read side",
     "    uint16_t bits = oracle_bf16_rne(y[kRopeStart + j]);\n"
     "    dst[kRopeStart + 2 * j + 1] = static_cast<uint8_t>(bits & 0xFF);\n"
     "    dst[kRopeStart + 2 * j] = static_cast<uint8_t>(bits >> 8);\n"
     "  }\n}\n\n// The walk of the read side"),
    ("slot_bound_off_by_one",
     "if (slot < 0 || slot >= num_slots) continue;  // skipped token",
     "if (slot < 0 || slot >= num_slots - 1) continue;  // skipped token"),
    ("scalar_scale_multiplies",
     "to_fp32(to_fp32(y[d]) / static_cast<double>(kv_cache_scale))",
     "to_fp32(to_fp32(y[d]) * static_cast<double>(kv_cache_scale))"),
    ("scalar_decides_in_double",
     "to_fp32(to_fp32(y[d]) / static_cast<double>(kv_cache_scale))",
     "y[d] / static_cast<double>(kv_cache_scale)"),
    # separate stages
    ("rms_rows_wrong_row", "rms_norm(x + r * kHeadDim, weight, kHeadDim, eps, y);",
     "rms_norm(x, weight, kHeadDim, eps, y);"),
    ("rope_rows_pair_swapped", "rotate_pair(&a, &b, row[i], row[kRopeDim / 2 + i]);",
     "rotate_pair(&b, &a, row[i], row[kRopeDim / 2 + i]);"),
    # read side
    ("dequant_block_index",
     "const int e = static_cast<int>(scale[d / kQuantBlock]) - 127;",
     "const int e = static_cast<int>(scale[d / kQuantBlock + (d >= kQuantBlock ? 0 : 1)]) - 127;"),
    ("dequant_bias", "const int e = static_cast<int>(scale[d / kQuantBlock]) - 127;",
     "const int e = static_cast<int>(scale[d / kQuantBlock]) - 126;"),
    ("paged_offset_in_page", "page * kPageSize + j % kPageSize;",
     "page * kPageSize + (j + 1) % kPageSize;"),
    ("paged_length_cap",
     "for (int64_t j = 0; j < len && j < int64_t{max_blocks_per_seq} * kPageSize; ++j) {",
     "for (int64_t j = 0; j <= len && j < int64_t{max_blocks_per_seq} * kPageSize; ++j) {"),
    # packed Q/K norm + RoPE
    ("packed_interleaved_pairs",
     "for (int i = 0; i < half; ++i) rotate_pair(&y[i], &y[i + half], cosv[i], sinv[i]);",
     "for (int i = 0; i < half; ++i) rotate_pair(&y[2 * i], &y[2 * i + 1], cosv[i], sinv[i]);"),
    ("packed_weight_boundary",
     "      const uint16_t* w = h < num_heads_q ? q_weight : k_weight;\n"
     "      rms_norm(xh, w, head_dim, eps, y);",
     "      const uint16_t* w = h <= num_heads_q ? q_weight : k_weight;\n"
     "      rms_norm(xh, w, head_dim, eps, y);"),
    ("packed_ex_mean_over_rotary",
     "const double inv_rms = 1.0 / std::sqrt(sum_sq / head_dim + eps);",
     "const double inv_rms = 1.0 / std::sqrt(sum_sq / (rotary_dim > 0 ? rotary_dim : head_dim) + eps);"),
    ("packed_ex_interleaved_cos_sin",
     "rotate_pair(&y[2 * i], &y[2 * i + 1], row[i], row[half + i]);",
     "rotate_pair(&y[2 * i], &y[2 * i + 1], row[half + i], row[i]);"),
    ("packed_ex_fp16_weight_as_bf16", "y[d] = decode(xh[d]) * inv_rms * decode(w[d]);",
     "y[d] = decode(xh[d]) * inv_rms * oracle_bf16_to_double(w[d]);"),
    ("packed_ex_partial_rotary_short",
     "      for (int i = 0; i < half; ++i) {\n        if (is_neox)",
     "      for (int i = 0; i < half - 1; ++i) {\n        if (is_neox)"),
    ("packed_sin_offset", "    const float* sinv = row + half;",
     "    const float* sinv = row + half - 1;"),
    # decoders
    ("bf16_decode_shift", "uint32_t u = static_cast<uint32_t>(bits) << 16;",
     "uint32_t u = static_cast<uint32_t>(bits) << 15;"),
    ("fp16_decode_subnormal", "mag = std::ldexp(static_cast<double>(mant), -24);",
     "mag = std::ldexp(static_cast<double>(mant), -25);"),
    ("fp16_decode_bias", "mag = std::ldexp(1.0 + mant / 1024.0, exp_field - 15);",
     "mag = std::ldexp(1.0 + mant / 1024.0, exp_field - 14);"),
    ("e4m3_decode_no_nan", "if (exp_field == 0xF && mant == 0x7) return std::nan(\"\");", ""),
    ("e4m3_encode_bias",
     "int exp_field = (k - 1) + 7;\n    int mant = static_cast<int>((2.0 * m - 1.0) * 8.0);",
     "int exp_field = (k - 1) + 8;\n    int mant = static_cast<int>((2.0 * m - 1.0) * 8.0);"),
    # scalar-scale convention
    ("scalar_read_divides",
     "dst[d] = oracle_bf16_rne(oracle_e4m3_decode(row[d]) *\n"
     "                               static_cast<double>(kv_cache_scale));",
     "dst[d] = oracle_bf16_rne(oracle_e4m3_decode(row[d]) /\n"
     "                               static_cast<double>(kv_cache_scale));"),
    ("scalar_read_rope_bytes_swapped",
     "          row[kRopeStart + 2 * j] | (row[kRopeStart + 2 * j + 1] << 8));\n  }\n}\n\n"
     "void oracle_rms_norm_rows",
     "          row[kRopeStart + 2 * j + 1] | (row[kRopeStart + 2 * j] << 8));\n  }\n}\n\n"
     "void oracle_rms_norm_rows"),
    ("scalar_q_uses_kv_weight",
     "      rms_norm(qh, q_weight, kHeadDim, eps, y);\n"
     "      for (int i = 0; i < kRopeDim / 2; ++i)\n"
     "        rotate_pair(&y[kRopeStart + 2 * i], &y[kRopeStart + 2 * i + 1],\n"
     "                    cosv[i], sinv[i]);\n"
     "      for (int d = 0; d < kHeadDim; ++d) qh[d] = oracle_bf16_rne(y[d]);\n"
     "    }\n    const int64_t slot",
     "      rms_norm(qh, kv_weight, kHeadDim, eps, y);\n"
     "      for (int i = 0; i < kRopeDim / 2; ++i)\n"
     "        rotate_pair(&y[kRopeStart + 2 * i], &y[kRopeStart + 2 * i + 1],\n"
     "                    cosv[i], sinv[i]);\n"
     "      for (int d = 0; d < kHeadDim; ++d) qh[d] = oracle_bf16_rne(y[d]);\n"
     "    }\n    const int64_t slot"),
    ("scalar_drops_sign",
     "to_fp32(to_fp32(y[d]) / static_cast<double>(kv_cache_scale))",
     "to_fp32(to_fp32(std::fabs(y[d])) / static_cast<double>(kv_cache_scale))"),
    # read side through block tables, unrounded KV, separate quantiser
    ("paged_page_zero_invalid",
     "const int64_t slot = page < 0 || page >= num_pages ? -1 : page * kPageSize + j % kPageSize;",
     "const int64_t slot = page <= 0 || page >= num_pages ? -1 : page * kPageSize + j % kPageSize;"),
    ("paged_row_bound", "if (row < 0 || row >= num_rows) continue;",
     "if (row < 0 || row >= num_rows - 1) continue;"),
    ("kv_normalised_eps_dropped",
     "    kv_head(kv + t * kHeadDim, kv_weight, row, row + kRopeDim / 2, eps,\n"
     "            y_out + t * kHeadDim);",
     "    kv_head(kv + t * kHeadDim, kv_weight, row, row + kRopeDim / 2, 0.0,\n"
     "            y_out + t * kHeadDim);"),
    ("scalar_paged_scale_doubled",
     "                           kv_cache, kv_cache_scale, &slot, 1, num_pages,",
     "                           kv_cache, 2.0f * kv_cache_scale, &slot, 1, num_pages,"),
    ("rms_norm_heads_token_stride",
     "      rms_norm(x + t * x_token_stride + static_cast<int64_t>(h) * head_dim,",
     "      rms_norm(x + t * num_heads * head_dim + static_cast<int64_t>(h) * head_dim,"),
    ("rope_neox_heads_sine_sign",
     "        rotate_pair(&a, &b, row[i], row[half + i]);\n        xh[i] = oracle_bf16_rne(a);",
     "        rotate_pair(&a, &b, row[i], -row[half + i]);\n        xh[i] = oracle_bf16_rne(a);"),
    ("rope_neox_heads_interleaved",
     "        double a = oracle_bf16_to_double(xh[i]);\n"
     "        double b = oracle_bf16_to_double(xh[i + half]);",
     "        double a = oracle_bf16_to_double(xh[2 * i]);\n"
     "        double b = oracle_bf16_to_double(xh[2 * i + 1]);"),
    ("q_not_rotated",
     "      for (int i = 0; i < kRopeDim / 2; ++i)\n"
     "        rotate_pair(&y[kRopeStart + 2 * i], &y[kRopeStart + 2 * i + 1],\n"
     "                    cosv[i], sinv[i]);\n"
     "      for (int d = 0; d < kHeadDim; ++d) qh[d] = oracle_bf16_rne(y[d]);\n"
     "    }\n\n    // KV",
     "      for (int i = 0; i < 0; ++i)\n"
     "        rotate_pair(&y[kRopeStart + 2 * i], &y[kRopeStart + 2 * i + 1],\n"
     "                    cosv[i], sinv[i]);\n"
     "      for (int d = 0; d < kHeadDim; ++d) qh[d] = oracle_bf16_rne(y[d]);\n"
     "    }\n\n    // KV"),
    ("skipped_token_skips_q",
     "    const float* sinv = row + kRopeDim / 2;\n\n    // Q:",
     "    const float* sinv = row + kRopeDim / 2;\n    if (slot_mapping[t] < 0) continue;\n\n    // Q:"),
    ("packed_normalises_v",
     "    for (int32_t h = 0; h < num_heads_q + num_heads_k; ++h) {\n"
     "      uint16_t* xh = qkv + t * row_elems + static_cast<int64_t>(h) * head_dim;\n"
     "      const uint16_t* w = h < num_heads_q ? q_weight : k_weight;\n"
     "      rms_norm(xh, w, head_dim, eps, y);",
     "    for (int32_t h = 0; h < num_heads_q + num_heads_k + num_heads_v; ++h) {\n"
     "      uint16_t* xh = qkv + t * row_elems + static_cast<int64_t>(h) * head_dim;\n"
     "      const uint16_t* w = h < num_heads_q ? q_weight : k_weight;\n"
     "      rms_norm(xh, w, head_dim, eps, y);"),
    ("packed_ex_normalises_v",
     "    for (int32_t h = 0; h < num_heads_q + num_heads_k; ++h) {\n"
     "      uint16_t* xh = qkv + t * row_elems + static_cast<int64_t>(h) * head_dim;\n"
     "      const uint16_t* w = h < num_heads_q ? q_weight : k_weight;\n"
     "      // RMSNorm over the whole head",
     "    for (int32_t h = 0; h < num_heads_q + num_heads_k + num_heads_v; ++h) {\n"
     "      uint16_t* xh = qkv + t * row_elems + static_cast<int64_t>(h) * head_dim;\n"
     "      const uint16_t* w = h < num_heads_q ? q_weight : k_weight;\n"
     "      // RMSNorm over the whole head"),
    ("packed_ex_fp16_output_as_bf16",
     "    return is_fp16 ? oracle_fp16_rne(v) : oracle_bf16_rne(v);",
     "    return oracle_bf16_rne(v);"),
    ("dequant_invalid_row_kept",
     "    for (int d = 0; d < kHeadDim; ++d) dst[d] = 0;\n    return;",
     "    return;"),
    ("scalar_dequant_invalid_row_kept",
     "      for (int d = 0; d < kHeadDim; ++d) dst[d] = 0;\n      continue;",
     "      continue;"),
    ("paged_invalid_page_row_skipped",
     "      row_fn(slot, row);",
     "      if (slot >= 0) row_fn(slot, row);"),
    ("quant_insert_stage_bound",
     "    if (slot < 0 || slot >= num_slots) continue;\n    for (int d = 0; d < kHeadDim; ++d) y[d]",
     "    if (slot < 0 || slot >= num_slots - 1) continue;\n    for (int d = 0; d < kHeadDim; ++d) y[d]"),
]

# Runs the pin tests in a fresh interpreter with the oracle package pointed at
# the library named by argv[1]; exits with pytest's status.
RUNNER = (
    "import sys, oracle\n"
    "oracle.LIB_PATH = sys.argv[1]\n"
    "import pytest\n"
    "sys.exit(pytest.main(['-x', '-q', '-m', 'not gpu', '-p', 'no:cacheprovider',"
    " *sys.argv[2:]]))\n")


def _run_pins(lib: str) -> subprocess.CompletedProcess:
    return subprocess.run([sys.executable, "-c", RUNNER, lib, *PIN_FILES],
                          cwd=ROOT, capture_output=True, text=True, timeout=600)


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    """Build the control and every mutant, run the pins against each, with a
    few processes at a time; returns {name: CompletedProcess}."""
    with open(SRC) as f:
        source = f.read()
    work = tmp_path_factory.mktemp("oracle_mutants")

    def one(item):
        name, old, new = item
        assert source.count(old) == 1, f"{name}: text not found exactly once"
        src = os.path.join(work, f"{name}.cpp")
        with open(src, "w") as f:
            f.write(source.replace(old, new))
        lib = obuild.build(src, os.path.join(work, f"lib{name}.so"))
        return name, _run_pins(lib)

    jobs = [("control", "", "")] + MUTATIONS
    workers = max(1, min(8, (os.cpu_count() or 2) // 2))
    with cf.ThreadPoolExecutor(workers) as ex:
        return dict(ex.map(lambda m: one(m) if m[0] != "control" else
                           ("control", _run_pins(obuild.build(
                               SRC, os.path.join(work, "libcontrol.so")))), jobs))


def test_unmutated_oracle_passes_its_pins(outcomes):
    r = outcomes["control"]
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name", [m[0] for m in MUTATIONS])
def test_pins_kill_mutant(outcomes, name):
    r = outcomes[name]
    # 1 = some test failed; anything else (0 = all passed, a signal, an
    # internal error) means the pins did not catch the mistake cleanly
    assert r.returncode == 1, (f"mutant {name}: pytest exited {r.returncode}\n"
                               + r.stdout[-1500:] + r.stderr[-1500:])
