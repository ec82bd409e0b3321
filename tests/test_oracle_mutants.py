"""Plant plausible mistakes in copies of the oracle source (on the CPU) and
show that each one fails at least one pin from pins.py.  The real oracle is
never modified; each mutant is compiled into a temporary directory."""
import os

import pytest

import oracle
import pins

# (id, text in fp8_oracle.c, replacement): a dropped term, a wrong sign or
# index, a transposed operand, a wrong rounding or guard rule
MUTANTS = [
    ("rne_ties_away", "if (rem > half || (rem == half && (k & 1))) k += 1;",
     "if (rem >= half) k += 1;"),
    ("rne_truncate", "if (rem > half || (rem == half && (k & 1))) k += 1;", "(void)half; (void)rem;"),
    ("no_saturation", "if (code > d.max_code) code = d.max_code;", "if (code > 0x7F) code = 0x7F;"),
    ("subnormal_emin_off_by_one", "int64_t code = round_magnitude(u, d.mbits, 1 - d.bias, d.bias);",
     "int64_t code = round_magnitude(u, d.mbits, 2 - d.bias, d.bias);"),
    ("lost_negative_zero", "if (ef == 0 && mf == 0) return sbit;\n    int64_t code = round_magnitude(u, d.mbits",
     "if (ef == 0 && mf == 0) return 0;\n    int64_t code = round_magnitude(u, d.mbits"),
    ("decode_bias_wrong", ": ldexp((double)((1 << d.mbits) + m), E - d.bias - d.mbits);",
     ": ldexp((double)((1 << d.mbits) + m), E - d.bias - d.mbits + 1);"),
    ("bf16_truncates", "if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1;", "(void)lower;"),
    ("group_scale_inv_is_reciprocal", "scale_inv[r * groups + g] = amax / fmax;",
     "scale_inv[r * groups + g] = 1.0f / scale;"),
    ("channel_scale_inv_is_reciprocal", "scale_inv[r] = a / fmax;", "scale_inv[r] = 1.0f / scale;"),
    ("tensor_scale_inv_is_amax_over_max", "*scale_inv = 1.0f / s;", "*scale_inv = a / oracle_fp8_max(fmt);"),
    ("group_clamp_dropped", "if (amax < clamp_min) amax = clamp_min;", "(void)clamp_min;"),
    ("tensor_zero_guard_dropped", "float a = (amax > 0.0f) ? amax : 1.0f;\n    float s = oracle_fp8_max(fmt) / a;",
     "float a = amax;\n    float s = oracle_fp8_max(fmt) / a;"),
    ("scale_transposed", "float scale = fmax / amax;", "float scale = amax / fmax;"),
    ("amax_drops_nan", "if (isnan(a)) saw_nan = 1;", "if (isnan(a)) continue;"),
    ("amax_signed_max", "float a = fabsf(load_elem(x, dtype, i));", "float a = load_elem(x, dtype, i);"),
    ("block_index_transposed", "scale_inv[(i / 128) * nb + j / 128]", "scale_inv[(j / 128) * nb + i / 128]"),
    ("group_dequant_index", "scale_inv[r * groups + c / 128]", "scale_inv[r * groups + c % groups]"),
    ("channel_dequant_uses_col", "oracle_fp8_decode(q[r * cols + c], fmt) * scale_inv[r]);",
     "oracle_fp8_decode(q[r * cols + c], fmt) * scale_inv[c % rows]);"),
    ("f16_overflow_saturates", "if (code >= 0x7C00) code = 0x7C00;", "if (code >= 0x7C00) code = 0x7BFF;"),
    ("empty_channel_scale", "if (cols == 0) { scale_inv[r] = 1.0f; continue; }",
     "if (cols == 0) { scale_inv[r] = 0.0f; continue; }"),
    ("sum_in_f32_round_once", "            acc = round_to(acc + term, ydtype);", "            acc = acc + term;"),
    ("sum_term_unrounded", "float term = round_to(oracle_fp8_decode(q[w * n + i], fmt) * scale_inv[w], ydtype);",
     "float term = oracle_fp8_decode(q[w * n + i], fmt) * scale_inv[w];"),
    ("sum_starts_from_first_term", "        float acc = 0.0f;\n        for (int64_t w = 0; w < W; ++w) {",
     "        float acc = -0.0f;\n        for (int64_t w = 0; w < W; ++w) {"),
    ("average_by_reciprocal", "if (average) acc = round_to(acc / (float)W, ydtype);",
     "if (average) acc = round_to(acc * (1.0f / (float)W), ydtype);"),
    ("fsdp_dequant_by_reciprocal", "store_elem(y, ydtype, i, oracle_fp8_decode(q[i], fmt) / scale);",
     "store_elem(y, ydtype, i, oracle_fp8_decode(q[i], fmt) * (1.0f / scale));"),
    ("fsdp_guard_dropped", "    return (amax > 0.0f) ? amax : 1.0f;\n}", "    return amax;\n}"),
    ("sum_reversed_order", "float term = round_to(oracle_fp8_decode(q[w * n + i], fmt) * scale_inv[w], ydtype);",
     "float term = round_to(oracle_fp8_decode(q[(W - 1 - w) * n + i], fmt) * scale_inv[W - 1 - w], ydtype);"),
    ("pipeline_threshold_inclusive", "int fmt = (amax > oracle_fp8_max(ORC_E4M3FN)) ? ORC_E5M2 : ORC_E4M3FN;",
     "int fmt = (amax >= oracle_fp8_max(ORC_E4M3FN)) ? ORC_E5M2 : ORC_E4M3FN;"),
    ("pipeline_guard_positive", "float scale = (amax == 0.0f) ? 1.0f : oracle_fp8_max(fmt) / amax;",
     "float scale = (amax > 0.0f) ? oracle_fp8_max(fmt) / amax : 1.0f;"),
    ("pipeline_scale_e4m3_max", "float scale = (amax == 0.0f) ? 1.0f : oracle_fp8_max(fmt) / amax;",
     "float scale = (amax == 0.0f) ? 1.0f : oracle_fp8_max(ORC_E4M3FN) / amax;"),
    ("pipeline_amax_from_max_only", "float amax = saw_nan ? NAN : (fabsf(lo) > fabsf(hi) ? fabsf(lo) : fabsf(hi));",
     "float amax = saw_nan ? NAN : fabsf(hi);"),
    ("pipeline_scale_inv_is_amax_over_max", "    *scale_inv = 1.0f / scale;\n    *fmt_out = fmt;",
     "    *scale_inv = amax / oracle_fp8_max(fmt);\n    *fmt_out = fmt;"),
    ("pipeline_dequant_scale_rounded", "round_to(oracle_fp8_decode(q[i], fmt), ydtype) * scale_inv);",
     "round_to(oracle_fp8_decode(q[i], fmt), ydtype) * round_to(scale_inv, ydtype));"),
    ("packed_header_after_payload",
     "int rc = oracle_cast_per_tensor(x, dtype, n, fmt, slot + 4, &scale_inv);\n    if (rc != 0) return rc;\n"
     "    memcpy(slot, &scale_inv, 4);",
     "int rc = oracle_cast_per_tensor(x, dtype, n, fmt, slot, &scale_inv);\n    if (rc != 0) return rc;\n"
     "    memcpy(slot + n, &scale_inv, 4);"),
    ("packed_slot_stride_without_header", "const uint8_t* slot = slots + w * (4 + n);",
     "const uint8_t* slot = slots + w * n;"),
    ("packed_header_read_as_scale", "oracle_fp8_decode(slot[4 + i], fmt) * scale_inv);",
     "oracle_fp8_decode(slot[4 + i], fmt) / scale_inv);"),
    ("packed_output_row_dropped", "store_elem(y, ydtype, w * n + i,", "store_elem(y, ydtype, i,"),
]


@pytest.mark.parametrize("mid,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, mid, old, new):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {mid} must occur exactly once"
    msrc = tmp_path / "fp8_oracle.c"
    msrc.write_text(src.replace(old, new))
    lib = oracle.build(force=True, src=str(msrc), out=str(tmp_path / "libmutant.so"))
    L = oracle.OracleLib(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(L)
        except Exception as e:  # noqa: BLE001  (any failure of a pin counts as caught)
            failed.append((pin.__name__, type(e).__name__))
            break                # caught: the remaining pins need not run
    assert failed, f"mutant {mid} passed every pin"
