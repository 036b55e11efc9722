"""Plant plausible mistakes in copies of the oracle and check the pins catch each.

Every mutation rewrites one expression of ``oracle/moe_oracle.c`` (a dropped
term, a wrong index or operand, a bf16 accumulator, a wrong rounding mode, a
misplaced epsilon ...), compiles the copy with gcc into a temporary folder and
runs the whole pin battery against it.  The unmodified oracle passes every
pin; each mutant must fail at least one.  Mutations are chosen to stay inside
the buffers, so a broken copy can only compute wrong values.
"""
import os

import pytest

import oracle
import pins

# (name, anchor text, replacement[, which occurrence of the anchor]); the
# per-copy dispatch comes before the per-region one in the source, so shared
# anchors name the per-copy code with occurrence 0 and the per-region code
# with occurrence 1.
MUTATIONS = [
    # combine
    ("drop_last_term",
     "for (int64_t j = 0; j < k; ++j) {\n        int32_t row = slot_index[t * k + j];",
     "for (int64_t j = 0; j < k - 1; ++j) {\n        int32_t row = slot_index[t * k + j];"),
    ("bf16_accumulator",
     "acc = acc + v;",
     "acc = oracle_bf16_to_f32(oracle_f32_to_bf16(acc + v));"),
    ("bf16_accumulator_weighted",
     "acc = fmaf(w[t * k + j], v, acc);",
     "acc = oracle_bf16_to_f32(oracle_f32_to_bf16(fmaf(w[t * k + j], v, acc)));"),
    ("gates_ignored",
     "acc = fmaf(w[t * k + j], v, acc);",
     "acc = fmaf(1.0f, v, acc);"),
    ("gates_reversed",
     "acc = fmaf(w[t * k + j], v, acc);",
     "acc = fmaf(w[t * k + (k - 1 - j)], v, acc);"),
    ("subtract_term",
     "acc = acc + v;",
     "acc = acc - v;"),
    ("weighted_sum_reduced_twice",
     "acc = fmaf(w[t * k + j], v, acc);",
     "acc = fmaf(w[t * k + j], v, acc) + fmaf(w[t * k + j], v, 0.0f) * (j == k - 1);"),
    # codec
    ("truncate_instead_of_round",
     "double q = nearbyint(ldexp(a, -qexp));",
     "double q = floor(ldexp(a, -qexp));"),
    ("ties_away_from_zero",
     "double q = nearbyint(ldexp(a, -qexp));",
     "double q = round(ldexp(a, -qexp));"),
    ("no_subnormal_floor",
     "if (qexp < -133)\n        qexp = -133;",
     "if (qexp < -160)\n        qexp = -160;"),
    ("decode_wrong_shift",
     "uint32_t bits = (uint32_t)h << 16;",
     "uint32_t bits = (uint32_t)h << 15;"),
    # dispatch
    ("copy_region_by_modulo",
     "int64_t r = e / epr;",
     "int64_t r = e % ep;"),
    ("src_index_holds_token",
     "src_index[row] = (int32_t)f;",
     "src_index[row] = (int32_t)(f / k);"),
    ("copy_wrong_row",
     "memcpy(ws + row * H, x + (f / k) * H, (size_t)H * sizeof(uint16_t));",
     "memcpy(ws + row * H, x + (f % k) * H, (size_t)H * sizeof(uint16_t));"),
    ("rows_fill_from_the_end",
     "int64_t row = r * cap + s;",
     "int64_t row = r * cap + (cap - 1 - s);"),
    ("all_negative_ids_silent",
     "if (e == -1)\n            continue;",
     "if (e < 0)\n            continue;"),
    ("counts_clamped",
     "status |= ORACLE_STATUS_OVERFLOW;",
     "status |= ORACLE_STATUS_OVERFLOW; counts[r] -= 1;"),
    # fused epilogue
    ("eps_outside_sqrt",
     "double inv = 1.0 / sqrt(sumsq / (double)H + (double)eps);",
     "double inv = 1.0 / (sqrt(sumsq / (double)H) + (double)eps);"),
    ("sum_not_mean",
     "double inv = 1.0 / sqrt(sumsq / (double)H + (double)eps);",
     "double inv = 1.0 / sqrt(sumsq + (double)eps);"),
    ("gamma_dropped",
     "double n = (double)s_scratch[h] * inv * (double)oracle_bf16_to_f32(gamma[h]);",
     "double n = (double)s_scratch[h] * inv;"),
    ("residual_not_added",
     "float s = acc + oracle_bf16_to_f32(residual[t * H + h]);",
     "float s = acc;"),
    ("residual_out_from_combine_only",
     "residual_out[t * H + h] = oracle_f32_to_bf16(s_scratch[h]);",
     "residual_out[t * H + h] = oracle_f32_to_bf16(s_scratch[h] - oracle_bf16_to_f32(residual[t * H + h]));"),
    # per-region layout (second occurrences are in oracle_dispatch_region)
    ("region_by_modulo", "int64_t r = e / epr;", "int64_t r = e % ep;", 1),
    ("region_src_holds_token", "src_index[row] = (int32_t)f;",
     "src_index[row] = (int32_t)(f / k);", 1),
    ("region_rows_fill_from_the_end", "int64_t row = r * cap + s;",
     "int64_t row = r * cap + (cap - 1 - s);", 1),
    ("region_no_dedup", "*first_j = i;\n            return 0;",
     "*first_j = i;\n            return 1;"),
    ("region_duplicate_added_twice",
     "if (once_per_row && row_seen_before(slot_index, t, j, k))", "if (0)"),
    ("region_duplicate_loses_row", "slot_index[f] = slot_index[t * k + first_j];",
     "slot_index[f] = slot_index[f];"),
    ("region_copies_wrong_token", "memcpy(ws + row * H, x + t * H,",
     "memcpy(ws + row * H, x + (t + 1 == T ? 0 : t + 1) * H,"),
    # reduction of tensor-parallel partials
    ("partials_drop_last", "for (int64_t p = 0; p < P; ++p)", "for (int64_t p = 0; p < P - 1; ++p)"),
    ("partials_bf16_accumulator",
     "acc = acc + oracle_bf16_to_f32(partials[(p * T + t) * H + h]);",
     "acc = oracle_bf16_to_f32(oracle_f32_to_bf16(acc + oracle_bf16_to_f32(partials[(p * T + t) * H + h])));"),
    ("partials_token_major",
     "acc = acc + oracle_bf16_to_f32(partials[(p * T + t) * H + h]);",
     "acc = acc + oracle_bf16_to_f32(partials[(t * P + p) * H + h]);"),
    ("partials_residual_not_added",
     "float s = sum + oracle_bf16_to_f32(residual[t * H + h]);", "float s = sum;"),
    ("partials_eps_outside_sqrt",
     "double rinv = 1.0 / sqrt(sumsq / (double)H + (double)eps);",
     "double rinv = 1.0 / (sqrt(sumsq / (double)H) + (double)eps);"),
    ("partials_gamma_dropped",
     "double n = (double)s_scratch[h] * rinv * (double)oracle_bf16_to_f32(gamma[h]);",
     "double n = (double)s_scratch[h] * rinv;"),
    ("partials_residual_out_from_sum_only",
     "residual_out[t * H + h] = oracle_f32_to_bf16(s_scratch[h]);",
     "residual_out[t * H + h] = oracle_f32_to_bf16(s_scratch[h] - oracle_bf16_to_f32(residual[t * H + h]));", 1),
    # FP8 payload
    ("e4m3_truncates", "double r = isinf(a) ? INFINITY : ldexp(nearbyint(ldexp(a, -qexp)), qexp);",
     "double r = isinf(a) ? INFINITY : ldexp(floor(ldexp(a, -qexp)), qexp);"),
    ("e4m3_subnormal_step", "if (qexp < -9)\n        qexp = -9;", "if (qexp < -10)\n        qexp = -10;"),
    ("e4m3_bias", "return (uint8_t)(sign | ((re - 1 + 7) << 3) | frac);",
     "return (uint8_t)(sign | ((re - 1 + 8) << 3) | frac);"),
    ("e4m3_decode_bias", "v = ldexp(1.0 + frac / 8.0, exp - 7);", "v = ldexp(1.0 + frac / 8.0, exp - 8);"),
    ("fp8_scale_to_480", "float inv = amax > 0.0f ? 448.0f / amax : 0.0f;",
     "float inv = amax > 0.0f ? 480.0f / amax : 0.0f;"),
    ("fp8_scale_inverted", "scale[t] = amax / 448.0f;", "scale[t] = 448.0f / amax;"),
    ("fp8_amax_signed", "float a = fabsf(oracle_bf16_to_f32(x[t * H + h]));",
     "float a = oracle_bf16_to_f32(x[t * H + h]);"),
    ("region_first_copy_scan_skips_copy_0", "for (int64_t i = 0; i < j; ++i) {\n        int32_t e = ids[t * k + i];",
     "for (int64_t i = 1; i < j; ++i) {\n        int32_t e = ids[t * k + i];"),
]


def _failed_pins(o, first_only=False):
    """Names of the pins the oracle ``o`` fails (only the first with
    ``first_only``: a mutant needs one failing pin to count as caught)."""
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except Exception:             # a wrong value, or a pin that cannot even index it
            failed.append(pin.__name__)
            if first_only:
                break
    return failed


def test_unmodified_oracle_passes_every_pin(orc):
    assert _failed_pins(orc) == []


def _replace_nth(text, old, new, nth):
    start = -1
    for _ in range(nth + 1):
        start = text.index(old, start + 1)
    return text[:start] + new + text[start + len(old):]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(tmp_path, mutation):
    name, old, new = mutation[:3]
    nth = mutation[3] if len(mutation) > 3 else 0
    src = open(oracle.SOURCE).read()
    assert src.count(old) > nth, f"mutation anchor for {name} not found"
    mutated = os.path.join(tmp_path, "mutant.c")
    with open(mutated, "w") as fh:
        fh.write(_replace_nth(src, old, new, nth))
    lib = oracle.build(mutated, os.path.join(tmp_path, f"libmutant_{name}.so"))
    failed = _failed_pins(oracle.Oracle(lib), first_only=True)
    assert failed, f"mutation {name} passed every pin"
