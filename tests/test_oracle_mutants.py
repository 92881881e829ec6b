"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that the
pins catch every one: a dropped term, a wrong sign or index, a swapped operand,
the inclusive/exclusive mix-up, a wrong identity, a signed/unsigned slip."""
import os

import pytest

import oracle
from oracle_pins import PINS

# (name, text in oracle.c, replacement); each text must occur exactly once.
MUTANTS = [
    ("exclusive_becomes_inclusive",
     "            y[i] = acc;\n            acc = op_u32(dtype, op, acc, x[i]);",
     "            acc = op_u32(dtype, op, acc, x[i]);\n            y[i] = acc;"),
    ("inclusive_wrong_index",
     "acc = (i == 0) ? x[0] : op_u32(dtype, op, acc, x[i]);",
     "acc = (i == 0) ? x[0] : op_u32(dtype, op, acc, x[i - 1]);"),
    ("sum_sign", "return a + b; /* wraps mod 2^32 */", "return a - b;"),
    ("xor_is_or", "return a ^ b;", "return a | b;"),
    ("max_identity_zero", "return dtype == OR_INT32 ? 0x80000000u : 0u;", "return 0u;"),
    ("int32_max_unsigned", "return ((int32_t)a > (int32_t)b) ? a : b;", "return (a > b) ? a : b;"),
    ("uint32_max_signed", "        return (a > b) ? a : b;\n    case OR_MIN:",
     "        return ((int32_t)a > (int32_t)b) ? a : b;\n    case OR_MIN:"),
    ("f32_sum_sign", "acc = (i == 0) ? v : acc + v;", "acc = (i == 0) ? v : acc - v;"),
    ("f32_exclusive_dropped_term",
     "acc = (i == 0) ? v : acc + v;\n            y[i] = acc;\n        } else {\n            y[i] = acc;\n            acc += v;",
     "acc = (i == 0) ? v : acc + v;\n            y[i] = acc;\n        } else {\n            y[i] = acc;\n            acc = v;"),
    ("f32_bound_not_abs", "        double v = (double)x[i];\n        mag += (v < 0.0) ? -v : v;",
     "        double v = (double)x[i];\n        mag += v;"),
    ("f32_max_tie_left", "    return (a > b) ? a : b;\n}", "    return (a >= b) ? a : b;\n}"),
    ("f32_max_identity_zero", "uint32_t ninf_bits = 0xff800000u;", "uint32_t ninf_bits = 0u;"),
    ("compact_negated", "        if (pred_holds(dtype, cmp, x[i], thr_bits))\n            out[c++] = x[i];",
     "        if (!pred_holds(dtype, cmp, x[i], thr_bits))\n            out[c++] = x[i];"),
    ("compact_inclusive_index", "        index[i] = run;\n        run += flags[i];",
     "        run += flags[i];\n        index[i] = run;"),
    ("pred_lt_is_le", "    case 0: return lt;", "    case 0: return lt || eq;"),
    ("pred_int32_unsigned", "lt = (int32_t)vbits < (int32_t)tbits;", "lt = vbits < tbits;"),
    ("pred_float_gt_ge", "        case 2: return v > t;", "        case 2: return v >= t;"),
    ("batched_row_stride", "oracle_scan_u32(x + r * cols, y + r * cols,",
     "oracle_scan_u32(x + r, y + r * cols,"),
    ("batched_f32_carry", "oracle_scan_f32_sum(x + r * cols, y + r * cols,",
     "oracle_scan_f32_sum(x, y + r * cols,"),
    ("flags_keep_zero", "        if (flags[i] != 0)\n            out[c++] = x[i];",
     "        if (flags[i] == 0)\n            out[c++] = x[i];"),
    ("indices_off_by_one", "            out[c++] = (uint32_t)i;\n    }\n    return c;\n}\n\nint64_t oracle_indices_if",
     "            out[c++] = (uint32_t)(i + 1);\n    }\n    return c;\n}\n\nint64_t oracle_indices_if"),
    ("sort_unstable_ties", "take_left = oracle_sort_order_key(dtype, k[i]) <= oracle_sort_order_key(dtype, k[j]);",
     "take_left = oracle_sort_order_key(dtype, k[i]) < oracle_sort_order_key(dtype, k[j]);"),
    ("sort_int32_unsigned", "        return k ^ 0x80000000u;\n    if (dtype == OR_FLOAT32)",
     "        return k;\n    if (dtype == OR_FLOAT32)"),
    ("sort_float_negatives", "return (k & 0x80000000u) ? ~k : (k | 0x80000000u);",
     "return (k & 0x80000000u) ? (k ^ 0x80000000u) : (k | 0x80000000u);"),
    ("min_identity_zero", "return dtype == OR_INT32 ? 0x7fffffffu : 0xffffffffu; /* largest value */",
     "return 0u;"),
    ("int32_min_unsigned", "            return ((int32_t)a < (int32_t)b) ? a : b;",
     "            return (a < b) ? a : b;"),
    ("and_identity_zero", "    case OR_AND:\n        return 0xffffffffu;", "    case OR_AND:\n        return 0u;"),
    ("prod_identity_zero", "    case OR_PROD:\n        return 1u;", "    case OR_PROD:\n        return 0u;"),
    ("or_is_xor", "        return a | b;", "        return a ^ b;"),
    ("affine_order_swapped", "        return affine_then(a, b);", "        return affine_then(b, a);"),
    ("affine_offset_term", "uint32_t b = (a2 * b1 + b2) & 0xffffu;", "uint32_t b = (a1 * b2 + b1) & 0xffffu;"),
    ("f32_min_tie_left", "    return (a < b) ? a : b;\n}\n\nvoid oracle_scan_f32_min",
     "    return (a <= b) ? a : b;\n}\n\nvoid oracle_scan_f32_min"),
    ("seg_carry_across_head", "        int head = (i == 0) || heads[i] != 0;", "        int head = (i == 0);"),
    ("seg_exclusive_wrong_operand", "op_u32(dtype, op, prev_y, prev_x);", "op_u32(dtype, op, prev_y, x[i]);"),
    ("seg_f32_sum_no_restart", "            acc = 0.0;\n            mag = 0.0;", "            mag = 0.0;"),
    ("seg_minmax_tie_lost", "            acc = is_min ? fmin_right(acc, x[i]) : fmax_right(acc, x[i]);\n            y[i] = acc;",
     "            acc = is_min ? fmin_right(x[i], acc) : fmax_right(x[i], acc);\n            y[i] = acc;"),
    ("offsets_drop_last_segment", "    for (int64_t k = 0; k < nseg; ++k) {", "    for (int64_t k = 0; k < nseg - 1; ++k) {"),
    ("seg_f32_prod_no_restart",
     "        if (i == 0 || heads[i] != 0)\n            acc = 1.0;\n",
     ""),
    ("seg_f32_prod_restart_zero",
     "        if (i == 0 || heads[i] != 0)\n            acc = 1.0;\n",
     "        if (i == 0 || heads[i] != 0)\n            acc = 0.0;\n"),
    ("seg_f32_prod_exclusive_is_inclusive",
     "            y[i] = acc;\n            acc *= (double)x[i];",
     "            acc *= (double)x[i];\n            y[i] = acc;"),
    ("batched_f32_prod_row_stride", "oracle_scan_f32_prod(x + r * cols, y + r * cols,",
     "oracle_scan_f32_prod(x + r, y + r * cols,"),
    ("batched_f32_prod_carry", "oracle_scan_f32_prod(x + r * cols, y + r * cols,",
     "oracle_scan_f32_prod(x, y + r * cols,"),
    ("f32_prod_exclusive_dropped_term", "            y[i] = acc;\n            acc *= v;",
     "            acc *= v;\n            y[i] = acc;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path):
    src = oracle.source_text()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    mutant = oracle.compile_variant(src.replace(old, new), os.path.join(tmp_path, f"{name}.so"))
    caught = []
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
            break
    assert caught, f"no pin caught the planted mistake {name}"
