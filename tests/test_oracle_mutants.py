"""Planted mistakes in the oracle must be caught by its pins.

Each case copies the oracle's C core, plants one plausible mistake (a wrong
sign, a swapped operand, truncation instead of rounding, a flushed subnormal,
a transposed index ...), builds it with the same flags, swaps it in, and checks
that the pin suite's fast checks fail.  CPU only.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads as W
from specs import SPECS
import test_oracle_pins as P

MUTANTS = {
    "sub_operands_swapped": ("if (op == OR_SUB) return a - b;", "if (op == OR_SUB) return b - a;"),
    "f32_sub_as_add": ("\n    else if (op == OR_SUB) z = x - y;", "\n    else if (op == OR_SUB) z = x + y;"),
    "f16_sub_as_add": ("\n        else if (op == OR_SUB) z = x - y;", "\n        else if (op == OR_SUB) z = x + y;"),
    "i32_add_through_float": ("if (op == OR_ADD) return a + b;",
                              "if (op == OR_ADD) return (uint32_t)(int32_t)((float)(int32_t)a + (float)(int32_t)b);"),
    "neg_as_zero_minus": ("if (dst_dtype == OR_F32) return a ^ 0x80000000u;",
                          "if (dst_dtype == OR_F32) return bits_from_f32(0.0f - f32_from_bits(a));"),
    "f16_round_truncates": ("double q = nearbyint(ldexp(a, -spacing_exp));",
                            "double q = trunc(ldexp(a, -spacing_exp));"),
    "f16_round_half_up": ("double q = nearbyint(ldexp(a, -spacing_exp));",
                          "double q = floor(ldexp(a, -spacing_exp) + 0.5);"),
    "f16_out_subnormal_flushed": ("return sign | (uint16_t)q;", "return sign;"),
    "f16_in_subnormal_flushed": ("mag = ldexp((double)m, -24);", "mag = 0.0;"),
    "f16_exponent_bias_off": ("mag = ldexp((double)(1024 + m), (int)e - 25);",
                              "mag = ldexp((double)(1024 + m), (int)e - 24);"),
    "view_index_transposed": ("return idx[0] * g->stride[0] + idx[1] * g->stride[1] + idx[2] * g->stride[2] + idx[3] * g->stride[3];",
                              "return idx[0] * g->stride[0] + idx[1] * g->stride[1] + idx[3] * g->stride[2] + idx[2] * g->stride[3];"),
    "leading_dim_dropped": ("return idx[0] * g->stride[0] + idx[1] * g->stride[1] + idx[2] * g->stride[2] + idx[3] * g->stride[3];",
                            "return idx[1] * g->stride[1] + idx[2] * g->stride[2] + idx[3] * g->stride[3];"),
    "scalar_ignored": ("val[t] = J->args[n->arg].bits;", "val[t] = 0u;"),
    "f32_to_i32_rounds": ("return (int32_t)truncf(f);", "return (int32_t)nearbyintf(f);"),
    "second_operand_is_first": ("n->b >= 0 ? val[n->b] : 0u", "n->b >= 0 ? val[n->a] : 0u"),
    "select_swapped": ("return a != 0u ? b : c;", "return a != 0u ? c : b;"),
    "unsigned_compare_signed": ("if (op == OR_CMP_LTU) r = a < b;",
                                "if (op == OR_CMP_LTU) r = (int32_t)a < (int32_t)b;"),
    "float_ne_ordered": ("else if (op == OR_CMP_NE) r = x != y;  /* true when either is NaN */",
                         "else if (op == OR_CMP_NE) r = (x < y) || (x > y);"),
    "min_keeps_nan": ("static double min_number(double x, double y)\n{\n    if (isnan(x)) return y;\n    if (isnan(y)) return x;\n",
                      "static double min_number(double x, double y)\n{\n"),
    "min_zero_sign": ("return signbit(x) ? x : y;          /* equal: pick -0 over +0 */", "return x;"),
    "abs_int_saturates": ("return (a & 0x80000000u) ? 0u - a : a;",
                          "return (a & 0x80000000u) ? (a == 0x80000000u ? 0x7fffffffu : 0u - a) : a;"),
    # binary16 / bfloat16 arithmetic and bfloat16 conversions
    "bf16_round_truncates": ("double units = nearbyint(ldexp(a, -unit_exp));",
                             "double units = trunc(ldexp(a, -unit_exp));"),
    "bf16_subnormal_flushed": ("return sign | (uint16_t)units;", "return sign;"),
    "bf16_exponent_bias_off": ("mag = ldexp((double)(128 + m), (int)e - 134);",
                               "mag = ldexp((double)(128 + m), (int)e - 133);"),
    "bf16_overflow_one_binade_early": ("if (rounded >= ldexp(1.0, 128))", "if (rounded >= ldexp(1.0, 127))"),
    "i32_bf16_through_f32": ("return src_dtype == OR_I32 ? bf16_round_from_exact((double)(int32_t)a)",
                             "return src_dtype == OR_I32 ? bf16_round_from_exact((double)(float)(int32_t)a)"),
    "f16_arith_rounded_to_bf16": ("return dtype == OR_F16 ? f16_round_from_exact(v) : bf16_round_from_exact(v);",
                                  "return bf16_round_from_exact(v);"),
    "f16_operands_read_as_f32": ("double x = float_value(dst_dtype, a), y = float_value(dst_dtype, b), z;",
                                 "double x = float_value(OR_F32, a), y = float_value(OR_F32, b), z;"),
    "bf16_round_half_away": ("double units = nearbyint(ldexp(a, -unit_exp));",
                             "double units = floor(ldexp(a, -unit_exp) + 0.5);"),
    "min16_returns_first": ("        return m == x ? a : b;", "        return a;"),
    "mul_high_dropped": ("return a * b;                        /* low 32 bits of the product */",
                         "return (a & 0xffffu) * (b & 0xffffu);"),
}


def _fast_pins(oracle_mod):
    """Run the quick pins; return the number that fail."""
    P.PAIRS_RANDOM, P.PAIRS_SPECIAL_BF16 = 1 << 16, 400
    failures = 0
    checks = [lambda c=c: P.test_hand_worked(oracle_mod, c) for c in P.GOLDEN_CASES]
    checks += [
        lambda: P.test_add_f32_vs_numpy(oracle_mod),
        lambda: P.test_int_fused_vs_numpy(oracle_mod, True),
        lambda: P.test_axpby_vs_numpy_and_binary64(oracle_mod),
        lambda: P.test_mixed_vs_numpy(oracle_mod),
        lambda: P.test_int32_invariants(oracle_mod),
        lambda: P.test_f32_invariants(oracle_mod),
        lambda: P.test_f16_to_f32_all_patterns(oracle_mod),
        lambda: P.test_f32_to_f16_every_tie_and_neighbour(oracle_mod),
        lambda: P.test_transposed_brute_force(oracle_mod, (17, 33), 1, 3),
        lambda: P.test_i32_conversions_vs_numpy(oracle_mod),
        lambda: P.test_rank_n_views_brute_force(oracle_mod, 3),
        lambda: P.test_new_ops_vs_numpy(oracle_mod),
        lambda: P.test_16bit_arith_vs_libraries(oracle_mod, "add", "bf16"),
        lambda: P.test_16bit_arith_vs_libraries(oracle_mod, "mul", "bf16"),
        lambda: P.test_16bit_arith_vs_libraries(oracle_mod, "mul", "f16"),
        lambda: P.test_bf16_conversions_vs_torch(oracle_mod),
        lambda: P.test_16bit_min_max_compare_vs_libraries(oracle_mod, "bf16"),
    ]
    for chk in checks:
        try:
            chk()
        except AssertionError:
            failures += 1
    return failures


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


def test_unmutated_copy_passes(oracle_mod, mutant_dir):
    src = open(oracle_mod.SRC).read()
    path = str(mutant_dir / "clean.c")
    open(path, "w").write(src)
    so = path[:-2] + ".so"
    subprocess.run(["gcc", *oracle_mod.GCC_FLAGS, "-o", so, path, "-lm"], check=True)
    prev = oracle_mod.use_library(so)
    try:
        assert _fast_pins(oracle_mod) == 0
    finally:
        oracle_mod.use_library(prev)


def _run_pins_in_child(so):
    """Run the fast pins against the library at so in a child process: a
    planted mistake may read out of bounds and abort, which also counts as
    caught.  Returns (failures or None if the child crashed, output)."""
    here = os.path.dirname(os.path.abspath(__file__))
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "from oracle import oracle\n"
            "import test_oracle_mutants as M\n"
            "oracle.use_library(%r)\n"
            "print('FAILURES', M._fast_pins(oracle))\n") % (os.path.dirname(here), here, so)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    for line in r.stdout.splitlines():
        if line.startswith("FAILURES"):
            return int(line.split()[1]), r.stdout + r.stderr
    return None, r.stdout + r.stderr


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(oracle_mod, mutant_dir, name):
    old, new = MUTANTS[name]
    src = open(oracle_mod.SRC).read()
    assert src.count(old) == 1, "mutation anchor for %s not found exactly once" % name
    path = str(mutant_dir / (name + ".c"))
    open(path, "w").write(src.replace(old, new))
    so = path[:-2] + ".so"
    subprocess.run(["gcc", *oracle_mod.GCC_FLAGS, "-Wno-unused-function", "-o", so, path, "-lm"],
                   check=True)
    failures, out = _run_pins_in_child(so)
    assert failures is None or failures > 0, "planted mistake %s went unnoticed" % name
