"""Mutation check of the oracle's pins: each case plants one plausible mistake
in a copy of oracle/oracle.c (a wrong sign, a dropped term, a swapped index,
another tie rule, another rounding order, an off-by-one), builds it, and runs
the fast pin tests against that build in a subprocess.  The pins must reject
every mutant; a mutant they accept would be a mistake the oracle could carry
unnoticed.  The mistakes live only in temporary copies on the CPU."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = [os.path.join(ROOT, "tests", "test_oracle_pins.py"), os.path.join(ROOT, "tests", "test_oracle_reduce_pins.py")]
FAST = "not brute_force_sweep and not torch_cast_sweep"

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("sigmoid_sign", "expq(-(__float128)g)", "expq((__float128)g)"),
    ("sigmoid_in_double", "__float128 e = expq(-(__float128)g);\n    __float128 s = 1 / (1 + e);",
     "double e = exp(-(double)g);\n    double s = 1 / (1 + e);"),
    ("e4m3_ties_away", "code = ((e + 7) << 3) + (int)nearbyint(ldexp(a, 3 - e)) - 8;",
     "code = ((e + 7) << 3) + (int)round(ldexp(a, 3 - e)) - 8;"),
    ("e4m3_subnormal_step", "code = (int)nearbyint(a * 0x1p9);", "code = (int)nearbyint(a * 0x1p8);"),
    ("e2m1_ties_away", "code = (int)nearbyint(a * 2.0);", "code = (int)round(a * 2.0);"),
    ("ue8m0_off_by_one", "ldexp((double)fmt_max, k) < (double)amax", "ldexp((double)fmt_max, k) <= (double)amax"),
    ("amax_without_abs", "float m = fabsf(y[j]);", "float m = y[j];"),
    ("inverse_of_rounded_scale", "inv = fmt_max / amax; /* +inf when amax == 0 */", "inv = 1.0f / *scale_f32;"),
    ("clamp_count_at_limit", "if (g > clamp_limit) {", "if (g >= clamp_limit) {"),
    ("up_not_clamped", "if (u > clamp_limit)\n                u = clamp_limit;", ""),
    ("product_order", "float a = g * sig;\n            float b = a * u;", "float a = sig * u;\n            float b = a * g;"),
    ("weight_dropped", "float yv = w ? b * wr : b;", "float yv = b;"),
    ("fp4_nibbles_swapped", "(uint8_t)(tmp[2 * i] | (tmp[2 * i + 1] << 4))",
     "(uint8_t)(tmp[2 * i + 1] | (tmp[2 * i] << 4))"),
    ("topk_ties_to_larger_index", "return sa > sb || (sa == sb && a < b);", "return sa > sb || (sa == sb && a > b);"),
    ("topk_group_score_best_only", "gscore[g] = s[b1] + s[b2];", "gscore[g] = s[b1];"),
    ("topk_nan_group_score_kept_as_nan",
     "if (gscore[g] != gscore[g]) /* +inf + -inf: ranks as -inf */\n                    gscore[g] = -INFINITY;", ""),
    ("topk_sum_worst_first", "for (int64_t j = 0; j < k; ++j)\n                sum += w_out[t * k + j];",
     "for (int64_t j = k - 1; j >= 0; --j)\n                sum += w_out[t * k + j];"),
    ("reduce_scale_by_slot", "w[t * k + j] * row_scale[p]", "w[t * k + j] * row_scale[j]"),
    ("reduce_last_slot_skipped",
     "for (int64_t j = 0; j < k; ++j) {\n                const int64_t p = pos[t * k + j];",
     "for (int64_t j = 0; j < k - 1; ++j) {\n                const int64_t p = pos[t * k + j];"),
    ("reduce_slots_reversed",
     "for (int64_t j = 0; j < k; ++j) {\n                const int64_t p = pos[t * k + j];",
     "for (int64_t j = k - 1; j >= 0; --j) {\n                const int64_t p = pos[t * k + j];"),
    ("reduce_fused_multiply_add", "acc = acc + term;",
     "acc = fmaf(row_scale ? w[t * k + j] * row_scale[p] : w[t * k + j], bf16_to_float(x[p * hidden + c]), acc);"),
    ("reduce_scale_per_term", "const float o = acc * global_scale;", "const float o = acc * global_scale * 1.0000001f;"),
    ("bf16_ties_up", "up = (int)((lo_b >> 16) & 1u); /* tie: go to the even code */", "up = 1;"),
    ("bf16_truncates", "if (dlo < dhi)\n        up = 0;", "if (dlo <= dhi || 1)\n        up = 0;"),
    # the fused per-row form, written apart from the two stages
    ("fused_clamp_count_at_limit", "if (gv > clamp_limit) {", "if (gv >= clamp_limit) {"),
    ("fused_up_not_clamped",
     "if (uv < -clamp_limit)\n                        uv = -clamp_limit;\n                    else if (uv > clamp_limit)\n"
     "                        uv = clamp_limit;", ""),
    ("fused_product_order",
     "const float act = gv * oracle_sigmoid(gv);\n                const float prod = act * uv;",
     "const float act = oracle_sigmoid(gv) * uv;\n                const float prod = act * gv;"),
    ("fused_weight_dropped", "const float v = w != NULL ? prod * w[r] : prod;", "const float v = prod;"),
    ("fused_amax_without_abs", "const float mag = v < 0.0f ? -v : v;", "const float mag = v;"),
    ("fused_ue8m0_off_by_one", "int k = ea - ef + (ma > mf ? 1 : 0);", "int k = ea - ef + (ma >= mf ? 1 : 0);"),
    ("fused_inverse_of_rounded_scale", "mult = group_amax > 0.0f ? fmt_max / group_amax : FLT_MAX;",
     "mult = 1.0f / (group_amax / fmt_max);"),
    ("fused_fp4_nibbles_swapped", "} else if (col % 2 == 0) {", "} else if (col % 2 == 1) {"),
    ("fused_scale_index", "((float*)scales)[r * groups + k] = group_amax / fmt_max;",
     "((float*)scales)[r + k] = group_amax / fmt_max;"),
    # the stand-alone cast of bf16 rows
    ("cast_bf16_row_stride", "row[j] = bf16_to_float(x[r * hidden + j]);", "row[j] = bf16_to_float(x[j]);"),
    ("cast_bf16_widening_drops_a_bit", "row[j] = bf16_to_float(x[r * hidden + j]);",
     "row[j] = bf16_to_float((uint16_t)(x[r * hidden + j] & 0xFFFEu));"),
    ("cast_bf16_scale_stride", "(uint8_t*)scales + (size_t)(r * groups) * scale_bytes);",
     "(uint8_t*)scales + (size_t)r * scale_bytes);"),
    # the token/top-k -> position map
    ("pos_repeat_kept", "if (idx[t * k + i] == e)\n                    present = 0;", "if (0)\n                    present = 0;"),
    ("pos_offsets_inclusive", "offsets[e] = (int32_t)run;\n        run += count[e];",
     "run += count[e];\n        offsets[e] = (int32_t)run;"),
    ("pos_expert_zero_absent", "int present = e >= 0 && e < experts;", "int present = e > 0 && e < experts;"),
    ("pos_tokens_reversed",
     "for (int64_t t = 0; t < tokens; ++t) {\n        for (int64_t j = 0; j < k; ++j) {\n            if (pos[t * k + j] < 0)",
     "for (int64_t t = tokens - 1; t >= 0; --t) {\n        for (int64_t j = 0; j < k; ++j) {\n            if (pos[t * k + j] < 0)"),
]


def run_mutant(tmp_dir, name, old, new):
    """Build one mutant and run the fast pins against it; returns None when
    the pins reject it, else a report."""
    src = open(oracle.SOURCE).read()
    if src.count(old) != 1:
        return f"{name}: the mutation site must occur exactly once in oracle.c"
    mutant = os.path.join(tmp_dir, f"{name}.c")
    with open(mutant, "w") as fh:
        fh.write(src.replace(old, new))
    lib = os.path.join(tmp_dir, f"lib{name}.so")
    subprocess.run(oracle.build_command(lib, mutant), check=True, capture_output=True)
    env = dict(os.environ, ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-k", FAST] + PINS,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    # exit status 1 = tests ran and at least one failed (not an import or usage error)
    if r.returncode == 1 and " failed" in r.stdout:
        return None
    return f"{name}: pins did not reject the mutant\n" + (r.stdout + r.stderr)[-1200:]


def test_pins_reject_every_planted_mistake(tmp_path):
    workers = max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        reports = list(ex.map(lambda m: run_mutant(str(tmp_path), *m), MUTANTS))
    survivors = [r for r in reports if r]
    assert not survivors, "\n\n".join(survivors)
