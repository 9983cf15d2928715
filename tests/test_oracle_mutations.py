"""Pin sensitivity: plant plausible mistakes in a copy of the oracle (on the
CPU only) and check that the oracle pin tests fail for every one of them."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "tq_oracle.c")

# (name, original text, mutated text): a dropped term, a wrong sign, a wrong
# index, a transposed operand, a wrong rounding rule, ...
MUTATIONS = [
    ("b3_padding_digit", "tg[k] + 1 : 1;", "tg[k] + 1 : 0;"),
    ("b3_radix", "weight *= 3;", "weight *= 4;"),
    ("b3_reject_bound", "if (value >= 243) return", "if (value > 243) return"),
    ("b3_digit_map", "tg[k] = (int8_t)(digit - 1);", "tg[k] = (int8_t)(1 - digit);"),
    ("twobit_order", "value |= (tg[4 * b + i] + 1) << (2 * i);",
     "value |= (tg[4 * b + i] + 1) << (2 * (3 - i));"),
    ("quant_ties_away", "float v = rintf(x[k] * inv);", "float v = roundf(x[k] * inv);"),
    ("quant_max_not_absmax", "float m = fabsf(x[k]);", "float m = x[k];"),
    ("quant_scale_inverted", "float sc = a / 127.0f;", "float sc = 127.0f / a;"),
    ("quant_inv_128", "float inv = 127.0f / a;", "float inv = 128.0f / a;"),
    ("core_wrong_index", "(int32_t)qrow[g * ORC_GROUP + i];", "(int32_t)qrow[i];"),
    ("output_first_scale", "orc_half_to_float(srow[g])", "orc_half_to_float(srow[0])"),
    ("output_drops_act_scale", "return (float)((double)a * acc);", "return (float)acc;"),
    ("output_fp32_accumulate", "double acc = 0.0;", "float acc = 0.0f;"),
    ("swiglu_sign", "z / (1.0 + exp(-z));", "z / (1.0 + exp(z));"),
    ("half_exponent_bias", "e - 25);", "e - 24);"),
    ("half_subnormal", "ldexp((double)f, -24);", "ldexp((double)f, -25);"),
    ("hadamard_norm", "double v = sum / 8.0;", "double v = sum / 64.0;"),
    ("hadamard_parity_or", "bit_parity(i & j)", "bit_parity(i | j)"),
    ("hadamard_negated", "? -(double)u[j] : (double)u[j];", "? (double)u[j] : -(double)u[j];"),
    ("hadamard_sign_index", "(float)(signs[b * ORC_HBLOCK + i] * v)", "(float)(signs[b * ORC_HBLOCK] * v)"),
    ("hadamard_block_offset", "const float *u = x + m * K + b * ORC_HBLOCK;", "const float *u = x + m * K;"),
    ("tern_objective_mean", "double obj = prefix * prefix / (double)k;", "double obj = prefix / (double)k;"),
    ("tern_scale_over_group", "double scale = best_k ? best_sum / (double)best_k : 0.0;",
     "double scale = best_k ? best_sum / 128.0 : 0.0;"),
    ("tern_sign", "tg[i] = wg[i] > 0.0f ? 1 : (wg[i] < 0.0f ? -1 : 0);",
     "tg[i] = wg[i] > 0.0f ? -1 : (wg[i] < 0.0f ? 1 : 0);"),
    ("half_round_truncates", "double r = rint(ldexp(v, 10 - E));", "double r = floor(ldexp(v, 10 - E));"),
    ("half_subnormal_step", "double r = rint(ldexp(v, 24));", "double r = rint(ldexp(v, 23));"),
    ("bp_bit_order", "if (tg[8 * b + i] != 0) nz |= 1 << i;", "if (tg[8 * b + i] != 0) nz |= 1 << (7 - i);"),
    ("bp_sign_of_positive", "if (tg[8 * b + i] < 0) neg |= 1 << i;", "if (tg[8 * b + i] > 0) neg |= 1 << i;"),
    ("bp_accepts_sign_on_zero", "if (in[16 + b] & ~in[b]) return ORC_ERR_FORMAT;", "if (0) return ORC_ERR_FORMAT;"),
]


@pytest.mark.parametrize("name,orig,mut", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, orig, mut):
    src = open(SRC).read()
    assert src.count(orig) == 1, f"mutation anchor for {name} not unique / missing"
    msrc = tmp_path / "tq_oracle.c"
    msrc.write_text(src.replace(orig, mut))
    (tmp_path / "tq_oracle.h").write_text(open(SRC[:-2] + ".h").read())
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    "-o", str(so), str(msrc), "-lm"], check=True)
    env = dict(os.environ, TQ_ORACLE_LIB_OVERRIDE=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"planted mistake {name} went unnoticed:\n{r.stdout[-2000:]}"
