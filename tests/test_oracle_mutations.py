"""The pins catch plausible mistakes in the oracle (CPU only).

Each case plants one mistake in a copy of oracle/zs_oracle.c (a wrong
operand, a dropped term, a wrong sign or index, a different rounding or
order), compiles the copy, swaps it in for the oracle library and runs the
battery of pins: at least one pin must fail.  The committed oracle is never
modified.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_pins as P
from tests import test_oracle_q8 as Q
from tests import test_oracle_sharding as S
from tests import test_oracle_sr as R
from tests import test_oracle_variants as V

SRC = os.path.join(os.path.dirname(oracle.__file__), "zs_oracle.c")

# (name, text in the oracle, replacement): one plausible mistake each
MUTATIONS = [
    ("second moment decays with beta1",
     "float c = hp->beta2 * v_prev;", "float c = hp->beta1 * v_prev;"),
    ("first moment weighted by 1-beta2",
     "float b = s->c1 * g;", "float b = s->c2 * g;"),
    ("second moment of g instead of g^2",
     "float gg = g * g;", "float gg = g;"),
    ("no bias correction of m",
     "float m_hat = m_new / s->bc1;", "float m_hat = m_new;"),
    ("no bias correction of v",
     "float v_hat = v_new / s->bc2;", "float v_hat = v_new;"),
    ("bias correction at t-1",
     "pow((double)hp->beta1, (double)t)", "pow((double)hp->beta1, (double)(t - 1))"),
    ("epsilon inside the square root",
     "float denom = sqrtf(v_hat) + hp->eps;", "float denom = sqrtf(v_hat + hp->eps);"),
    ("decay with the wrong sign",
     "s.df = 1.0f - lrwd;", "s.df = 1.0f + lrwd;"),
    ("decay applied to every element",
     "float w_dec = decay ? (w_prev * s->df) : w_prev;", "float w_dec = w_prev * s->df;"),
    ("decay applied after the update",
     "float w_new = w_dec - step;",
     "float w_new = decay ? ((w_prev - step) * s->df) : (w_prev - step);"),
    ("update added instead of subtracted",
     "float w_new = w_dec - step;", "float w_new = w_dec + step;"),
    ("partials folded in reverse order",
     "        float g = bf16_to_f32(grads[0][i]);\n        for (int j = 1; j < k; ++j)\n"
     "            g = g + bf16_to_f32(grads[j][i]);",
     "        float g = bf16_to_f32(grads[k - 1][i]);\n        for (int j = k - 2; j >= 0; --j)\n"
     "            g = g + bf16_to_f32(grads[j][i]);"),
    ("last partial dropped",
     "        for (int j = 1; j < k; ++j)\n            g = g + bf16_to_f32(grads[j][i]);\n"
     "        g = g * hp->grad_scale;\n\n        adamw_element",
     "        for (int j = 1; j < k - 1; ++j)\n            g = g + bf16_to_f32(grads[j][i]);\n"
     "        g = g * hp->grad_scale;\n\n        adamw_element"),
    ("grad_scale ignored",
     "        g = g * hp->grad_scale;\n\n        adamw_element",
     "        g = g;\n\n        adamw_element"),
    ("segment entry chosen one element late",
     "while (seg + 1 < nseg && segs[seg + 1].start <= i)",
     "while (seg + 1 < nseg && segs[seg + 1].start < i)"),
    ("bf16 cast truncates",
     "if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))", "if (0)"),
    ("bf16 ties round up instead of to even",
     "if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))", "if (lo >= 0x8000u)"),
    ("param cast from the old weight",
     "        adamw_element(&master[i], &m[i], &v[i], g, decay, hp, &sc);\n"
     "        param_bf16[i] = zs_oracle_bf16_rne(master[i]);",
     "        param_bf16[i] = zs_oracle_bf16_rne(master[i]);\n"
     "        adamw_element(&master[i], &m[i], &v[i], g, decay, hp, &sc);"),
]

# Mistakes in the variant routines (quantized payload, quantized partials,
# bf16 moments): caught by the variant pins.
VARIANT_MUTATIONS = [
    ("q8 scale over 128 levels",
     "float s = a / 127.0f;", "float s = a / 128.0f;"),
    ("q8 ties rounded away from zero",
     "float r = rintf(bf16_to_f32(x_bf16[i]) / s);", "float r = roundf(bf16_to_f32(x_bf16[i]) / s);"),
    ("q8 codes truncated",
     "float r = rintf(bf16_to_f32(x_bf16[i]) / s);", "float r = truncf(bf16_to_f32(x_bf16[i]) / s);"),
    ("q8 block maximum of x instead of |x|",
     "else if (fabsf(x) > a) a = fabsf(x);", "else if (x > a) a = x;"),
    ("q8 NaN does not poison its block",
     "if (has_nan) a = NAN;", "if (0) a = NAN;"),
    ("q8grad every partial scaled by partial 0's scale",
     "float t = (float)q[j][i] * scale[j][b];", "float t = (float)q[j][i] * scale[0][b];"),
    ("q8grad last partial dropped",
     "for (int j = 1; j < k; ++j) {\n            float t = (float)q[j][i]",
     "for (int j = 1; j < k - 1; ++j) {\n            float t = (float)q[j][i]"),
    ("q8grad grad_scale ignored",
     "g = g * hp->grad_scale;\n        adamw_element(&master[i], &m[i], &v[i], g, segs[seg].wd_on",
     "g = g;\n        adamw_element(&master[i], &m[i], &v[i], g, segs[seg].wd_on"),
    ("bf16mv first moment not carried across steps",
     "float mf = bf16_to_f32(m[i]);", "float mf = 0.0f;"),
    ("bf16mv second moment stored from the first",
     "v[i] = zs_oracle_bf16_rne(vf);", "v[i] = zs_oracle_bf16_rne(mf);"),
    ("bf16mv moments truncated",
     "m[i] = zs_oracle_bf16_rne(mf);\n        v[i] = zs_oracle_bf16_rne(vf);",
     "{ union { float f; uint32_t u; } cm, cv; cm.f = mf; cv.f = vf;\n"
     "          m[i] = (uint16_t)(cm.u >> 16); v[i] = (uint16_t)(cv.u >> 16); }"),
]

# Mistakes in the stochastic rounding of the bf16 moments: caught by its pins.
SR_MUTATIONS = [
    ("SR truncates",
     "return (uint16_t)((u + (r & 0xffffu)) >> 16);", "return (uint16_t)(u >> 16);"),
    ("SR rounds up once too often",
     "return (uint16_t)((u + (r & 0xffffu)) >> 16);",
     "return (uint16_t)((u + (r & 0xffffu) + 1u) >> 16);"),
    ("SR carries NaN payloads",
     "    if ((u & 0x7fffffffu) > 0x7f800000u)\n        return (uint16_t)0x7FC0u;\n"
     "    return (uint16_t)((u + (r & 0xffffu)) >> 16);",
     "    return (uint16_t)((u + (r & 0xffffu)) >> 16);"),
    ("SR m and v share one stream",
     "zs_oracle_sr_bits(seed, step, 1, index0 + i)", "zs_oracle_sr_bits(seed, step, 0, index0 + i)"),
    ("SR one random field for a whole quad",
     "(word >> (16 * (i % 4))) & 0xffffu", "word & 0xffffu"),
    ("SR streams not keyed by the step",
     "2u * (uint64_t)step + (uint64_t)which", "(uint64_t)which"),
    ("SR streams not keyed by the seed",
     "uint64_t key = zs_oracle_splitmix64(seed,", "uint64_t key = zs_oracle_splitmix64(0,"),
    ("SR window bits taken from the window's own index",
     "zs_oracle_sr_bits(seed, step, 0, index0 + i)", "zs_oracle_sr_bits(seed, step, 0, i)"),
    ("SR generator's increment wrong",
     "return sm64_mix(key + (i + 1u) * 0x9E3779B97F4A7C15ull);",
     "return sm64_mix(key + i * 0x9E3779B97F4A7C15ull);"),
]

SR_BATTERY = [R.test_generator_is_the_published_splitmix64, R.test_rounding_distribution_is_exact,
              R.test_specials, R.test_first_step_matches_round_to_nearest_step,
              R.test_first_step_is_unbiased, R.test_random_streams_are_independent,
              R.test_random_bits_are_uniform,
              R.test_a_window_takes_the_bits_of_its_place_in_the_shard]

VARIANT_BATTERY = [Q.test_hand_worked_block_with_ties, Q.test_zero_block_and_single_element,
                   Q.test_nonfinite_blocks_only_poison_themselves,
                   lambda: Q.test_error_bound_and_extremes(7),
                   lambda: Q.test_error_bound_and_extremes(256),
                   Q.test_matches_torch_elementwise_formula,
                   V.test_q8grad_reduce_scatter_exercise,
                   lambda: V.test_q8grad_equals_bf16_path_on_exact_partials(1.0),
                   lambda: V.test_q8grad_equals_bf16_path_on_exact_partials(0.125),
                   V.test_q8grad_products_round_once, V.test_bf16mv_first_step_equals_fp32_path,
                   V.test_bf16mv_closed_form_with_halving_betas,
                   V.test_bf16mv_stays_close_to_fp32_path]

BATTERY = [P.test_reduce_scatter_exercise_values, P.test_ring_demo_values,
           P.test_reduce_brute_force_small_integers, P.test_reduce_is_a_left_fold,
           P.test_grad_scale_multiplies_after_the_sum, P.test_bias_correction_scalars,
           P.test_step1_update_is_lr_times_sign, P.test_constant_gradient_closed_form,
           P.test_zero_gradient_exact, P.test_power_of_two_scaling_invariance,
           P.test_bf16_rne_special_cases, P.test_matches_torch_adamw_float64,
           S.test_segment_lookup_semantics, S.test_k1_is_unsharded_adamw]


def _compile(src_text, d):
    c = os.path.join(d, "mut.c")
    so = os.path.join(d, "libmut.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", so, c, "-lm"], check=True)
    return so


def _first_failing_pin(lib, battery=None):
    saved = oracle._lib
    oracle._lib = lib
    try:
        for pin in battery or BATTERY:
            try:
                pin()
            except (AssertionError, ValueError, FloatingPointError):
                return getattr(pin, "__name__", "pin")
        return None
    finally:
        oracle._lib = saved


def test_unmutated_copy_passes_the_battery():
    with tempfile.TemporaryDirectory() as d:
        lib = oracle.load_library(_compile(open(SRC).read(), d))
        assert _first_failing_pin(lib) is None
        assert _first_failing_pin(lib, VARIANT_BATTERY) is None
        assert _first_failing_pin(lib, SR_BATTERY) is None


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation site not found: %s" % name
    mutated = text.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as d:
        lib = oracle.load_library(_compile(mutated, d))
        caught = _first_failing_pin(lib)
    assert caught is not None, "no pin catches: %s" % name
    print("%-45s caught by %s" % (name, caught))


@pytest.mark.parametrize("name,old,new", VARIANT_MUTATIONS, ids=[m[0] for m in VARIANT_MUTATIONS])
def test_planted_variant_mistake_is_caught(name, old, new):
    # the first occurrence is the routine the variant pins cover (the
    # stochastic-rounding step repeats some of its lines further down)
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation site not found: %s" % name
    mutated = text.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as d:
        lib = oracle.load_library(_compile(mutated, d))
        caught = _first_failing_pin(lib, VARIANT_BATTERY)
    assert caught is not None, "no pin catches: %s" % name
    print("%-50s caught by %s" % (name, caught))


@pytest.mark.parametrize("name,old,new", SR_MUTATIONS, ids=[m[0] for m in SR_MUTATIONS])
def test_planted_rounding_mistake_is_caught(name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation site not found once: %s" % name
    mutated = text.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as d:
        lib = oracle.load_library(_compile(mutated, d))
        caught = _first_failing_pin(lib, SR_BATTERY)
    assert caught is not None, "no pin catches: %s" % name
    print("%-50s caught by %s" % (name, caught))
