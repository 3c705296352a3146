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
from tests import test_oracle_sharding as S

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


def _first_failing_pin(lib):
    saved = oracle._lib
    oracle._lib = lib
    try:
        for pin in BATTERY:
            try:
                pin()
            except (AssertionError, ValueError, FloatingPointError):
                return pin.__name__
        return None
    finally:
        oracle._lib = saved


def test_unmutated_copy_passes_the_battery():
    with tempfile.TemporaryDirectory() as d:
        lib = oracle.load_library(_compile(open(SRC).read(), d))
        assert _first_failing_pin(lib) is None


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
