"""Pins of the oracle's step variants: int8 block-quantized partials and bf16
moments.  Each variant is tied to the pinned ordinary step where the two must
agree exactly, plus hand-worked closed forms."""
import numpy as np
import pytest

import oracle
from tests.conftest import read_golden

F32 = np.float32


def _state(n, w=None):
    w = np.zeros(n, F32) if w is None else np.asarray(w, F32).copy()
    return w, np.zeros(n, F32), np.zeros(n, F32), np.zeros(n, np.uint16)


def _bf16_of(x):
    h = (np.asarray(x, F32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_to_f32(h), np.asarray(x, F32)), "not exact in bf16"
    return h


# ------------------------------------------------------- int8 partials

def test_q8grad_reduce_scatter_exercise():
    """Integer partials with unit scales: beta1 = 0 exposes the reduced
    gradient, 28 32 36 40 as in the lecture notes' exercise 1."""
    g = read_golden("reduce_scatter_exercise.txt")
    qs = [np.array(g["input rank%d" % r], np.int8) for r in range(4)]
    ss = [np.ones(1, F32) for _ in range(4)]
    w, m, v, p = _state(4)
    hp = oracle.hparams(lr=0.0, beta1=0.0, beta2=0.5, eps=1.0, weight_decay=0.0)
    assert oracle.shard_step_q8grad(w, m, v, p, qs, ss, [(0, False)], hp, 1) == 0
    assert m.tolist() == g["all_reduce"]


@pytest.mark.parametrize("grad_scale", [1.0, 0.125, 3.0])
def test_q8grad_equals_bf16_path_on_exact_partials(grad_scale):
    """With power-of-two block scales every q*scale is exact in bf16, so the
    int8 path must equal the ordinary step fed those bf16 partials, bitwise,
    over 10 steps, ragged n, several segments, varying scales and grad_scale."""
    rng = np.random.default_rng(21)
    n, k, block = 1000, 3, 256
    nb = -(-n // block)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    segs = [(0, True), (300, False), (301, True), (777, False)]
    a = _state(n, w0)
    b = _state(n, w0)
    hp = oracle.hparams(grad_scale=grad_scale)
    for t in range(1, 11):
        qs = [rng.integers(-127, 128, n).astype(np.int8) for _ in range(k)]
        ss = [(2.0 ** rng.integers(-16, -8, nb)).astype(F32) for _ in range(k)]
        deq = [_bf16_of(q.astype(F32) * np.repeat(s, block)[:n]) for q, s in zip(qs, ss)]
        assert oracle.shard_step_q8grad(*a, qs, ss, segs, hp, t, block) == 0
        assert oracle.shard_step(*b, deq, segs, hp, t) == 0
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_q8grad_products_round_once():
    """A scale that is not a power of two: partial = q*s rounded once in fp32,
    then the left fold (pinned with beta1 = 0 against float32 arithmetic)."""
    q0 = np.array([3, -7, 127, 1], np.int8)
    q1 = np.array([5, 2, -127, 0], np.int8)
    s0 = np.array([0.1], F32)
    s1 = np.array([0.3], F32)
    w, m, v, p = _state(4)
    hp = oracle.hparams(lr=0.0, beta1=0.0, beta2=0.5, eps=1.0, weight_decay=0.0)
    oracle.shard_step_q8grad(w, m, v, p, [q0, q1], [s0, s1], [(0, False)], hp, 1)
    want = (q0.astype(F32) * s0[0]) + (q1.astype(F32) * s1[0])
    assert np.array_equal(m, want.astype(F32))


# ------------------------------------------------------- bf16 moments

def test_bf16mv_first_step_equals_fp32_path():
    """From zero moments (exact in bf16) one step gives the same weights as the
    fp32-moment step and moments equal to its rounded moments."""
    rng = np.random.default_rng(22)
    n = 5000
    w0 = rng.normal(0, 0.02, n).astype(F32)
    g = [(rng.normal(0, 1e-3, n).astype(F32).view(np.uint32) >> 16).astype(np.uint16)
         for _ in range(2)]
    segs = [(0, True), (100, False), (2000, True)]
    hp = oracle.hparams()
    a = _state(n, w0)
    assert oracle.shard_step(*a, g, segs, hp, 1) == 0
    w = w0.copy()
    mb = np.zeros(n, np.uint16)
    vb = np.zeros(n, np.uint16)
    p = np.zeros(n, np.uint16)
    assert oracle.shard_step_bf16mv(w, mb, vb, p, g, segs, hp, 1) == 0
    assert np.array_equal(w.view(np.uint32), a[0].view(np.uint32))
    assert np.array_equal(p, a[3])
    assert np.array_equal(mb, oracle.bf16_rne(a[1]))
    assert np.array_equal(vb, oracle.bf16_rne(a[2]))


def test_bf16mv_closed_form_with_halving_betas():
    """beta1 = beta2 = 0.5, g = 1: m_t = v_t = 1 - 2^-t, exact in bf16 up to
    t = 8 (so both state precisions agree bitwise); at t = 9 the value
    1 - 2^-9 is a tie between 1 - 2^-8 and 1 and rounds to even, 1.0."""
    n = 8
    hp = oracle.hparams(lr=1e-3, beta1=0.5, beta2=0.5, eps=1e-8, weight_decay=0.0)
    one = _bf16_of(np.ones(n, F32))
    a = _state(n, np.full(n, 0.25, F32))
    w = np.full(n, 0.25, F32)
    mb = np.zeros(n, np.uint16)
    vb = np.zeros(n, np.uint16)
    p = np.zeros(n, np.uint16)
    for t in range(1, 9):
        oracle.shard_step(*a, [one], [(0, False)], hp, t)
        oracle.shard_step_bf16mv(w, mb, vb, p, [one], [(0, False)], hp, t)
        want = F32(1.0 - 2.0 ** -t)
        assert np.all(oracle.bf16_to_f32(mb) == want) and np.all(a[1] == want)
        assert np.array_equal(w, a[0])
    oracle.shard_step_bf16mv(w, mb, vb, p, [one], [(0, False)], hp, 9)
    assert np.all(mb == 0x3F80) and np.all(vb == 0x3F80)


def test_bf16mv_stays_close_to_fp32_path():
    """Ten steps on random partials: the weight trajectory differs from the
    fp32-moment one only by the bf16 rounding of the moments (relative 2^-9
    each, so |u| changes by about 2^-8 of itself per step)."""
    rng = np.random.default_rng(23)
    n = 20000
    w0 = rng.normal(0, 0.02, n).astype(F32)
    hp = oracle.hparams(lr=1e-3)
    a = _state(n, w0)
    w = w0.copy()
    mb = np.zeros(n, np.uint16)
    vb = np.zeros(n, np.uint16)
    p = np.zeros(n, np.uint16)
    for t in range(1, 11):
        g = [(rng.normal(0, 1e-3, n).astype(F32).view(np.uint32) >> 16).astype(np.uint16)]
        oracle.shard_step(*a, g, [(0, True)], hp, t)
        oracle.shard_step_bf16mv(w, mb, vb, p, g, [(0, True)], hp, t)
    d = np.abs(w.astype(np.float64) - a[0].astype(np.float64))
    assert d.max() <= 10 * 1e-3 * 2.0 ** -6
    # m is an average of zero-mean terms: compare on the scale of its magnitude
    dm = np.abs(oracle.bf16_to_f32(mb).astype(np.float64) - a[1])
    assert dm.max() <= 2.0 ** -7 * np.abs(a[1]).max()
    assert np.allclose(oracle.bf16_to_f32(vb), a[2], rtol=2 ** -6, atol=0)
