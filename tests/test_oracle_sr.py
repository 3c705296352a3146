"""Pins of the oracle's stochastic bf16 rounding of the moments (CPU only).

The rounding is pinned by its exact distribution: over all 2^16 random words
a value rounds up (in magnitude) exactly (dropped bits) times, so the mean of
the rounded values is the value itself.  The random bits are pinned by the
published SplitMix64 sequence and by independence: the round-up decisions of
m and v, of neighbouring elements, of successive steps and of two seeds must
be uncorrelated.  The step itself is pinned to the round-to-nearest bf16-moment
step (same master and parameter after a first step; moments one of the two
bf16 neighbours of the exact value) and checked to be unbiased.
"""
import numpy as np
import pytest

import oracle

F32 = np.float32
ALL_R = np.arange(1 << 16, dtype=np.uint32)


def _bits(x):
    return np.asarray(x, F32).view(np.uint32)


def _f(u):
    return np.asarray(u, np.uint32).view(F32)


def test_generator_is_the_published_splitmix64():
    """SplitMix64 seeded with 0 (Steele, Lea and Flood 2014): the first three
    outputs of the reference generator."""
    assert [oracle.splitmix64(0, i) for i in range(3)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def _values():
    rng = np.random.default_rng(3)
    xs = [rng.normal(0, 1, 40) * 10.0 ** rng.integers(-30, 30, 40)]
    xs.append(np.array([1.0, -1.0, 3.0, 1e-3, -2.5e-5, 6.5e4], F32))
    base = _bits(np.array([1.5, -7.25, 1e-20, -3e30], F32)) & 0xffff0000
    for low in (0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFE, 0xFFFF):
        xs.append(_f(base | low))
    xs.append(_f(np.array([0x00000001, 0x0000ABCD, 0x8000FFFF, 0x007FFFFF], np.uint32)))  # denormals
    return np.concatenate([np.asarray(x, F32) for x in xs])


def test_rounding_distribution_is_exact():
    """For every value and all 2^16 random words: the result is the bf16
    below the value in magnitude or the one above, it moves up exactly
    (dropped bits) times and never down again as the word grows, so the mean
    of the rounded values equals the value."""
    for x in _values():
        u = int(_bits(x))
        lo, low = u >> 16, u & 0xffff
        out = oracle.bf16_sr(np.full(1 << 16, x, F32), ALL_R).astype(np.int64)
        assert set(np.unique(out)) <= {lo, lo + 1}, hex(u)
        assert int((out == lo + 1).sum()) == low, hex(u)
        assert np.all(np.diff(out) >= 0), hex(u)
        assert out[0] == lo  # r = 0 truncates
        vals = _f((out.astype(np.uint32) << 16)).astype(np.float64)
        if np.all(np.isfinite(vals)):
            assert vals.mean() == float(x), (hex(u), vals.mean(), float(x))


def test_specials():
    nans = _f(np.array([0x7FC00000, 0x7F800001, 0xFFC12345, 0x7FFFFFFF], np.uint32))
    for x in nans:
        assert np.all(oracle.bf16_sr(np.full(1 << 16, x, F32), ALL_R) == 0x7FC0)
    for x, want in ((np.inf, 0x7F80), (-np.inf, 0xFF80), (0.0, 0x0000), (-0.0, 0x8000)):
        assert np.all(oracle.bf16_sr(np.full(1 << 16, x, F32), ALL_R) == want)
    top = _f(np.array([0x7F7FFFFF], np.uint32))[0]  # largest finite: up is infinity
    out = oracle.bf16_sr(np.full(1 << 16, top, F32), ALL_R)
    assert int((out == 0x7F80).sum()) == 0xFFFF and int((out == 0x7F7F).sum()) == 1


def _segs(n):
    return [(0, True), (n // 3, False), (n // 3 + 7, True)]


def _first_step(n, k, seed, step=1, sr=True, grads=None):
    """One step from zero moments (t = `step`): (master, m, v, param, grads)."""
    rng = np.random.default_rng(11)
    w = rng.normal(0, 0.02, n).astype(F32)
    if grads is None:
        grads = [(rng.normal(0, 1e-3, n).astype(F32).view(np.uint32) >> 16).astype(np.uint16)
                 for _ in range(k)]
    m = np.zeros(n, np.uint16)
    v = np.zeros(n, np.uint16)
    p = np.zeros(n, np.uint16)
    hp = oracle.hparams()
    if sr:
        rc = oracle.shard_step_bf16mv_sr(w, m, v, p, grads, _segs(n), hp, step, seed)
    else:
        rc = oracle.shard_step_bf16mv(w, m, v, p, grads, _segs(n), hp, step)
    assert rc == 0
    return w, m, v, p, grads


def test_first_step_matches_round_to_nearest_step():
    """The weight update uses the unrounded new moments, so master and the
    parameter copy after a first step equal the round-to-nearest step's;
    each stored moment is one of the two bf16 values around the exact one,
    so it is within one bf16 step of the round-to-nearest moment."""
    n = 50_000
    w1, m1, v1, p1, g = _first_step(n, 2, seed=5)
    w0, m0, v0, p0, _ = _first_step(n, 2, seed=5, sr=False, grads=g)
    assert np.array_equal(w1.view(np.uint32), w0.view(np.uint32))
    assert np.array_equal(p1, p0)
    for a, b in ((m1, m0), (v1, v0)):
        assert np.abs(a.astype(np.int64) - b.astype(np.int64)).max() <= 1
        assert (a != b).any()


def _exact_moments(grads):
    """m' and v' after a first step from zero moments, k = 1, grad_scale 1:
    (1 - beta1) * g and (1 - beta2) * (g * g), one binary32 rounding each."""
    hp = oracle.hparams()
    g = _f(grads[0].astype(np.uint32) << 16)
    c1, c2 = F32(1) - F32(hp.beta1), F32(1) - F32(hp.beta2)
    return c1 * g, c2 * (g * g)


def _round_ups(stored, exact):
    """Indicator: the stored bf16 is the one above the exact value in magnitude."""
    return (stored.astype(np.int64) == (_bits(exact).astype(np.int64) >> 16) + 1)


def test_first_step_is_unbiased():
    """Over 2^20 elements the number of moments rounded up matches the sum of
    their probabilities (dropped bits / 2^16) within five standard deviations."""
    n = 1 << 20
    _, m, v, _, g = _first_step(n, 1, seed=123)
    mx, vx = _exact_moments(g)
    for stored, exact in ((m, mx), (v, vx)):
        prob = (_bits(exact) & 0xffff).astype(np.float64) / 65536.0
        ups = _round_ups(stored, exact)
        down = stored.astype(np.int64) == (_bits(exact).astype(np.int64) >> 16)
        assert np.all(ups | down)
        sd = np.sqrt((prob * (1 - prob)).sum())
        assert abs(ups.sum() - prob.sum()) < 5 * sd, (ups.sum(), prob.sum(), sd)


def _resid(stored, exact):
    """Round-up indicator minus its probability (dropped bits / 2^16): zero
    mean, and uncorrelated between two roundings with independent bits, even
    where both use the same probabilities."""
    prob = (_bits(exact) & 0xffff).astype(np.float64) / 65536.0
    return _round_ups(stored, exact).astype(np.float64) - prob


def _corr(a, b):
    return float(np.corrcoef(a, b)[0, 1])


def test_random_streams_are_independent():
    """Round-up decisions (through the step, from known thresholds) of m and
    v of one element, of neighbouring elements, of the same element at two
    steps and under two seeds are uncorrelated (|r| < 0.01 over 2^20 pairs,
    about ten standard errors; a shared stream gives correlations far above
    that)."""
    n = 1 << 20
    _, m, v, _, g = _first_step(n, 1, seed=99)
    mx, vx = _exact_moments(g)
    rm, rv = _resid(m, mx), _resid(v, vx)
    assert abs(_corr(rm, rv)) < 0.01
    assert abs(_corr(rm[:-1], rm[1:])) < 0.01
    assert abs(_corr(rm[:-4], rm[4:])) < 0.01
    # the same thresholds at step 2 (zero moments: m' does not depend on t)
    _, m2, _, _, _ = _first_step(n, 1, seed=99, step=2, grads=g)
    assert abs(_corr(rm, _resid(m2, mx))) < 0.01
    _, m3, _, _, _ = _first_step(n, 1, seed=100, grads=g)
    assert abs(_corr(rm, _resid(m3, mx))) < 0.01
    _, m4, _, _, _ = _first_step(n, 1, seed=99, grads=g)
    assert np.array_equal(m4, m)  # the same seed and step repeat exactly


def test_random_bits_are_uniform():
    """The 16-bit words of one stream: each of 16 equal bins within 5 sd."""
    n = 1 << 16
    r = np.array([oracle.sr_bits(7, 3, 0, i) for i in range(n)], np.int64)
    assert r.min() >= 0 and r.max() < 65536
    counts = np.bincount(r >> 12, minlength=16)
    sd = np.sqrt(n / 16 * (1 - 1 / 16))
    assert np.all(np.abs(counts - n / 16) < 5 * sd), counts


def test_a_window_takes_the_bits_of_its_place_in_the_shard():
    """Replaying elements [lo, hi) alone, with index0 = lo, gives exactly the
    whole run's values there (the step is elementwise and each element's
    random bits depend on its shard index); with index0 = 0 it does not."""
    n, lo, hi = 40_000, 12_345, 23_457
    rng = np.random.default_rng(8)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    g = [(rng.normal(0, 1e-3, n).astype(F32).view(np.uint32) >> 16).astype(np.uint16)]
    segs = [(0, True), (20_000, False)]
    hp = oracle.hparams()
    full = [w0.copy(), np.zeros(n, np.uint16), np.zeros(n, np.uint16), np.zeros(n, np.uint16)]
    win = [w0[lo:hi].copy(), np.zeros(hi - lo, np.uint16), np.zeros(hi - lo, np.uint16),
           np.zeros(hi - lo, np.uint16)]
    shifted = [x.copy() for x in win]
    wsegs = [(0, True), (20_000 - lo, False)]
    for t in (1, 2, 3):
        assert oracle.shard_step_bf16mv_sr(*full, g, segs, hp, t, 31) == 0
        assert oracle.shard_step_bf16mv_sr(*win, [g[0][lo:hi]], wsegs, hp, t, 31, lo) == 0
        assert oracle.shard_step_bf16mv_sr(*shifted, [g[0][lo:hi]], wsegs, hp, t, 31, 0) == 0
    for a, b in zip(full, win):
        assert np.array_equal(a[lo:hi].view(np.uint8), b.view(np.uint8))
    assert not np.array_equal(shifted[1], win[1])
