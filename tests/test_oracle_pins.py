"""Pins of the CPU oracle to what the pages and the mathematics fix.

Each test ties the oracle to something other than itself: values the pages
print, closed forms of Adam's recurrences, exact invariants (power-of-two
scaling, the bias-correction limit), torch's library AdamW and bf16
conversion, and brute force on small integers.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import accounting
from tests.conftest import read_golden

F32 = np.float32


def _state(n, w=None):
    w = np.zeros(n, F32) if w is None else np.asarray(w, F32).copy()
    return w, np.zeros(n, F32), np.zeros(n, F32), np.zeros(n, np.uint16)


def _bf16(vals):
    """Exactly representable values -> bf16 bit patterns (checked exact)."""
    f = np.asarray(vals, F32)
    h = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_to_f32(h), f), "value not exact in bf16"
    return h


def _reduce_via_m(partials):
    """Run one step with beta1 = 0 so that m' is the reduced gradient itself
    (c1 = 1, bc1 = 1), and return m'."""
    n = len(partials[0])
    w, m, v, p = _state(n)
    hp = oracle.hparams(lr=0.0, beta1=0.0, beta2=0.5, eps=1.0, weight_decay=0.0)
    assert oracle.shard_step(w, m, v, p, [_bf16(x) for x in partials], [(0, False)], hp, 1) == 0
    return m


# ---------------------------------------------------------------- the reduce

def test_reduce_scatter_exercise_values():
    """Four ranks' vectors reduce-scattered: rank r's shard is element r of the
    sum; 28, 32, 36, 40 as printed in the exercise answer."""
    g = read_golden("reduce_scatter_exercise.txt")
    partials = [g["input rank%d" % r] for r in range(4)]
    for r in range(4):
        # rank r's shard is element r of every partial: a one-element shard, k = 4
        shard_partials = [[p[r]] for p in partials]
        m = _reduce_via_m(shard_partials)
        assert m[0] == g["reduce_scatter rank%d" % r][0]
    full = _reduce_via_m(partials)
    assert full.tolist() == g["all_reduce"]


def test_ring_demo_values():
    g = read_golden("ring_allreduce_demo.txt")
    partials = [g["device%d" % r] for r in range(4)]
    assert _reduce_via_m(partials).tolist() == g["all_reduce"]


def test_reduce_brute_force_small_integers():
    """Integer partials whose fp32 sums are exact: the reduce is the exact sum
    for every k up to 16."""
    rng = np.random.default_rng(1)
    for k in range(1, 17):
        parts = rng.integers(-256, 257, size=(k, 37)).astype(F32)
        m = _reduce_via_m(list(parts))
        assert np.array_equal(m, parts.astype(np.int64).sum(0).astype(F32))


def test_reduce_is_a_left_fold():
    """1 + 2^-24 + 2^-24 folded left stays 1 (each add ties to even); another
    order would give 1 + 2^-23.  Pins the fixed j = 0..k-1 order."""
    tiny = 2.0 ** -24
    m = _reduce_via_m([[1.0], [tiny], [tiny]])
    assert m[0] == F32(1.0)
    m = _reduce_via_m([[tiny], [tiny], [1.0]])
    assert m[0] == F32(1.0 + 2.0 ** -23)


def test_grad_scale_multiplies_after_the_sum():
    n = 5
    parts = [_bf16([1.0, 2.0, 3.0, -4.0, 0.5]), _bf16([3.0, 2.0, 1.0, 4.0, 0.25])]
    w, m, v, p = _state(n)
    hp = oracle.hparams(lr=0.0, beta1=0.0, beta2=0.5, eps=1.0, weight_decay=0.0, grad_scale=0.25)
    oracle.shard_step(w, m, v, p, parts, [(0, True)], hp, 1)
    assert m.tolist() == [1.0, 1.0, 1.0, 0.0, 0.1875]


# ------------------------------------------------------- the Adam recurrence

def test_bias_correction_scalars():
    hp = oracle.hparams(lr=1e-3, beta1=0.9, beta2=0.95, weight_decay=0.1)
    c1, c2, bc1, bc2, df = oracle.scalars(hp, 1)
    assert c1 == F32(1.0) - F32(0.9) and c2 == F32(1.0) - F32(0.95)
    # at t = 1 the correction equals 1 - beta exactly
    assert bc1 == c1 and bc2 == c2
    # t = 2: 1 - beta^2 to within half an ulp of binary32
    _, _, bc1, bc2, _ = oracle.scalars(hp, 2)
    assert abs(float(bc1) - (1 - float(F32(0.9)) ** 2)) <= 2.0 ** -24 * float(bc1)
    assert abs(float(bc2) - (1 - float(F32(0.95)) ** 2)) <= 2.0 ** -24 * float(bc2)
    # t -> infinity: beta^t vanishes below half an ulp of 1, corrections are exactly 1
    _, _, bc1, bc2, _ = oracle.scalars(hp, 10000)
    assert bc1 == F32(1.0) and bc2 == F32(1.0)
    # decoupled decay factor 1 - lr*wd
    assert abs(float(df) - (1 - 1e-4)) < 1e-7


def test_step1_update_is_lr_times_sign():
    """First step with wd = 0: m^ = g, v^ = g^2, so the move is
    lr * g / (|g| + eps), i.e. about lr * sign(g)."""
    rng = np.random.default_rng(2)
    n = 4096
    w0 = rng.normal(0, 0.02, n).astype(F32)
    g = (rng.normal(0, 0.01, n).astype(F32).view(np.uint32) >> 16).astype(np.uint16)
    gf = oracle.bf16_to_f32(g).astype(np.float64)
    for lr, eps in ((1e-3, 1e-8), (1e-3, 1e-3), (0.05, 1e-8)):
        w, m, v, p = _state(n, w0)
        hp = oracle.hparams(lr=lr, beta1=0.9, beta2=0.95, eps=eps, weight_decay=0.0)
        assert oracle.shard_step(w, m, v, p, [g], [(0, True)], hp, 1) == 0
        moved = w.astype(np.float64) - w0.astype(np.float64)
        expect = -lr * gf / (np.abs(gf) + eps)
        tol = 1e-5 * lr + 4 * np.spacing(np.abs(w0)).astype(np.float64)
        assert np.all(np.abs(moved - expect) <= tol)
        if eps == 1e-8:
            big = np.abs(gf) > 1e-4
            assert np.all(np.abs(np.abs(moved[big]) - lr) <= 1e-3 * lr)
            assert np.all(np.sign(moved[big]) == -np.sign(gf[big]))


def test_constant_gradient_closed_form():
    """g_t = c for all t: m^_t = c and v^_t = c^2 at every t, so each step moves
    w by lr*c/(|c|+eps); with decay w_T = df^T w_0 - lr*u*sum_{i<T} df^i."""
    n = 64
    rng = np.random.default_rng(3)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    c = _bf16(np.where(np.arange(n) % 2 == 0, 1.0, -0.0078125) * (1 + np.arange(n) % 5))
    cf = oracle.bf16_to_f32(c).astype(np.float64)
    T, lr, eps = 10, 1e-3, 1e-8
    for wd, decay in ((0.0, False), (0.1, True)):
        w, m, v, p = _state(n, w0)
        hp = oracle.hparams(lr=lr, beta1=0.9, beta2=0.95, eps=eps, weight_decay=wd)
        for t in range(1, T + 1):
            assert oracle.shard_step(w, m, v, p, [c], [(0, decay)], hp, t) == 0
        u = cf / (np.abs(cf) + eps)
        df = 1 - lr * wd
        expect = df ** T * w0.astype(np.float64) - lr * u * sum(df ** i for i in range(T))
        # each of the T steps rounds w once (half an ulp) plus relative 1e-6 on u
        tol = 1e-6 * lr * T + T * np.spacing(np.abs(w0)).astype(np.float64)
        assert np.all(np.abs(w - expect) <= tol)
        # the moments are the geometric sums of the constant input
        assert np.allclose(m, cf * (1 - 0.9 ** T), rtol=1e-5)
        assert np.allclose(v, cf * cf * (1 - 0.95 ** T), rtol=1e-5)


def test_zero_gradient_exact():
    """g = 0, m = v = 0: u = 0/(0+eps) = 0, so undecayed weights are bitwise
    unchanged and decayed ones are w*df exactly; moments stay 0."""
    n = 1000
    rng = np.random.default_rng(4)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    segs = [(0, True), (300, False), (301, True), (700, False)]
    mask = np.zeros(n, bool)
    mask[0:300] = True
    mask[301:700] = True
    w, m, v, p = _state(n, w0)
    hp = oracle.hparams(lr=1e-3, weight_decay=0.1)
    _, _, _, _, df = oracle.scalars(hp, 1)
    oracle.shard_step(w, m, v, p, [np.zeros(n, np.uint16)] * 3, segs, hp, 1)
    assert np.array_equal(w[~mask], w0[~mask])
    assert np.array_equal(w[mask], w0[mask] * df)
    assert not m.any() and not v.any()


def test_zero_padding_stays_zero():
    """Zero padding (state and partials all +0, decay off) stays +0 forever."""
    n = 17
    w, m, v, p = _state(n)
    hp = oracle.hparams()
    for t in range(1, 11):
        oracle.shard_step(w, m, v, p, [np.zeros(n, np.uint16)] * 2, [(0, False)], hp, t)
    for a in (w, m, v):
        assert np.all(a.view(np.uint32) == 0)
    assert np.all(p == 0)


def test_power_of_two_scaling_invariance():
    """With eps = 0, scaling every partial (and the moments) by 2^s scales m by
    2^s and v by 2^2s exactly and leaves the weights bitwise unchanged."""
    n = 2000
    rng = np.random.default_rng(5)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    parts = [rng.normal(0, 1e-3, n).astype(F32) for _ in range(3)]
    for s in (-7, 5, 20):
        wa, ma, va, pa = _state(n, w0)
        wb, mb, vb, pb = _state(n, w0)
        hp = oracle.hparams(lr=1e-3, eps=0.0, weight_decay=0.1)
        for t in range(1, 6):
            ga = [((x * F32(1 + 0.1 * t)).view(np.uint32) >> 16).astype(np.uint16)
                  for x in parts]
            gb = [_bf16(oracle.bf16_to_f32(h) * F32(2.0 ** s)) for h in ga]
            oracle.shard_step(wa, ma, va, pa, ga, [(0, True)], hp, t)
            oracle.shard_step(wb, mb, vb, pb, gb, [(0, True)], hp, t)
            # eps = 0 makes 0/0 = NaN wherever m = v = 0 (the partials cancel):
            # the same elements on both sides
            assert np.array_equal(wa, wb, equal_nan=True)
            assert np.array_equal(ma * F32(2.0 ** s), mb)
            assert np.array_equal(va * F32(2.0 ** (2 * s)), vb)
        assert np.isnan(wa).sum() <= 2


def test_bias_correction_limit_equals_uncorrected_step():
    """At t = 10000 both corrections are exactly 1, so the step equals the
    same step with beta1, beta2 corrections removed: pinned by comparing with
    a step at t = 10^6 (also exactly 1)."""
    n = 3000
    rng = np.random.default_rng(6)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    m0 = rng.normal(0, 1e-4, n).astype(F32)
    v0 = np.abs(rng.normal(0, 1e-7, n)).astype(F32)
    g = (rng.normal(0, 1e-3, n).astype(F32).view(np.uint32) >> 16).astype(np.uint16)
    hp = oracle.hparams(lr=3e-4)
    outs = []
    for t in (10000, 10001, 10 ** 6):
        w, m, v, p = w0.copy(), m0.copy(), v0.copy(), np.zeros(n, np.uint16)
        oracle.shard_step(w, m, v, p, [g], [(0, True)], hp, t)
        outs.append((w, m, v, p))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)
    # and with beta = 0.999 the limit is not reached at t = 10000
    _, _, bc1, bc2, _ = oracle.scalars(oracle.hparams(beta1=0.999, beta2=0.999), 10000)
    assert bc1 < 1.0 and abs(float(bc1) - (1 - 0.999 ** 10000)) < 1e-6


def test_matches_torch_adamw_float64():
    """Library cross-check: torch.optim.AdamW (CPU, float64, decoupled decay
    w*(1-lr*wd)) on the same fp32 inputs.  Compares the accumulated move of w
    and the moments after 10 steps; decay on and off via two param groups."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    n = 3000
    for lr, b1, b2, eps, wd in ((1e-3, 0.9, 0.95, 1e-8, 0.1), (3e-4, 0.8, 0.999, 1e-3, 0.3),
                                (1e-2, 0.0, 0.5, 1e-6, 0.0)):
        w0 = rng.normal(0, 0.02, n).astype(F32)
        segs = [(0, True), (1000, False), (2000, True)]
        dec = np.zeros(n, bool)
        dec[:1000] = True
        dec[2000:] = True
        w, m, v, p = _state(n, w0)
        hp = oracle.hparams(lr, b1, b2, eps, wd)
        tw = torch.tensor(w0.astype(np.float64))
        pa = torch.nn.Parameter(tw[dec].clone())
        pb = torch.nn.Parameter(tw[~dec].clone())
        f = lambda x: float(F32(x))  # noqa: E731  the fp32 hparams, as float64
        opt = torch.optim.AdamW([{"params": [pa], "weight_decay": f(wd)},
                                 {"params": [pb], "weight_decay": 0.0}],
                                lr=f(lr), betas=(f(b1), f(b2)), eps=f(eps), foreach=False)
        for t in range(1, 11):
            g = (rng.normal(0, 1e-3, n).astype(F32).view(np.uint32) >> 16).astype(np.uint16)
            oracle.shard_step(w, m, v, p, [g], segs, hp, t)
            gt = torch.tensor(oracle.bf16_to_f32(g).astype(np.float64))
            pa.grad = gt[dec].clone()
            pb.grad = gt[~dec].clone()
            opt.step()
        ref_w = np.empty(n)
        ref_w[dec] = pa.detach().numpy()
        ref_w[~dec] = pb.detach().numpy()
        ref_m = np.empty(n)
        ref_v = np.empty(n)
        ref_m[dec] = opt.state[pa]["exp_avg"].numpy()
        ref_m[~dec] = opt.state[pb]["exp_avg"].numpy()
        ref_v[dec] = opt.state[pa]["exp_avg_sq"].numpy()
        ref_v[~dec] = opt.state[pb]["exp_avg_sq"].numpy()
        moved_o = w.astype(np.float64) - w0
        moved_t = ref_w - w0
        tol = 2e-5 * np.abs(moved_t) + 20 * np.spacing(np.abs(w0)).astype(np.float64)
        assert np.all(np.abs(moved_o - moved_t) <= tol), (lr, b1, b2, eps, wd)
        # m is a sum of zero-mean terms: absolute error of a few fp32 ulps of
        # the gradient scale (1e-3), relative error elsewhere
        assert np.allclose(m, ref_m, rtol=1e-5, atol=1e-9)
        assert np.allclose(v, ref_v, rtol=1e-5, atol=1e-16)


def test_nan_and_inf_propagate_per_element():
    n = 16
    w, m, v, p = _state(n, np.full(n, 0.5, F32))
    g = np.zeros(n, F32)
    g[3] = np.nan
    g[7] = np.inf
    h = (g.view(np.uint32) >> 16).astype(np.uint16)
    oracle.shard_step(w, m, v, p, [h], [(0, True)], oracle.hparams(), 1)
    bad = np.zeros(n, bool)
    bad[[3, 7]] = True
    assert np.all(np.isnan(w[bad])) and np.all(p[bad] == 0x7FC0)
    assert np.all(np.isfinite(w[~bad]))
    assert np.isnan(m[3]) and np.isinf(m[7]) and np.isinf(v[7])


# ------------------------------------------------------------------ the cast

def test_bf16_rne_matches_torch_on_every_non_nan_pattern():
    """All 2^32 binary32 patterns except NaNs: the oracle's cast equals torch's
    CPU float32 -> bfloat16 conversion (round to nearest even).  NaNs all map
    to the canonical 0x7FC0."""
    torch = pytest.importorskip("torch")
    from concurrent.futures import ThreadPoolExecutor
    chunk = 1 << 24

    def check(base):
        u = np.arange(chunk, dtype=np.uint32) + np.uint32(base)
        f = u.view(F32)
        ours = oracle.bf16_rne(f)
        ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = (u & np.uint32(0x7fffffff)) > np.uint32(0x7f800000)
        bad = (ours != ref) & ~nan
        bad_nan = (ours != 0x7FC0) & nan
        return base, int(bad.sum()), int(bad_nan.sum())

    torch.set_num_threads(1)
    try:
        with ThreadPoolExecutor(8) as ex:
            for base, nbad, nbad_nan in ex.map(check, range(0, 1 << 32, chunk)):
                assert nbad == 0 and nbad_nan == 0, hex(base)
    finally:
        torch.set_num_threads(8)


def test_bf16_rne_special_cases():
    vals = [(1.0, 0x3F80), (-2.0, 0xC000), (float("inf"), 0x7F80), (float("-inf"), 0xFF80),
            (0.0, 0x0000), (-0.0, 0x8000)]
    for x, h in vals:
        assert oracle.bf16_rne(np.array([x], F32))[0] == h
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert oracle.bf16_rne(np.array([1 + 2 ** -8], F32))[0] == 0x3F80
    assert oracle.bf16_rne(np.array([1 + 3 * 2 ** -8], F32))[0] == 0x3F82
    # the largest finite float rounds up to infinity
    assert oracle.bf16_rne(np.array([np.finfo(F32).max], F32))[0] == 0x7F80


# ------------------------------------------------------------- accounting

def test_accounting_pins():
    g = {k: v[0] for k, v in read_golden("zero_memory.txt").items()}
    assert accounting.bytes_per_param() == g["bytes_per_param"]
    assert accounting.optimizer_state_bytes_per_param() == g["optimizer_state_bytes_per_param"]
    psi, nd = g["ex6_psi"], int(g["ex6_nd"])
    assert math.isclose(accounting.ddp_bytes_per_gpu(psi), g["ex6_ddp_bytes"])
    assert math.isclose(accounting.zero1_bytes_per_gpu(psi, nd), g["ex6_zero1_bytes"])
    assert math.isclose(accounting.zero2_bytes_per_gpu(psi, nd), g["ex6_zero2_bytes"])
    assert math.isclose(accounting.zero3_bytes_per_gpu(psi, nd), g["ex6_zero3_bytes"])
    assert math.isclose((accounting.BF16_PARAM + accounting.BF16_GRAD) * 175e9,
                        g["gpt3_175b_param_grad_bytes"])
    assert math.isclose(accounting.optimizer_state_bytes_per_param() * 175e9,
                        g["gpt3_175b_adam_bytes"])
    n = accounting.transformer_params(int(g["gpt3_layers"]), int(g["gpt3_d"]))
    assert abs(n - g["gpt3_params_approx"]) / g["gpt3_params_approx"] < 0.005
    assert math.isclose(accounting.ddp_bytes_per_gpu(g["llama7b_psi"]), g["llama7b_ddp_bytes"])
    assert math.isclose(accounting.zero3_bytes_per_gpu(g["llama7b_psi"], int(g["llama7b_nd"])),
                        g["llama7b_zero3_bytes"])
    # traffic of one fused shard step: 26 + 2k bytes per parameter
    assert [accounting.shard_step_hbm_bytes_per_param(k) for k in (1, 2, 8)] == [28, 30, 42]


def test_shard_resident_bytes_pins():
    """Resident bytes per shard parameter: the fp32 state, the bf16 output
    and the k bf16 partials."""
    g = {k: v[0] for k, v in read_golden("zero_memory.txt").items()}
    # one partial is the one bf16 gradient of the page's five copies: 16 bytes
    assert accounting.shard_resident_bytes_per_param(1) == g["bytes_per_param"] == 16
    # hand-derived: k = 2 is 4 + 4 + 4 + 2 + 2 + 2 = 18 bytes; the 70B-shaped
    # rank-0 shard of 8,053,473,280 parameters then holds 144,962,519,040 bytes
    assert accounting.shard_resident_bytes_per_param(2) == 18
    assert accounting.shard_resident_bytes_per_param(2) * 8_053_473_280 == 144_962_519_040
    assert accounting.shard_resident_bytes_per_param(8) == 30
    # the buffers a shard step actually holds, counted from their dtypes
    n = 1000
    for k in (1, 2, 3, 16):
        bufs = [np.zeros(n, np.float32) for _ in range(3)] + [np.zeros(n, np.uint16)] + \
               [np.zeros(n, np.uint16) for _ in range(k)]
        assert sum(b.nbytes for b in bufs) == accounting.shard_resident_bytes_per_param(k) * n
    # what a step moves = what it holds + the fp32 state written back (12 B)
    for k in (1, 2, 8):
        assert accounting.shard_step_hbm_bytes_per_param(k) == \
            accounting.shard_resident_bytes_per_param(k) + 12


def test_resident_bytes_pins_catch_planted_mistakes(monkeypatch):
    """Each plausible slip in the resident-bytes formula fails the pins above."""
    good = accounting.shard_resident_bytes_per_param
    mistakes = [lambda k: 3 * 4 + 2 * k,          # the bf16 parameter copy dropped
                lambda k: 3 * 4 + 2 + 2,          # one partial whatever k is
                lambda k: 2 * 4 + 2 + 2 * k,      # one fp32 state array dropped
                lambda k: 3 * 4 + 4 + 2 * k,      # the parameter copy counted as fp32
                lambda k: 3 * 4 + 2 + 4 * k]      # partials counted as fp32
    for bad in mistakes:
        monkeypatch.setattr(accounting, "shard_resident_bytes_per_param", bad)
        try:
            test_shard_resident_bytes_pins()
        except AssertionError:
            continue
        finally:
            monkeypatch.setattr(accounting, "shard_resident_bytes_per_param", good)
        raise AssertionError("a planted mistake passed the pins")


# ---------------------------------------------------- argument validation

def test_oracle_rejects_invalid_arguments():
    n = 8
    w, m, v, p = _state(n)
    g = [np.zeros(n, np.uint16)]
    ok = oracle.hparams()
    assert oracle.shard_step(w, m, v, p, g, [(0, True)], ok, 0) == 2
    assert oracle.shard_step(w, m, v, p, [], [(0, True)], ok, 1) == 2
    assert oracle.shard_step(w, m, v, p, g, [(1, True)], ok, 1) == 2
    assert oracle.shard_step(w, m, v, p, g, [(0, True), (5, False), (3, True)], ok, 1) == 2
    assert oracle.shard_step(w, m, v, p, g, [(0, True)], oracle.hparams(beta1=1.0), 1) == 2
    assert oracle.shard_step(w, m, v, p, g, [(0, True)], oracle.hparams(eps=-1.0), 1) == 2
    assert oracle.shard_step(w, m, v, p, g, [(0, True)], oracle.hparams(lr=float("nan")), 1) == 2
