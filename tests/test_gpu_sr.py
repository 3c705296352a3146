"""The bf16-moment steps with stochastic rounding (zs_shard_step_bf16mv_sr and
its packed form) through the C ABI, against the oracle bit for bit.

The random bits are a function of (seed, step, moment, shard index) only, so
the kernel must reproduce the oracle exactly, for every size, partial count,
launch shape (one or two sub-windows per wavefront) and bias-correction path.
"""
import numpy as np
import pytest

import oracle
import sharded_mixed_precision_shard_amd as zs
import synth
from tests import _gpu_harness as H

pytestmark = pytest.mark.gpu

F32 = np.float32
SIZES = [1, 7, 255, 256, 257, 1023, 1025, 4097, 10007, 65539]


@pytest.fixture(scope="module")
def gpu():
    import torch
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    assert zs.zs_init(0) == zs.ZS_OK
    yield torch
    torch.cuda.synchronize()


def _dev(torch, a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).cuda()
    return torch.from_numpy(a.copy()).cuda()


def _bf16(x):
    return (np.asarray(x, F32).view(np.uint32) >> 16).astype(np.uint16)


def _segments(rng, n):
    segs, a = [], 0
    while a < n:
        segs.append((a, bool(rng.random() < 0.5)))
        a += int(rng.integers(1, 8)) if rng.random() < 0.4 else int(rng.integers(8, 3000))
    return segs


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("k", [1, 3, 16])
def test_bf16mv_sr_matches_oracle_and_its_packed_form(gpu, n, k):
    """Ten steps from non-zero moments: the separate-array and the packed
    stochastic steps equal the oracle bit for bit (and so each other)."""
    torch = gpu
    rng = np.random.default_rng(1300 + n * 3 + k)
    seed = int(rng.integers(0, 2 ** 63)) * 2 + 1
    segs = _segments(rng, n)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    m0 = _bf16(rng.normal(0, 1e-3, n))
    v0 = _bf16(rng.normal(0, 1e-3, n) ** 2)
    ref = [w0.copy(), m0.copy(), v0.copy(), np.zeros(n, np.uint16)]
    dw, dm, dv = _dev(torch, w0), _dev(torch, m0), _dev(torch, v0)
    dp = torch.zeros(n, dtype=torch.int16, device="cuda")
    dstate = _dev(torch, H.pack16_host(w0, m0, v0))
    pp = torch.zeros(n, dtype=torch.int16, device="cuda")
    table = H.segment_tensor(segs, "cuda")
    st = zs.seg_table(table)
    hpo, hpz = oracle.hparams(), zs.hparams()
    s = torch.cuda.current_stream()
    for t in range(1, 11):
        gs = [_bf16(rng.normal(0, 1e-3, n)) for _ in range(k)]
        dgs = [_dev(torch, g) for g in gs]
        zs.zs_shard_step_bf16mv_sr(dw, dm, dv, dp, dgs, k, n, st, hpz, t, seed, s)
        zs.zs_shard_step_packed_bf16mv_sr(dstate, pp, dgs, k, n, st, hpz, t, seed, s)
        assert oracle.shard_step_bf16mv_sr(*ref, gs, segs, hpo, t, seed) == 0
    torch.cuda.synchronize()
    got = (dw.cpu().numpy(), dm.cpu().numpy().view(np.uint16), dv.cpu().numpy().view(np.uint16),
           dp.cpu().numpy().view(np.uint16))
    assert H.assert_parity(got, ref, "bf16mv_sr n=%d k=%d" % (n, k)), "not bitwise"
    pk = H.unpack16_host(dstate.cpu().numpy(), n) + (pp.cpu().numpy().view(np.uint16),)
    assert H.assert_parity(pk, ref, "packed_bf16mv_sr n=%d k=%d" % (n, k)), "not bitwise"


def test_seed_and_rounding_change_only_what_they_should(gpu):
    """Two seeds give different moments but, after a first step from zero
    moments, the same master and parameters as the round-to-nearest step;
    the same seed gives the same bits again."""
    torch = gpu
    n, k = 100_003, 2
    rng = np.random.default_rng(5)
    segs = _segments(rng, n)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    gs = [_dev(torch, _bf16(rng.normal(0, 1e-3, n))) for _ in range(k)]
    table = H.segment_tensor(segs, "cuda")
    st, hp = zs.seg_table(table), zs.hparams()
    outs = {}
    for name, seed in (("a", 1), ("b", 2), ("a2", 1), ("rne", None)):
        w = _dev(torch, w0)
        m = torch.zeros(n, dtype=torch.int16, device="cuda")
        v = torch.zeros(n, dtype=torch.int16, device="cuda")
        p = torch.zeros(n, dtype=torch.int16, device="cuda")
        if seed is None:
            zs.zs_shard_step_bf16mv(w, m, v, p, gs, k, n, st, hp, 1)
        else:
            zs.zs_shard_step_bf16mv_sr(w, m, v, p, gs, k, n, st, hp, 1, seed)
        torch.cuda.synchronize()
        outs[name] = [x.cpu().numpy() for x in (w, m, v, p)]
    for j in (0, 3):
        assert np.array_equal(outs["a"][j].view(np.uint8), outs["rne"][j].view(np.uint8))
    for j in (1, 2):
        assert not np.array_equal(outs["a"][j], outs["b"][j])
        assert np.abs(outs["a"][j].astype(np.int64) - outs["rne"][j].astype(np.int64)).max() <= 1
    for x, y in zip(outs["a"], outs["a2"]):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def _sr_shard_windows(torch, name, variant, window, max_boundaries):
    """A model-shaped shard over its workload's steps (pre-warm included):
    windows at segment boundaries, both ends and at random equal the oracle
    replaying them with their shard indices."""
    w = synth.workload(name)
    free, _ = torch.cuda.mem_get_info()
    need = w.n * (8 + 4 + 2 + 2 * w.k) + (1 << 30)
    if free < need:
        pytest.skip("needs %.1f GB of free device memory" % (need / 1e9))
    ts = list(range(1, w.prewarm_steps + 1)) + w.step_ts()
    ds = H.DeviceShard(w, variant)
    for t in ts:
        ds.fill_grads(t)
        ds.step(t)
    torch.cuda.synchronize()
    wins = H.boundary_windows(w, window, max_boundaries=max_boundaries, n_random=4, seed=9)
    got = [ds.window(lo, hi) for lo, hi in wins]
    ds.free()
    for (lo, hi), g in zip(wins, got):
        ref = H.oracle_window(w, lo, hi, ts, variant="bf16mv_sr")
        assert H.assert_parity(g, ref, "%s %s [%d,%d)" % (name, variant, lo, hi)), "not bitwise"
    print("%s %s: %d windows bitwise equal" % (name, variant, len(wins)), flush=True)


@pytest.mark.parametrize("variant", ["bf16mv_sr", "packed_bf16mv_sr"])
def test_70b_sr_windows(gpu, variant):
    """The 70B-shaped shard (two sub-windows per wavefront), t = 10000..10002."""
    w = synth.workload("70b")
    assert zs.zs_launch_plan(w.k, w.n, variant)["window_quads"] == 2
    _sr_shard_windows(gpu, "70b", variant, 1 << 14, 16)


@pytest.mark.parametrize("variant", ["bf16mv_sr", "packed_bf16mv_sr"])
def test_175b_sr_windows(gpu, variant):
    """The 175B-shaped shard (one sub-window per wavefront, k = 2, t = 1..5)."""
    w = synth.workload("175b")
    assert zs.zs_launch_plan(w.k, w.n, variant)["window_quads"] == 1
    _sr_shard_windows(gpu, "175b", variant, 1 << 18, 16)


@pytest.mark.parametrize("variant", ["bf16mv_sr", "packed_bf16mv_sr"])
def test_7b_sr_windows(gpu, variant):
    """The 7B-shaped shard (k = 8, heavy-tailed partials, 100 pre-warm steps
    then 10)."""
    _sr_shard_windows(gpu, "7b", variant, 1 << 12, 12)


@pytest.mark.parametrize("variant", ["bf16mv_sr", "packed_bf16mv_sr"])
def test_prepared_sr_call_matches_the_plain_call(gpu, variant):
    torch = gpu
    n, k, seed = 70_001, 3, 0xFFFFFFFFFFFFFFFF
    rng = np.random.default_rng(19)
    segs = _segments(rng, n)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    z = np.zeros(n, np.uint16)
    table = H.segment_tensor(segs, "cuda")
    st, hp = zs.seg_table(table), zs.hparams()
    gs = [_dev(torch, _bf16(rng.normal(0, 1e-2, n))) for _ in range(k)]
    pa = torch.zeros(n, dtype=torch.int16, device="cuda")
    pb = torch.zeros(n, dtype=torch.int16, device="cuda")
    if variant == "packed_bf16mv_sr":
        a, b = _dev(torch, H.pack16_host(w0, z, z)), _dev(torch, H.pack16_host(w0, z, z))
        call = zs.ShardStep(a, None, None, pa, gs, n, st, hp, variant=variant, seed=seed)
        plain = lambda t: zs.zs_shard_step_packed_bf16mv_sr(b, pb, gs, k, n, st, hp, t, seed)  # noqa
        bufs = [(a, b)]
    else:
        a = [_dev(torch, w0), _dev(torch, z), _dev(torch, z)]
        b = [_dev(torch, w0), _dev(torch, z), _dev(torch, z)]
        call = zs.ShardStep(*a, pa, gs, n, st, hp, variant=variant, seed=seed)
        plain = lambda t: zs.zs_shard_step_bf16mv_sr(*b, pb, gs, k, n, st, hp, t, seed)  # noqa
        bufs = list(zip(a, b))
    for t in (1, 2, 3):
        call(t)
        plain(t)
    torch.cuda.synchronize()
    for x, y in bufs + [(pa, pb)]:
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    c = _dev(torch, H.pack16_host(w0, z, z))
    with pytest.raises(ValueError, match="needs a seed"):
        zs.ShardStep(c, None, None, pa, gs, n, st, hp, variant="packed_bf16mv_sr")
    with pytest.raises(ValueError, match="stochastic-rounding forms only"):
        zs.ShardStep(c, None, None, pa, gs, n, st, hp, variant="packed_bf16mv", seed=3)
    with pytest.raises(ValueError, match="unsigned 64-bit"):
        zs.zs_shard_step_packed_bf16mv_sr(c, pb, gs, k, n, st, hp, 1, -1)
    with pytest.raises(ValueError, match="unsigned 64-bit"):
        zs.zs_shard_step_packed_bf16mv_sr(c, pb, gs, k, n, st, hp, 1, 2 ** 64)
