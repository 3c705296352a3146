"""GPU parity: the HIP shard step (through the C ABI) against the CPU oracle.

Bar: |d| <= 1e-6 * max(1, |x|) on fp32 master, m, v and <= 1 bf16 ulp on the
parameter copy, after every config's full step count (10 steps where the
config says so).  The kernel mirrors the oracle's operation order, so the
tests also report whether the results are bitwise equal (expected).
"""
import numpy as np
import pytest

import oracle
import sharded_mixed_precision_shard_amd as zs
import synth
from tests import _gpu_harness as H

pytestmark = pytest.mark.gpu

F32 = np.float32


@pytest.fixture(scope="module")
def gpu():
    import torch
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    rc = zs.zs_init(0)
    assert rc == zs.ZS_OK, zs.zs_status_string(rc)
    yield torch
    torch.cuda.synchronize()


def _dev(torch, a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).cuda()
    return torch.from_numpy(a.copy()).cuda()


def _run_both(torch, n, k, segs, steps, seed, hp_kw=None, cfg=None, w0=None, grads_fn=None,
              ref_segs=None, with_oracle=True):
    """Same inputs on GPU and oracle; returns (gpu outputs, oracle outputs).
    ref_segs: a different (valid) table for the oracle side; with_oracle=False
    skips the oracle (the second result is then None)."""
    hp_kw = hp_kw or {}
    w = synth.host_normal_f32(n, synth.stream_key(seed, 1, 0, 0), 0, n, 0.02) if w0 is None \
        else w0.copy()
    ref = [w.copy(), np.zeros(n, F32), np.zeros(n, F32), np.zeros(n, np.uint16)]
    dw, dm, dv = _dev(torch, w), _dev(torch, ref[1]), _dev(torch, ref[2])
    dp = torch.zeros(n, dtype=torch.int16, device="cuda")
    table = H.segment_tensor(segs, "cuda")
    hpo = oracle.hparams(**hp_kw)
    hpz = zs.hparams(**hp_kw)
    for t in steps:
        if grads_fn is None:
            gs = [synth.host_normal_bf16(n, synth.stream_key(seed, 2, j, t), 0, n, 0.01)
                  for j in range(k)]
        else:
            gs = grads_fn(t)
        dgs = [_dev(torch, g) for g in gs]
        if cfg is None:
            zs.zs_shard_step(dw, dm, dv, dp, dgs, k, n, zs.seg_table(table), hpz, t,
                             torch.cuda.current_stream())
        else:
            zs.zs_shard_step_cfg(dw, dm, dv, dp, dgs, k, n, zs.seg_table(table), hpz, t,
                                 torch.cuda.current_stream(), **cfg)
        if with_oracle:
            assert oracle.shard_step(*ref, gs, segs if ref_segs is None else ref_segs, hpo,
                                     t) == 0
    torch.cuda.synchronize()
    got = (dw.cpu().numpy(), dm.cpu().numpy(), dv.cpu().numpy(),
           dp.cpu().numpy().view(np.uint16))
    return got, (ref if with_oracle else None)


def _random_segments(rng, n, short_frac=0.5):
    segs, a = [], 0
    while a < n:
        segs.append((a, bool(rng.random() < 0.5)))
        a += int(rng.integers(1, 8)) if rng.random() < short_frac else int(rng.integers(8, 5000))
    return segs


# ---------------------------------------------------------------- ABI errors

def test_abi_rejects_bad_arguments(gpu):
    torch = gpu
    n = 1024
    f = [torch.zeros(n, dtype=torch.float32, device="cuda") for _ in range(3)]
    p = torch.zeros(n, dtype=torch.int16, device="cuda")
    g = [torch.zeros(n, dtype=torch.int16, device="cuda") for _ in range(2)]
    table = H.segment_tensor([(0, True)], "cuda")
    st = zs.seg_table(table)
    hp = zs.hparams()

    def call(*a, **kw):
        args = dict(master=f[0], m=f[1], v=f[2], param_bf16=p, grads=g, k=2, n=n, seg_table_=st,
                    hparams_=hp, step=1)
        args.update(kw)
        return zs.zs_shard_step(args["master"], args["m"], args["v"], args["param_bf16"],
                                args["grads"], args["k"], args["n"], args["seg_table_"],
                                args["hparams_"], args["step"], None, check=False)

    assert call() == zs.ZS_OK
    assert call(k=0, grads=[]) == zs.ZS_ERR_INVALID_ARGUMENT
    assert call(k=17, grads=(g * 9)[:17]) == zs.ZS_ERR_INVALID_ARGUMENT
    assert call(n=-1) == zs.ZS_ERR_INVALID_ARGUMENT
    assert call(step=0) == zs.ZS_ERR_INVALID_ARGUMENT
    assert call(master=0) == zs.ZS_ERR_INVALID_ARGUMENT
    assert call(grads=[g[0], 0]) == zs.ZS_ERR_INVALID_ARGUMENT
    assert call(hparams_=zs.hparams(beta1=1.0)) == zs.ZS_ERR_INVALID_ARGUMENT
    assert call(hparams_=zs.hparams(beta2=-0.1)) == zs.ZS_ERR_INVALID_ARGUMENT
    assert call(hparams_=zs.hparams(eps=-1e-8)) == zs.ZS_ERR_INVALID_ARGUMENT
    assert call(hparams_=zs.hparams(lr=float("inf"))) == zs.ZS_ERR_INVALID_ARGUMENT
    assert call(hparams_=zs.hparams(grad_scale=float("nan"))) == zs.ZS_ERR_INVALID_ARGUMENT
    assert call(seg_table_=zs.seg_table(table, 0)) == zs.ZS_ERR_INVALID_ARGUMENT
    assert call(seg_table_=zs.seg_table(table, zs.ZS_MAX_SEGMENTS + 1)) == \
        zs.ZS_ERR_TOO_MANY_SEGMENTS
    assert call(seg_table_=zs.seg_table(0, 1)) == zs.ZS_ERR_INVALID_ARGUMENT
    assert call(master=f[0].data_ptr() + 4, n=n - 4) == zs.ZS_ERR_MISALIGNED
    assert call(grads=[g[0], g[1].data_ptr() + 2], n=n - 8) == zs.ZS_ERR_MISALIGNED
    assert call(seg_table_=zs.seg_table(table.data_ptr() + 4, 1)) == zs.ZS_ERR_MISALIGNED
    assert call(v=f[1]) == zs.ZS_ERR_ALIASING
    assert call(param_bf16=f[0]) == zs.ZS_ERR_ALIASING
    assert call(grads=[g[0], p]) == zs.ZS_ERR_ALIASING
    assert call(m=f[0].data_ptr() + 2048, n=n) == zs.ZS_ERR_ALIASING
    assert call(grads=[g[0], g[0]]) == zs.ZS_OK  # partials may alias each other
    # n == 0 is a no-op even with null buffers
    assert call(n=0, master=0, m=0, v=0, param_bf16=0, grads=[0, 0]) == zs.ZS_OK
    assert call(hparams_=zs.hparams(), k=2, n=n, step=1,
                grads=g) == zs.ZS_OK
    torch.cuda.synchronize()
    assert zs.zs_status_string(zs.ZS_ERR_ALIASING) == "output buffers overlap"


def test_not_initialized_after_fini(gpu):
    torch = gpu
    n = 64
    f = [torch.zeros(n, dtype=torch.float32, device="cuda") for _ in range(3)]
    p = torch.zeros(n, dtype=torch.int16, device="cuda")
    g = torch.zeros(n, dtype=torch.int16, device="cuda")
    table = H.segment_tensor([(0, True)], "cuda")
    assert zs.zs_fini() == zs.ZS_OK
    rc = zs.zs_shard_step(f[0], f[1], f[2], p, [g], 1, n, zs.seg_table(table), zs.hparams(), 1,
                          None, check=False)
    assert rc == zs.ZS_ERR_NOT_INITIALIZED
    assert zs.zs_init(0) == zs.ZS_OK
    assert zs.zs_init(0) == zs.ZS_OK  # idempotent
    assert zs.zs_init(10 ** 6) == zs.ZS_ERR_INVALID_ARGUMENT


# ------------------------------------------------------------- generator twin

def test_device_generator_matches_host(gpu):
    torch = gpu
    n = 100_003
    key = synth.stream_key(77, synth.ROLE_GRAD, 5, 9)
    hkey = synth.stream_key(77, synth.ROLE_HEAVY, 5, 9)
    d16 = torch.empty(n, dtype=torch.int16, device="cuda")
    d32 = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.dev_normal_bf16(d16, n, key, 12345, 90000 + 12345, 1e-3, hkey, 0.01, 1.0)
    synth.dev_normal_f32(d32, n, key, 12345, 90000 + 12345, 0.02)
    torch.cuda.synchronize()
    h16 = synth.host_normal_bf16(n, key, 12345, 90000 + 12345, 1e-3, hkey, 0.01, 1.0)
    h32 = synth.host_normal_f32(n, key, 12345, 90000 + 12345, 0.02)
    assert np.array_equal(d16.cpu().numpy().view(np.uint16), h16)
    assert np.array_equal(d32.cpu().numpy().view(np.uint32), h32.view(np.uint32))


# ------------------------------------------------------------ small parity

def test_tiny_config_full_shard(gpu):
    """Tiny config: n = 2^20, one decayed segment, k = 4, 10 steps with fresh
    seeded partials per step; full-shard comparison."""
    torch = gpu
    w = synth.workload("tiny")
    ds = H.DeviceShard(w)
    for t in w.step_ts():
        ds.fill_grads(t)
        ds.step(t)
    torch.cuda.synchronize()
    got = ds.window(0, w.n)
    ref = H.oracle_window(w, 0, w.n, w.step_ts())
    bitwise = H.assert_parity(got, ref, "tiny")
    print("tiny: bitwise equal to the oracle:", bitwise)
    ds.free()


@pytest.mark.parametrize("n", [1, 2, 7, 8, 9, 15, 16, 17, 511, 512, 513, 2047, 2048, 2049, 4095,
                               4097, 65539, 100_003])
@pytest.mark.parametrize("k", [1, 3, 8, 16])
def test_ragged_sizes_and_tiny_segments(gpu, n, k):
    rng = np.random.default_rng(n * 31 + k)
    segs = _random_segments(rng, n)
    got, ref = _run_both(gpu, n, k, segs, range(1, 4), seed=n + k)
    H.assert_parity(got, ref, "n=%d k=%d" % (n, k))


def test_segment_overflow_and_restaging(gpu):
    """Segments every 1-3 elements: each 256-element window holds more table
    entries than a wavefront's 64-entry slot, so the per-element table lookup
    runs; over several chunk lengths.  Also duplicate starts (empty segments)
    and entries past n."""
    rng = np.random.default_rng(5)
    n = 2048 * 12 + 5
    segs, a = [], 0
    while a < n:
        segs.append((a, bool(rng.random() < 0.5)))
        if rng.random() < 0.05:
            segs.append((a, bool(rng.random() < 0.5)))  # duplicate start
        a += int(rng.integers(1, 4))
    segs += [(n, True), (n + 10, False)]
    # the lookup does not depend on k; two partial counts for good measure
    for k in (2, 4):
        for chunk_tiles in (1, 4, 12):
            got, ref = _run_both(gpu, n, k, segs, range(1, 3), seed=9,
                                 cfg=dict(chunk_tiles=chunk_tiles))
            H.assert_parity(got, ref, "k=%d chunk_tiles=%d" % (k, chunk_tiles))


@pytest.mark.parametrize("n", [1, 1023, 1024 * 8 - 5, 1024 * 8 * 9 + 3 * 1024 + 17, 70_000 * 1024 + 333])
def test_xcd_chunk_order_covers_every_element(gpu, n):
    """XCD-contiguous order is a bijection of the chunks for any grid size
    (grids that are and are not multiples of the XCD count, and one above the
    default threshold): the default launch matches the oracle over the whole
    shard, and the linear and XCD orders match it bitwise."""
    torch = gpu
    rng = np.random.default_rng(n % 1000)
    segs = _random_segments(rng, n, short_frac=0.05)
    dflt, ref = _run_both(torch, n, 2, segs, range(1, 3), seed=19)
    assert H.assert_parity(dflt, ref, "n=%d default launch" % n)
    lin, _ = _run_both(torch, n, 2, segs, range(1, 3), seed=19, cfg=dict(block_order=1),
                       with_oracle=False)
    xcd, _ = _run_both(torch, n, 2, segs, range(1, 3), seed=19, cfg=dict(block_order=2),
                       with_oracle=False)
    for a, b, c in zip(lin, xcd, dflt):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
        assert np.array_equal(a.view(np.uint8), c.view(np.uint8))


def test_largest_segment_table(gpu):
    """ZS_MAX_SEGMENTS entries (three rounds of the 64-way search), most of
    them one or two elements long, the last ones past n."""
    rng = np.random.default_rng(17)
    n = 100_000
    count = zs.ZS_MAX_SEGMENTS
    starts = np.sort(rng.choice(np.arange(1, n + 5000), count - 1, replace=False))
    segs = [(0, True)] + [(int(a), bool(rng.random() < 0.5)) for a in starts]
    assert len(segs) == count
    got, ref = _run_both(gpu, n, 2, segs, range(1, 4), seed=17)
    H.assert_parity(got, ref, "%d segments" % count)


@pytest.mark.parametrize("nseg", [65, 127, 128, 129, 1970, 4095, 4096, 4097])
def test_segment_search_probe_edges(gpu, nseg):
    """Tables of more than 64 entries, just above one search round and around
    the point where further rounds start, whose entries at the search's probe
    positions (every ceil(nseg/64)-th) start exactly on a 256-element window
    start, one element past one, or on the same element as the entry before
    (a duplicate start, so the later entry wins).  Every flag must equal the
    oracle's, bit for bit."""
    rng = np.random.default_rng(nseg)
    step = -(-nseg // 64)
    starts = [0]
    for i in range(1, nseg):
        if i % step == 0:
            kind = int(rng.integers(3))
            nxt = (starts[-1] // 256 + 1) * 256
            starts.append((starts[-1], nxt, nxt + 1)[kind])
        else:
            starts.append(starts[-1] + int(rng.integers(1, 300)))
    n = starts[-1] + int(rng.integers(1, 2000))
    segs = [(st, bool(rng.random() < 0.5)) for st in starts]
    got, ref = _run_both(gpu, n, 2, segs, range(1, 3), seed=nseg)
    assert H.assert_parity(got, ref, "nseg=%d" % nseg), "nseg=%d: not bitwise equal" % nseg


def test_table_rewritten_in_place_between_steps(gpu):
    """The step reads the segment table through the scalar cache; a table
    the caller overwrites in place on the same stream between two steps
    (other starts and flags, more than 64 entries so that the scalar search
    runs) must be seen whole by the next step: GPU and oracle, table A for
    step 1 and table B for step 2, bit for bit."""
    torch = gpu
    rng = np.random.default_rng(77)
    n, k, nseg = 150_001, 3, 300
    def table(seed):
        r = np.random.default_rng(seed)
        starts = np.concatenate([[0], np.sort(r.choice(np.arange(1, n), nseg - 1, replace=False))])
        return [(int(st), bool(r.random() < 0.5)) for st in starts]
    ta, tb = table(1), table(2)
    w = synth.host_normal_f32(n, synth.stream_key(77, 1, 0, 0), 0, n, 0.02)
    ref = [w.copy(), np.zeros(n, F32), np.zeros(n, F32), np.zeros(n, np.uint16)]
    dw, dm, dv = _dev(torch, w), _dev(torch, ref[1]), _dev(torch, ref[2])
    dp = torch.zeros(n, dtype=torch.int16, device="cuda")
    dtab = H.segment_tensor(ta, "cuda")
    st = zs.seg_table(dtab)
    hpo, hpz = oracle.hparams(), zs.hparams()
    s = torch.cuda.current_stream()
    for t, segs in ((1, ta), (2, tb)):
        if t == 2:
            dtab.copy_(H.segment_tensor(tb, "cuda"))  # same buffer, same stream
        gs = [synth.host_normal_bf16(n, synth.stream_key(77, 2, j, t), 0, n, 0.01)
              for j in range(k)]
        zs.zs_shard_step(dw, dm, dv, dp, [_dev(torch, g) for g in gs], k, n, st, hpz, t, s)
        assert oracle.shard_step(*ref, gs, segs, hpo, t) == 0
    torch.cuda.synchronize()
    got = [dw.cpu().numpy(), dm.cpu().numpy(), dv.cpu().numpy(), dp.cpu().numpy().view(np.uint16)]
    assert H.assert_parity(got, ref, "table A then B"), "not bitwise equal"
    # a step 2 that still saw table A would differ: the test can tell them apart
    stale = [w.copy(), np.zeros(n, F32), np.zeros(n, F32), np.zeros(n, np.uint16)]
    for t in (1, 2):
        gs = [synth.host_normal_bf16(n, synth.stream_key(77, 2, j, t), 0, n, 0.01)
              for j in range(k)]
        assert oracle.shard_step(*stale, gs, ta, hpo, t) == 0
    assert not np.array_equal(stale[0].view(np.uint32), ref[0].view(np.uint32))


def test_unsorted_table_stays_in_bounds(gpu):
    """An unsorted device table (which the library cannot check) gives
    unspecified decay flags but reads nothing outside the table: the call
    completes, m and v (which do not depend on the flags) equal the oracle's
    bitwise, and every weight is the oracle's with decay on or with decay off."""
    torch = gpu
    rng = np.random.default_rng(18)
    n = 50_003
    segs = [(int(a), bool(rng.random() < 0.5))
            for a in rng.integers(-1000, n + 1000, 3000)]  # unsorted, duplicates, out of range
    segs[0] = (0, True)
    for name, table in (("random order", segs), ("reversed", sorted(segs)[::-1])):
        got, _ = _run_both(torch, n, 3, table, range(1, 4), seed=18,
                           ref_segs=[(0, True)])
        on = _run_both(torch, n, 3, [(0, True)], range(1, 4), seed=18)[1]
        off = _run_both(torch, n, 3, [(0, False)], range(1, 4), seed=18)[1]
        for i in (1, 2):  # m, v
            assert np.array_equal(got[i].view(np.uint32), on[i].view(np.uint32)), name
        w, p = got[0].view(np.uint32), got[3]
        either = (w == on[0].view(np.uint32)) | (w == off[0].view(np.uint32))
        assert either.all(), "%s: %d weights are neither" % (name, int((~either).sum()))
        pe = np.where(w == on[0].view(np.uint32), on[3], off[3])
        assert np.array_equal(p, pe), name


def test_launch_geometry_is_bitwise_invariant(gpu):
    torch = gpu
    rng = np.random.default_rng(6)
    n = 2048 * 40 + 1234
    segs = _random_segments(rng, n, short_frac=0.2)
    outs = []
    for cfg in (dict(), dict(chunk_tiles=1), dict(chunk_tiles=3), dict(chunk_tiles=7),
                dict(chunk_tiles=64), dict(chunk_tiles=2, nontemporal=1),
                dict(chunk_tiles=5, nontemporal=2), dict(block_order=1), dict(block_order=2),
                dict(block_order=2, chunk_tiles=3), dict(block_order=2, groups_per_cu=4)):
        got, ref = _run_both(torch, n, 5, segs, range(1, 4), seed=3, cfg=cfg or None)
        H.assert_parity(got, ref, str(cfg))
        outs.append(got)
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_occupancy_cap_is_bitwise_invariant(gpu):
    """groups_per_cu only reserves LDS: every cap gives the same bits as the
    default launch, with two and with eight partials."""
    torch = gpu
    rng = np.random.default_rng(16)
    n = 4096 * 30 + 777
    segs = _random_segments(rng, n, short_frac=0.2)
    for k in (2, 8):
        base, ref = _run_both(torch, n, k, segs, range(1, 3), seed=16)
        H.assert_parity(base, ref, "k=%d default" % k)
        for g in (2, 3, 6, 32):
            got, _ = _run_both(torch, n, k, segs, range(1, 3), seed=16,
                               cfg=dict(groups_per_cu=g))
            for a, b in zip(base, got):
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (k, g)


def test_launch_cfg_errors(gpu):
    torch = gpu
    n = 1024
    f = [torch.zeros(n, dtype=torch.float32, device="cuda") for _ in range(3)]
    p = torch.zeros(n, dtype=torch.int16, device="cuda")
    g = [torch.zeros(n, dtype=torch.int16, device="cuda") for _ in range(2)]
    table = H.segment_tensor([(0, True)], "cuda")

    def call(**cfg):
        return zs.zs_shard_step_cfg(f[0], f[1], f[2], p, g, 2, n, zs.seg_table(table),
                                    zs.hparams(), 1, None, check=False, **cfg)

    assert call() == zs.ZS_OK
    for bad in (dict(chunk_tiles=-1), dict(chunk_tiles=4097), dict(nontemporal=3),
                dict(groups_per_cu=-1), dict(groups_per_cu=zs.ZS_MAX_GROUPS_PER_CU + 1),
                dict(block_order=-1), dict(block_order=3)):
        assert call(**bad) == zs.ZS_ERR_INVALID_ARGUMENT, bad
    # a one-workgroup-per-unit cap fits only where one workgroup may take the
    # whole LDS of a unit; either way the call answers synchronously
    assert call(groups_per_cu=1) in (zs.ZS_OK, zs.ZS_ERR_INVALID_ARGUMENT)
    assert call(groups_per_cu=zs.ZS_MAX_GROUPS_PER_CU) == zs.ZS_OK
    torch.cuda.synchronize()


def test_hparam_variants(gpu):
    rng = np.random.default_rng(8)
    n = 30_001
    segs = _random_segments(rng, n, short_frac=0.1)
    for hp in (dict(lr=3e-4, beta1=0.0, beta2=0.999, eps=1e-3, weight_decay=0.0),
               dict(lr=1e-2, beta1=0.5, beta2=0.5, eps=0.0, weight_decay=1.0, grad_scale=0.125),
               dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1,
                    grad_scale=3.0)):
        got, ref = _run_both(gpu, n, 4, segs, range(1, 6), seed=4, hp_kw=hp)
        H.assert_parity(got, ref, str(hp))


@pytest.mark.parametrize("hp,ts", [
    (dict(lr=1.0, weight_decay=1.0), (1, 2, 3)),                 # df = 0: decayed weights -> 0
    (dict(beta1=0.999999, beta2=0.999999), (1, 2)),              # corrections near 1e-6
    (dict(eps=1e-45), (1, 2, 3)),                                # subnormal epsilon
    (dict(grad_scale=0.0), (1, 2)),                              # every gradient scaled to 0
    (dict(lr=3e-4, beta1=0.5, beta2=0.25), (10 ** 9, 10 ** 9 + 1)),  # huge t
])
def test_extreme_hyperparameters(gpu, hp, ts):
    rng = np.random.default_rng(20)
    n = 20_011
    segs = _random_segments(rng, n, short_frac=0.2)
    got, ref = _run_both(gpu, n, 3, segs, ts, seed=20, hp_kw=hp)
    H.assert_parity(got, ref, str(hp))


def test_zero_epsilon_with_zero_gradient_is_nan_on_both_sides(gpu):
    """The degenerate case of the update: eps = 0, m = v = 0 and a zero
    gradient give 0/0; both sides produce NaN weights and the canonical bf16
    NaN, and zero moments."""
    n = 3000
    zeros = lambda t: [np.zeros(n, np.uint16) for _ in range(2)]  # noqa: E731
    got, ref = _run_both(gpu, n, 2, [(0, True), (1000, False)], (1, 2), seed=21,
                         hp_kw=dict(eps=0.0), grads_fn=zeros)
    H.assert_parity(got, ref, "eps=0, g=0")
    assert np.isnan(got[0]).all() and (got[3] == 0x7FC0).all()
    assert not got[1].any() and not got[2].any()


def test_bias_correction_limit_steps(gpu):
    """t = 10000, 10001, 10002: bias corrections are exactly 1."""
    rng = np.random.default_rng(10)
    n = 50_000
    segs = _random_segments(rng, n, short_frac=0.1)
    got, ref = _run_both(gpu, n, 2, segs, [10000, 10001, 10002], seed=10,
                         hp_kw=dict(lr=3e-4))
    H.assert_parity(got, ref, "t=10000")


def test_nan_inf_and_denormals(gpu):
    """NaN and Inf in a partial poison only their own element; denormal
    weights, moments and gradients are kept (not flushed)."""
    torch = gpu
    n = 4099
    rng = np.random.default_rng(12)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    w0[100:200] = (rng.integers(1, 1 << 20, 100).astype(np.uint32)).view(F32)  # denormals

    def grads(t):
        g = rng.normal(0, 1e-3, (2, n)).astype(F32)
        g[0, 7] = np.nan
        g[1, 9] = np.inf
        g[0, 11] = -np.inf
        g[1, 300:350] = (rng.integers(1, 1 << 22, 50).astype(np.uint32) << 0).view(F32)
        return [(x.view(np.uint32) >> 16).astype(np.uint16) for x in g]

    segs = [(0, True), (150, False), (160, True)]
    got, ref = _run_both(torch, n, 2, segs, range(1, 4), seed=0, w0=w0, grads_fn=grads,
                         hp_kw=dict(eps=1e-30))
    H.assert_parity(got, ref, "nan/inf/denormal")
    assert np.isnan(got[0][7]) and np.isnan(got[0][9]) and got[3][7] == 0x7FC0


def test_resume_is_exact(gpu):
    """Steps 1..5, state round-tripped through the host, steps 6..10 equal
    steps 1..10 run straight through (the step is a pure function)."""
    torch = gpu
    w = synth.workload("tiny")
    a = H.DeviceShard(w)
    b = H.DeviceShard(w)
    for t in range(1, 11):
        a.fill_grads(t)
        a.step(t)
    for t in range(1, 6):
        b.fill_grads(t)
        b.step(t)
    torch.cuda.synchronize()
    saved = [x.cpu() for x in (b.master, b.m, b.v)]
    b.free()
    c = H.DeviceShard(w)
    c.master.copy_(saved[0])
    c.m.copy_(saved[1])
    c.v.copy_(saved[2])
    for t in range(6, 11):
        c.fill_grads(t)
        c.step(t)
    torch.cuda.synchronize()
    for x, y in zip(a.window(0, w.n), c.window(0, w.n)):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
    a.free()
    c.free()


def test_side_stream(gpu):
    torch = gpu
    n = 70_000
    s = torch.cuda.Stream()
    rng = np.random.default_rng(13)
    segs = _random_segments(rng, n, short_frac=0.1)
    with torch.cuda.stream(s):
        got, ref = _run_both(torch, n, 3, segs, range(1, 3), seed=13)
    H.assert_parity(got, ref, "side stream")


def test_concurrent_calls_from_threads_and_streams(gpu):
    """Four host threads, each with its own stream and buffers, call the step
    at the same time (the library keeps no mutable state after zs_init);
    every thread's result equals the oracle's."""
    import threading
    torch = gpu
    jobs = []
    for j in range(4):
        n = 40_000 + 777 * j
        rng = np.random.default_rng(100 + j)
        segs = _random_segments(rng, n, short_frac=0.2)
        w0 = rng.normal(0, 0.02, n).astype(F32)
        gs = [[(rng.normal(0, 1e-2, n).astype(F32).view(np.uint32) >> 16).astype(np.uint16)
               for _ in range(j + 1)] for _ in range(3)]
        jobs.append(dict(n=n, k=j + 1, segs=segs, w0=w0, gs=gs))
    dev = []
    for jb in jobs:
        n = jb["n"]
        dev.append(dict(w=_dev(torch, jb["w0"]), m=torch.zeros(n, device="cuda"),
                        v=torch.zeros(n, device="cuda"),
                        p=torch.zeros(n, dtype=torch.int16, device="cuda"),
                        g=[[_dev(torch, g) for g in step] for step in jb["gs"]],
                        table=H.segment_tensor(jb["segs"], "cuda"), stream=torch.cuda.Stream()))
    torch.cuda.synchronize()
    errors = []
    start = threading.Barrier(len(jobs))

    def run(jb, d):
        try:
            start.wait()
            for t in range(1, 4):
                zs.zs_shard_step(d["w"], d["m"], d["v"], d["p"], d["g"][t - 1], jb["k"], jb["n"],
                                 zs.seg_table(d["table"]), zs.hparams(), t, d["stream"])
            d["stream"].synchronize()
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(e)

    threads = [threading.Thread(target=run, args=(jb, d)) for jb, d in zip(jobs, dev)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    assert not errors, errors
    torch.cuda.synchronize()
    for jb, d in zip(jobs, dev):
        n = jb["n"]
        ref = [jb["w0"].copy(), np.zeros(n, F32), np.zeros(n, F32), np.zeros(n, np.uint16)]
        for t in range(1, 4):
            assert oracle.shard_step(*ref, jb["gs"][t - 1], jb["segs"], oracle.hparams(), t) == 0
        got = (d["w"].cpu().numpy(), d["m"].cpu().numpy(), d["v"].cpu().numpy(),
               d["p"].cpu().numpy().view(np.uint16))
        H.assert_parity(got, ref, "thread k=%d" % jb["k"])


# ------------------------------------------------------- model-shaped shards

def test_gpt2_small_rank0_full_shard(gpu):
    """GPT-2-small rank 0 of 8 (15,554,976 elements, 27 segments, k = 8),
    10 steps; full-shard comparison."""
    torch = gpu
    w = synth.workload("gpt2-small")
    ds = H.DeviceShard(w)
    for t in w.step_ts():
        ds.fill_grads(t)
        ds.step(t)
    torch.cuda.synchronize()
    got = ds.window(0, w.n)
    ds.free()
    ref = H.oracle_window(w, 0, w.n, w.step_ts())
    print("gpt2 rank0: bitwise equal:", H.assert_parity(got, ref, "gpt2 r0"))


def test_gpt2_small_all_ranks_windows(gpu):
    """All 8 ranks of the GPT-2-small flat buffer, run one after another on
    the one GPU (2 steps each), compared on windows around every segment
    boundary of each shard."""
    torch = gpu
    base = synth.workload("gpt2-small")
    for r in range(base.p):
        w = base.with_rank(r)
        ds = H.DeviceShard(w)
        for t in (1, 2):
            ds.fill_grads(t)
            ds.step(t)
        torch.cuda.synchronize()
        for lo, hi in H.boundary_windows(w, 4096, max_boundaries=64, n_random=2, seed=r):
            H.assert_parity(ds.window(lo, hi), H.oracle_window(w, lo, hi, (1, 2)),
                            "rank %d [%d,%d)" % (r, lo, hi))
        ds.free()


def _large_config(torch, name, window, max_boundaries):
    w = synth.workload(name)
    free, _ = torch.cuda.mem_get_info()
    need = w.n * (14 + 2 * w.k) + (1 << 30)
    if free < need:
        pytest.skip("needs %.1f GB of free device memory" % (need / 1e9))
    print("%s: n=%d k=%d segments=%d" % (name, w.n, w.k, len(w.shard.segments)), flush=True)
    ds = H.DeviceShard(w)
    ts = list(range(1, w.prewarm_steps + 1)) + w.step_ts()
    for t in ts:
        ds.fill_grads(t)
        ds.step(t)
    torch.cuda.synchronize()
    wins = H.boundary_windows(w, window, max_boundaries=max_boundaries, n_random=4, seed=1)
    got = [ds.window(lo, hi) for lo, hi in wins]
    ds.free()
    allbit = True
    for (lo, hi), g in zip(wins, got):
        allbit &= H.assert_parity(g, H.oracle_window(w, lo, hi, ts), "%s [%d,%d)" % (name, lo, hi))
    print("%s: %d windows, bitwise equal: %s" % (name, len(wins), allbit), flush=True)


def test_7b_rank0_windows(gpu):
    """7B-shaped rank 0 of 8 (805M elements, k = 8, 1% heavy-tailed partials):
    100 pre-warm steps then 10 measured steps, windowed comparison (windows of
    2^13 elements: the oracle regenerates and replays all 110 steps of eight
    partials for each)."""
    _large_config(gpu, "7b", 1 << 13, 40)


def test_175b_rank0_windows(gpu):
    """GPT-3-175B-shaped rank 0 of 64 (2.72e9 elements, k = 2), 5 steps:
    windows of 2^20 elements at every segment boundary, both ends and random."""
    _large_config(gpu, "175b", 1 << 20, 32)


def test_70b_rank0_windows(gpu):
    """70B-shaped rank 0 of 8 (8.05e9 elements, 1970 segments, k = 2) at
    t = 10000..10002: windows of 2^20 elements at 64 of the segment
    boundaries, both ends and random."""
    _large_config(gpu, "70b", 1 << 20, 64)
