"""The packed-state steps (zs_shard_step_packed and its int8 and bf16-moment
forms) and the layout conversions (zs_pack_state, zs_unpack_state and their
bf16-moment forms) through the C ABI.  The packed layouts are built and read
back here with numpy reshapes of (blocks, 3, 256) and byte slices of 2 KB
blocks, written independently of the library's conversion kernels; each step
must equal the oracle, and its separate-array entry point on the same inputs,
bit for bit."""
import numpy as np
import pytest

import oracle
import sharded_mixed_precision_shard_amd as zs
import synth
from tests import _gpu_harness as H

pytestmark = pytest.mark.gpu

F32 = np.float32
SIZES = [1, 7, 255, 256, 257, 1023, 1024, 1025, 4097, 10007, 65539]


@pytest.fixture(scope="module")
def gpu():
    import torch
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    assert zs.zs_init(0) == zs.ZS_OK
    yield torch
    torch.cuda.synchronize()


pack = H.pack_host
unpack = H.unpack_host


def _dev(torch, a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).cuda()
    return torch.from_numpy(a.copy()).cuda()


def _segments(rng, n):
    segs, a = [], 0
    while a < n:
        segs.append((a, bool(rng.random() < 0.5)))
        a += int(rng.integers(1, 8)) if rng.random() < 0.4 else int(rng.integers(8, 3000))
    return segs


def _partials(rng, k, n, sigma=1e-2):
    return [(rng.normal(0, sigma, n).astype(F32).view(np.uint32) >> 16).astype(np.uint16)
            for _ in range(k)]


def test_packed_floats_matches_the_header():
    for n in (0, 1, 255, 256, 257, 10 ** 9 + 1):
        assert zs.packed_floats(n) == 768 * (-(-n // 256))


@pytest.mark.parametrize("n", SIZES)
def test_pack_and_unpack(gpu, n):
    """zs_pack_state writes the host packing (padding +0); zs_unpack_state
    restores the arrays bit for bit and writes nothing past n."""
    torch = gpu
    rng = np.random.default_rng(n)
    w, m, v = (rng.normal(0, 1, n).astype(F32) for _ in range(3))
    w[::7] = -0.0
    dstate = torch.full((zs.packed_floats(n),), 7.0, dtype=torch.float32, device="cuda")
    zs.zs_pack_state(_dev(torch, w), _dev(torch, m), _dev(torch, v), dstate, n)
    torch.cuda.synchronize()
    got = dstate.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), pack(w, m, v).view(np.uint32))
    guard = 5
    outs = [torch.full((n + guard,), 3.0, dtype=torch.float32, device="cuda") for _ in range(3)]
    zs.zs_unpack_state(dstate, *outs, n)
    torch.cuda.synchronize()
    for o, x in zip(outs, (w, m, v)):
        h = o.cpu().numpy()
        assert np.array_equal(h[:n].view(np.uint32), x.view(np.uint32))
        assert np.all(h[n:] == 3.0)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("k", [1, 2, 5, 16])
def test_packed_step_matches_oracle_and_base(gpu, n, k):
    torch = gpu
    rng = np.random.default_rng(300 + n * 3 + k)
    segs = _segments(rng, n)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    ref = [w0.copy(), np.zeros(n, F32), np.zeros(n, F32), np.zeros(n, np.uint16)]
    dstate = _dev(torch, pack(w0, ref[1], ref[2]))
    dp = torch.zeros(n, dtype=torch.int16, device="cuda")
    bw, bm, bv = _dev(torch, w0), _dev(torch, ref[1]), _dev(torch, ref[2])
    bp = torch.zeros(n, dtype=torch.int16, device="cuda")
    table = H.segment_tensor(segs, "cuda")
    hpo, hpz = oracle.hparams(), zs.hparams()
    s = torch.cuda.current_stream()
    for t in range(1, 4):
        gs = _partials(rng, k, n)
        dgs = [_dev(torch, g) for g in gs]
        zs.zs_shard_step_packed(dstate, dp, dgs, k, n, zs.seg_table(table), hpz, t, s)
        zs.zs_shard_step(bw, bm, bv, bp, dgs, k, n, zs.seg_table(table), hpz, t, s)
        assert oracle.shard_step(*ref, gs, segs, hpo, t) == 0
    torch.cuda.synchronize()
    state = dstate.cpu().numpy()
    got = list(unpack(state, n)) + [dp.cpu().numpy().view(np.uint16)]
    assert H.assert_parity(got, ref, "packed n=%d k=%d" % (n, k)), "not bitwise"
    base = [bw.cpu().numpy(), bm.cpu().numpy(), bv.cpu().numpy(),
            bp.cpu().numpy().view(np.uint16)]
    for a, b in zip(got, base):
        assert np.array_equal(np.ascontiguousarray(a).view(np.uint8), b.view(np.uint8))
    # the step leaves the padding of the last block as it found it
    pad = state.reshape(-1, 3, 256)[-1, :, n % 256:] if n % 256 else np.zeros(0, F32)
    assert np.all(pad == 0.0)


def test_packed_step_on_a_large_grid_equals_the_base_step(gpu):
    """A shard above 2^26 elements (XCD chunk order, occupancy cap), many
    segments and a ragged tail: packed and base steps agree bit for bit, and
    a few windows agree with the oracle."""
    torch = gpu
    n, k = (1 << 26) + 12345, 2
    rng = np.random.default_rng(26)
    starts = np.concatenate([[0], np.sort(rng.choice(np.arange(1, n), 1969, replace=False))])
    segs = [(int(a), bool(rng.random() < 0.5)) for a in starts]
    assert zs.zs_launch_plan(k, n, "packed")["groups_per_cu"] == 5
    w0 = synth.host_normal_f32(n, synth.stream_key(26, 1, 0, 0), 0, n, 0.02)
    zeros = np.zeros(n, F32)
    dstate = torch.zeros(zs.packed_floats(n), dtype=torch.float32, device="cuda")
    zs.zs_pack_state(_dev(torch, w0), _dev(torch, zeros), _dev(torch, zeros), dstate, n)
    bw, bm, bv = _dev(torch, w0), _dev(torch, zeros), _dev(torch, zeros)
    dp = torch.zeros(n, dtype=torch.int16, device="cuda")
    bp = torch.zeros(n, dtype=torch.int16, device="cuda")
    table = H.segment_tensor(segs, "cuda")
    hpz = zs.hparams()
    s = torch.cuda.current_stream()
    gs_all = []
    for t in (1, 2):
        gs = [synth.host_normal_bf16(n, synth.stream_key(26, 2, j, t), 0, n, 0.01)
              for j in range(k)]
        gs_all.append(gs)
        dgs = [_dev(torch, g) for g in gs]
        zs.zs_shard_step_packed(dstate, dp, dgs, k, n, zs.seg_table(table), hpz, t, s)
        zs.zs_shard_step(bw, bm, bv, bp, dgs, k, n, zs.seg_table(table), hpz, t, s)
    outs = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3)]
    zs.zs_unpack_state(dstate, *outs, n)
    torch.cuda.synchronize()
    for o, b in zip(outs + [dp], (bw, bm, bv, bp)):
        assert torch.equal(o.view(torch.int32) if o.dtype == torch.float32 else o,
                           b.view(torch.int32) if b.dtype == torch.float32 else b)
    hpo = oracle.hparams()
    for lo, hi in ((0, 4096), (n // 2 - 777, n // 2 + 1500), (n - 3000, n)):
        ref = [w0[lo:hi].copy(), np.zeros(hi - lo, F32), np.zeros(hi - lo, F32),
               np.zeros(hi - lo, np.uint16)]
        wsegs = synth.clip_segments(segs, lo, hi)
        for t, gs in zip((1, 2), gs_all):
            assert oracle.shard_step(*ref, [g[lo:hi] for g in gs], wsegs, hpo, t) == 0
        got = [outs[0][lo:hi].cpu().numpy(), outs[1][lo:hi].cpu().numpy(),
               outs[2][lo:hi].cpu().numpy(), dp[lo:hi].cpu().numpy().view(np.uint16)]
        assert H.assert_parity(got, ref, "window [%d,%d)" % (lo, hi)), "not bitwise"


def test_prepared_packed_call_matches_the_plain_call(gpu):
    torch = gpu
    n, k = 70_001, 3
    rng = np.random.default_rng(7)
    segs = _segments(rng, n)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    z = np.zeros(n, F32)
    a = _dev(torch, pack(w0, z, z))
    b = _dev(torch, pack(w0, z, z))
    pa = torch.zeros(n, dtype=torch.int16, device="cuda")
    pb = torch.zeros(n, dtype=torch.int16, device="cuda")
    table = H.segment_tensor(segs, "cuda")
    st, hp = zs.seg_table(table), zs.hparams()
    gs = [_dev(torch, g) for g in _partials(rng, k, n)]
    call = zs.ShardStep(a, None, None, pa, gs, n, st, hp, variant="packed")
    for t in (1, 2, 3):
        call(t)
        zs.zs_shard_step_packed(b, pb, gs, k, n, st, hp, t)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32)) and torch.equal(pa, pb)


def test_packed_argument_errors(gpu):
    torch = gpu
    n, k = 1000, 2
    state = torch.zeros(zs.packed_floats(n) + 64, dtype=torch.float32, device="cuda")
    p = torch.zeros(n, dtype=torch.int16, device="cuda")
    g = [torch.zeros(n, dtype=torch.int16, device="cuda") for _ in range(k)]
    table = H.segment_tensor([(0, True)], "cuda")
    st, hp = zs.seg_table(table), zs.hparams()
    sp, pp = state.data_ptr(), p.data_ptr()
    gp = [x.data_ptr() for x in g]
    call = lambda *a: zs.zs_shard_step_packed(*a, check=False)
    assert call(sp, pp, gp, k, n, st, hp, 1) == zs.ZS_OK
    assert call(0, pp, gp, k, n, st, hp, 1) == zs.ZS_ERR_INVALID_ARGUMENT
    assert call(sp + 4, pp, gp, k, n, st, hp, 1) == zs.ZS_ERR_MISALIGNED
    # the param copy, or a partial, inside the state
    assert call(sp, sp + 4 * 1024, gp, k, n, st, hp, 1) == zs.ZS_ERR_ALIASING
    assert call(sp, pp, [gp[0], sp + 4 * 2048], k, n, st, hp, 1) == zs.ZS_ERR_ALIASING
    assert call(sp, pp, gp, k, 0, st, hp, 1) == zs.ZS_OK
    assert call(sp, pp, gp, k, n, st, hp, 0) == zs.ZS_ERR_INVALID_ARGUMENT
    arrs = [torch.zeros(n, dtype=torch.float32, device="cuda") for _ in range(3)]
    ap = [x.data_ptr() for x in arrs]
    pk = lambda *a: zs.zs_pack_state(*a, check=False)
    up = lambda *a: zs.zs_unpack_state(*a, check=False)
    assert pk(*ap, sp, n) == zs.ZS_OK and up(sp, *ap, n) == zs.ZS_OK
    assert pk(ap[0], ap[1], ap[2], sp, 0) == zs.ZS_OK
    assert pk(ap[0], ap[1], 0, sp, n) == zs.ZS_ERR_INVALID_ARGUMENT
    assert pk(ap[0] + 4, ap[1], ap[2], sp, n) == zs.ZS_ERR_MISALIGNED
    assert pk(ap[0], ap[0], ap[2], sp, n) == zs.ZS_ERR_ALIASING
    assert up(sp, ap[0], ap[1], sp + 16, n) == zs.ZS_ERR_ALIASING
    assert pk(*ap, sp, -1) == zs.ZS_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()


def _packed_shard_windows(torch, name, variant, window, max_boundaries):
    """A model-shaped shard with packed state over its workload's steps (the
    pre-warm steps included): windows at segment boundaries, both ends and at
    random equal the oracle bit for bit."""
    w = synth.workload(name)
    free, _ = torch.cuda.mem_get_info()
    state = 8 if variant == "packed_bf16mv" else 12
    need = w.n * (state + 4 + 2 + 2 * w.k) + (1 << 30)
    if free < need:
        pytest.skip("needs %.1f GB of free device memory" % (need / 1e9))
    ts = list(range(1, w.prewarm_steps + 1)) + w.step_ts()
    ds = H.DeviceShard(w, variant)
    for t in ts:
        ds.fill_grads(t)
        ds.step(t)
    torch.cuda.synchronize()
    wins = H.boundary_windows(w, window, max_boundaries=max_boundaries, n_random=4, seed=5)
    got = [ds.window(lo, hi) for lo, hi in wins]
    ds.free()
    arith = "bf16mv" if variant == "packed_bf16mv" else "base"
    for (lo, hi), g in zip(wins, got):
        ref = H.oracle_window(w, lo, hi, ts, variant=arith)
        assert H.assert_parity(g, ref, "%s %s [%d,%d)" % (name, variant, lo, hi)), "not bitwise"
    print("%s %s: %d windows bitwise equal" % (name, variant, len(wins)), flush=True)


def test_70b_packed_windows(gpu):
    """The 70B-shaped shard with packed state, t = 10000..10002."""
    _packed_shard_windows(gpu, "70b", "packed", 1 << 14, 16)


@pytest.mark.parametrize("variant", ["packed", "packed_bf16mv"])
def test_175b_packed_windows(gpu, variant):
    """The 175B-shaped shard (13 segments, k = 2, five steps) with packed state:
    windows of 2^20 elements."""
    _packed_shard_windows(gpu, "175b", variant, 1 << 20, 16)


@pytest.mark.parametrize("variant", ["packed", "packed_bf16mv"])
def test_7b_packed_windows(gpu, variant):
    """The 7B-shaped shard (k = 8, heavy-tailed partials, 100 pre-warm steps
    then 10) with packed state."""
    _packed_shard_windows(gpu, "7b", variant, 1 << 12, 12)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("k", [1, 3, 16])
def test_packed_q8ag_matches_oracle_and_q8ag(gpu, n, k):
    """The int8 all-gather payload from the packed state: the oracle's state,
    parameters, codes and scales, and zs_shard_step_q8ag's bits."""
    torch = gpu
    rng = np.random.default_rng(500 + n * 3 + k)
    segs = _segments(rng, n)
    nb = -(-n // 256)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    z = np.zeros(n, F32)
    ref = [w0.copy(), z.copy(), z.copy(), np.zeros(n, np.uint16)]
    dstate = _dev(torch, pack(w0, z, z))
    dp = torch.zeros(n, dtype=torch.int16, device="cuda")
    dq = torch.full((n,), 99, dtype=torch.int8, device="cuda")
    ds = torch.zeros(nb, dtype=torch.float32, device="cuda")
    bw, bm, bv = _dev(torch, w0), _dev(torch, z), _dev(torch, z)
    bp = torch.zeros(n, dtype=torch.int16, device="cuda")
    bq = torch.full((n,), 99, dtype=torch.int8, device="cuda")
    bs = torch.zeros(nb, dtype=torch.float32, device="cuda")
    table = H.segment_tensor(segs, "cuda")
    hpo, hpz = oracle.hparams(), zs.hparams()
    s = torch.cuda.current_stream()
    for t in (1, 2, 3):
        gs = _partials(rng, k, n)
        if t == 2 and n > 300:
            gs[0][n // 2] = 0x7FC0  # a NaN partial poisons one element and its block
        dgs = [_dev(torch, g) for g in gs]
        zs.zs_shard_step_packed_q8ag(dstate, dp, dq, ds, dgs, k, n, zs.seg_table(table), hpz, t, s)
        zs.zs_shard_step_q8ag(bw, bm, bv, bp, bq, bs, dgs, k, n, zs.seg_table(table), hpz, t, s)
        assert oracle.shard_step(*ref, gs, segs, hpo, t) == 0
    torch.cuda.synchronize()
    q, sc = oracle.q8_blocks(ref[3], 256)
    got = list(unpack(dstate.cpu().numpy(), n)) + [dp.cpu().numpy().view(np.uint16),
                                                   dq.cpu().numpy(), ds.cpu().numpy()]
    # the planted NaN's sign and payload are not fixed by the method, so only
    # the tolerances hold against the oracle; the base kernel's bits must match
    H.assert_parity(got, tuple(ref) + (q, sc), "packed q8ag n=%d k=%d" % (n, k))
    if n > 300:
        assert np.isnan(got[5][(n // 2) // 256])
    base = [bw.cpu().numpy(), bm.cpu().numpy(), bv.cpu().numpy(),
            bp.cpu().numpy().view(np.uint16), bq.cpu().numpy(), bs.cpu().numpy()]
    for a, b in zip(got, base):
        assert np.array_equal(np.ascontiguousarray(a).view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("k", [1, 3, 16])
def test_packed_q8grad_matches_oracle_and_q8grad(gpu, n, k):
    """int8 partials dequantized in the reduce, on the packed state: the
    oracle's state and parameters, and zs_shard_step_q8grad's bits."""
    torch = gpu
    rng = np.random.default_rng(700 + n * 3 + k)
    segs = _segments(rng, n)
    nb = -(-n // 256)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    z = np.zeros(n, F32)
    ref = [w0.copy(), z.copy(), z.copy(), np.zeros(n, np.uint16)]
    dstate = _dev(torch, pack(w0, z, z))
    dp = torch.zeros(n, dtype=torch.int16, device="cuda")
    bw, bm, bv = _dev(torch, w0), _dev(torch, z), _dev(torch, z)
    bp = torch.zeros(n, dtype=torch.int16, device="cuda")
    table = H.segment_tensor(segs, "cuda")
    hpo, hpz = oracle.hparams(), zs.hparams()
    s = torch.cuda.current_stream()
    for t in (1, 2, 3):
        qs = [rng.integers(-127, 128, n).astype(np.int8) for _ in range(k)]
        ss = [(rng.random(nb) * 1e-4).astype(F32) for _ in range(k)]
        dq = [_dev(torch, q) for q in qs]
        dss = [_dev(torch, x) for x in ss]
        zs.zs_shard_step_packed_q8grad(dstate, dp, dq, dss, k, n, zs.seg_table(table), hpz, t, s)
        zs.zs_shard_step_q8grad(bw, bm, bv, bp, dq, dss, k, n, zs.seg_table(table), hpz, t, s)
        assert oracle.shard_step_q8grad(*ref, qs, ss, segs, hpo, t) == 0
    torch.cuda.synchronize()
    got = list(unpack(dstate.cpu().numpy(), n)) + [dp.cpu().numpy().view(np.uint16)]
    assert H.assert_parity(got, ref, "packed q8grad n=%d k=%d" % (n, k))
    base = [bw.cpu().numpy(), bm.cpu().numpy(), bv.cpu().numpy(),
            bp.cpu().numpy().view(np.uint16)]
    for a, b in zip(got, base):
        assert np.array_equal(np.ascontiguousarray(a).view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("variant", ["packed_q8ag", "packed_q8grad"])
def test_prepared_packed_q8_calls_match_the_plain_calls(gpu, variant):
    torch = gpu
    n, k = 70_001, 2
    rng = np.random.default_rng(9)
    segs = _segments(rng, n)
    nb = -(-n // 256)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    z = np.zeros(n, F32)
    a, b = _dev(torch, pack(w0, z, z)), _dev(torch, pack(w0, z, z))
    pa = torch.zeros(n, dtype=torch.int16, device="cuda")
    pb = torch.zeros(n, dtype=torch.int16, device="cuda")
    table = H.segment_tensor(segs, "cuda")
    st, hp = zs.seg_table(table), zs.hparams()
    if variant == "packed_q8ag":
        gs = [_dev(torch, g) for g in _partials(rng, k, n)]
        qa = torch.zeros(n, dtype=torch.int8, device="cuda")
        qb = torch.zeros(n, dtype=torch.int8, device="cuda")
        sa = torch.zeros(nb, dtype=torch.float32, device="cuda")
        sb = torch.zeros(nb, dtype=torch.float32, device="cuda")
        call = zs.ShardStep(a, None, None, pa, gs, n, st, hp, variant=variant, param_q8=qa,
                            param_q8_scale=sa)
        plain = lambda t: zs.zs_shard_step_packed_q8ag(b, pb, qb, sb, gs, k, n, st, hp, t)  # noqa
        extra = [(qa, qb), (sa, sb)]
    else:
        qs = [_dev(torch, rng.integers(-127, 128, n).astype(np.int8)) for _ in range(k)]
        ss = [_dev(torch, (rng.random(nb) * 1e-4).astype(F32)) for _ in range(k)]
        call = zs.ShardStep(a, None, None, pa, qs, n, st, hp, variant=variant, qscales=ss)
        plain = lambda t: zs.zs_shard_step_packed_q8grad(b, pb, qs, ss, k, n, st, hp, t)  # noqa
        extra = []
    for t in (1, 2, 3):
        call(t)
        plain(t)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32)) and torch.equal(pa, pb)
    for x, y in extra:
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


# ---- the bf16-moment state packed per block (zs_shard_step_packed_bf16mv)

pack16 = H.pack16_host
unpack16 = H.unpack16_host


def _bf16_bits(x):
    return (x.astype(F32).view(np.uint32) >> 16).astype(np.uint16)


def test_packed_bf16mv_floats_matches_the_header():
    for n in (0, 1, 255, 256, 257, 10 ** 9 + 1):
        assert zs.packed_bf16mv_floats(n) == 512 * (-(-n // 256))


@pytest.mark.parametrize("n", SIZES)
def test_pack_and_unpack_bf16mv(gpu, n):
    """zs_pack_state_bf16mv writes the host packing (zero padding);
    zs_unpack_state_bf16mv restores the arrays bit for bit and writes nothing
    past n."""
    torch = gpu
    rng = np.random.default_rng(1000 + n)
    w = rng.normal(0, 1, n).astype(F32)
    m = rng.integers(0, 1 << 16, n).astype(np.uint16)
    v = rng.integers(0, 1 << 16, n).astype(np.uint16)
    dstate = torch.full((zs.packed_bf16mv_floats(n),), 7.0, dtype=torch.float32, device="cuda")
    zs.zs_pack_state_bf16mv(_dev(torch, w), _dev(torch, m), _dev(torch, v), dstate, n)
    torch.cuda.synchronize()
    got = dstate.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), pack16(w, m, v).view(np.uint32))
    guard = 5
    ow = torch.full((n + guard,), 3.0, dtype=torch.float32, device="cuda")
    om = torch.full((n + guard,), 77, dtype=torch.int16, device="cuda")
    ov = torch.full((n + guard,), 77, dtype=torch.int16, device="cuda")
    zs.zs_unpack_state_bf16mv(dstate, ow, om, ov, n)
    torch.cuda.synchronize()
    hw = ow.cpu().numpy()
    hm, hv = om.cpu().numpy().view(np.uint16), ov.cpu().numpy().view(np.uint16)
    assert np.array_equal(hw[:n].view(np.uint32), w.view(np.uint32)) and np.all(hw[n:] == 3.0)
    assert np.array_equal(hm[:n], m) and np.all(hm[n:] == 77)
    assert np.array_equal(hv[:n], v) and np.all(hv[n:] == 77)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("k", [1, 3, 16])
def test_packed_bf16mv_matches_oracle_and_bf16mv(gpu, n, k):
    """Ten steps from non-zero bf16 moments: the oracle's bits, and
    zs_shard_step_bf16mv's on the same inputs; the padding stays zero."""
    torch = gpu
    rng = np.random.default_rng(900 + n * 3 + k)
    segs = _segments(rng, n)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    m0 = _bf16_bits(rng.normal(0, 1e-3, n))
    v0 = _bf16_bits(rng.normal(0, 1e-3, n) ** 2)
    ref = [w0.copy(), m0.copy(), v0.copy(), np.zeros(n, np.uint16)]
    dstate = _dev(torch, pack16(w0, m0, v0))
    dp = torch.zeros(n, dtype=torch.int16, device="cuda")
    bw, bm, bv = _dev(torch, w0), _dev(torch, m0), _dev(torch, v0)
    bp = torch.zeros(n, dtype=torch.int16, device="cuda")
    table = H.segment_tensor(segs, "cuda")
    hpo, hpz = oracle.hparams(), zs.hparams()
    s = torch.cuda.current_stream()
    for t in range(1, 11):
        gs = _partials(rng, k, n, 1e-3)
        dgs = [_dev(torch, g) for g in gs]
        zs.zs_shard_step_packed_bf16mv(dstate, dp, dgs, k, n, zs.seg_table(table), hpz, t, s)
        zs.zs_shard_step_bf16mv(bw, bm, bv, bp, dgs, k, n, zs.seg_table(table), hpz, t, s)
        assert oracle.shard_step_bf16mv(*ref, gs, segs, hpo, t) == 0
    torch.cuda.synchronize()
    state = dstate.cpu().numpy()
    got = list(unpack16(state, n)) + [dp.cpu().numpy().view(np.uint16)]
    assert H.assert_parity(got, ref, "packed bf16mv n=%d k=%d" % (n, k)), "not bitwise"
    base = [bw.cpu().numpy(), bm.cpu().numpy().view(np.uint16), bv.cpu().numpy().view(np.uint16),
            bp.cpu().numpy().view(np.uint16)]
    for a, b in zip(got, base):
        assert np.array_equal(np.ascontiguousarray(a).view(np.uint8), b.view(np.uint8))
    if n % 256:
        blk = state.view(np.uint8).reshape(-1, 2048)[-1]
        r = n % 256
        for a, z, size in ((0, 1024, 4), (1024, 1536, 2), (1536, 2048, 2)):
            assert not blk[a + r * size:z].any()


def test_prepared_packed_bf16mv_call_matches_the_plain_call(gpu):
    torch = gpu
    n, k = 70_001, 3
    rng = np.random.default_rng(17)
    segs = _segments(rng, n)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    z = np.zeros(n, np.uint16)
    a, b = _dev(torch, pack16(w0, z, z)), _dev(torch, pack16(w0, z, z))
    pa = torch.zeros(n, dtype=torch.int16, device="cuda")
    pb = torch.zeros(n, dtype=torch.int16, device="cuda")
    table = H.segment_tensor(segs, "cuda")
    st, hp = zs.seg_table(table), zs.hparams()
    gs = [_dev(torch, g) for g in _partials(rng, k, n)]
    call = zs.ShardStep(a, None, None, pa, gs, n, st, hp, variant="packed_bf16mv")
    for t in (1, 2, 3):
        call(t)
        zs.zs_shard_step_packed_bf16mv(b, pb, gs, k, n, st, hp, t)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32)) and torch.equal(pa, pb)


def test_packed_bf16mv_argument_errors(gpu):
    torch = gpu
    n, k = 1000, 2
    state = torch.zeros(zs.packed_bf16mv_floats(n) + 64, dtype=torch.float32, device="cuda")
    p = torch.zeros(n, dtype=torch.int16, device="cuda")
    g = [torch.zeros(n, dtype=torch.int16, device="cuda") for _ in range(k)]
    table = H.segment_tensor([(0, True)], "cuda")
    st, hp = zs.seg_table(table), zs.hparams()
    sp, pp = state.data_ptr(), p.data_ptr()
    gp = [x.data_ptr() for x in g]
    call = lambda *a: zs.zs_shard_step_packed_bf16mv(*a, check=False)  # noqa: E731
    assert call(sp, pp, gp, k, n, st, hp, 1) == zs.ZS_OK
    assert call(0, pp, gp, k, n, st, hp, 1) == zs.ZS_ERR_INVALID_ARGUMENT
    assert call(sp + 8, pp, gp, k, n, st, hp, 1) == zs.ZS_ERR_MISALIGNED
    # the state spans 2 KB per 256 elements: a param copy 3 KB in overlaps it
    assert call(sp, sp + 3 * 1024, gp, k, n, st, hp, 1) == zs.ZS_ERR_ALIASING
    assert call(sp, pp, [gp[0], sp + 4 * 1024], k, n, st, hp, 1) == zs.ZS_ERR_ALIASING
    assert call(sp, pp, gp, k, 0, st, hp, 1) == zs.ZS_OK
    w = torch.zeros(n, dtype=torch.float32, device="cuda")
    m = torch.zeros(n, dtype=torch.int16, device="cuda")
    v = torch.zeros(n, dtype=torch.int16, device="cuda")
    wp, mp, vp = w.data_ptr(), m.data_ptr(), v.data_ptr()
    pk = lambda *a: zs.zs_pack_state_bf16mv(*a, check=False)  # noqa: E731
    up = lambda *a: zs.zs_unpack_state_bf16mv(*a, check=False)  # noqa: E731
    assert pk(wp, mp, vp, sp, n) == zs.ZS_OK and up(sp, wp, mp, vp, n) == zs.ZS_OK
    assert pk(wp, mp, vp, sp, 0) == zs.ZS_OK
    assert pk(wp, mp, 0, sp, n) == zs.ZS_ERR_INVALID_ARGUMENT
    assert pk(wp, mp + 2, vp, sp, n) == zs.ZS_ERR_MISALIGNED
    assert pk(wp, mp, mp, sp, n) == zs.ZS_ERR_ALIASING
    assert up(sp, wp, mp, sp + 16, n) == zs.ZS_ERR_ALIASING
    assert pk(wp, mp, vp, sp, -1) == zs.ZS_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()


def test_70b_packed_bf16mv_windows(gpu):
    """The 70B-shaped shard with the packed bf16-moment state, which takes the
    wide launch (two sub-windows per wave), t = 10000..10002."""
    w = synth.workload("70b")
    assert zs.zs_launch_plan(w.k, w.n, "packed_bf16mv")["window_quads"] == 2
    _packed_shard_windows(gpu, "70b", "packed_bf16mv", 1 << 14, 16)


def test_packed_bf16mv_on_a_large_grid_equals_the_bf16mv_step(gpu):
    """A shard above 2^26 elements (XCD chunk order) with a ragged tail: the
    device conversions of the bf16-moment state both ways and the packed
    step (nearest and stochastic rounding) agree bit for bit with the
    separate-array steps."""
    torch = gpu
    n, k = (1 << 26) + 4321, 2
    rng = np.random.default_rng(27)
    starts = np.concatenate([[0], np.sort(rng.choice(np.arange(1, n), 999, replace=False))])
    segs = [(int(a), bool(rng.random() < 0.5)) for a in starts]
    w0 = synth.host_normal_f32(n, synth.stream_key(27, 1, 0, 0), 0, n, 0.02)
    m0 = _bf16_bits(synth.host_normal_f32(n, synth.stream_key(27, 1, 1, 0), 0, n, 1e-3))
    v0 = _bf16_bits(synth.host_normal_f32(n, synth.stream_key(27, 1, 2, 0), 0, n, 1e-3) ** 2)
    table = H.segment_tensor(segs, "cuda")
    st, hp = zs.seg_table(table), zs.hparams()
    s = torch.cuda.current_stream()
    for sr in (False, True):
        bw, bm, bv = _dev(torch, w0), _dev(torch, m0), _dev(torch, v0)
        state = torch.empty(zs.packed_bf16mv_floats(n), dtype=torch.float32, device="cuda")
        zs.zs_pack_state_bf16mv(bw, bm, bv, state, n)
        bp = torch.zeros(n, dtype=torch.int16, device="cuda")
        pp = torch.zeros(n, dtype=torch.int16, device="cuda")
        for t in (1, 2):
            gs = [_dev(torch, synth.host_normal_bf16(n, synth.stream_key(27, 2, j, t), 0, n, 0.01))
                  for j in range(k)]
            if sr:
                zs.zs_shard_step_packed_bf16mv_sr(state, pp, gs, k, n, st, hp, t, 77, s)
                zs.zs_shard_step_bf16mv_sr(bw, bm, bv, bp, gs, k, n, st, hp, t, 77, s)
            else:
                zs.zs_shard_step_packed_bf16mv(state, pp, gs, k, n, st, hp, t, s)
                zs.zs_shard_step_bf16mv(bw, bm, bv, bp, gs, k, n, st, hp, t, s)
        ow = torch.empty(n, dtype=torch.float32, device="cuda")
        om = torch.empty(n, dtype=torch.int16, device="cuda")
        ov = torch.empty(n, dtype=torch.int16, device="cuda")
        zs.zs_unpack_state_bf16mv(state, ow, om, ov, n)
        torch.cuda.synchronize()
        assert torch.equal(ow.view(torch.int32), bw.view(torch.int32))
        assert torch.equal(om, bm) and torch.equal(ov, bv) and torch.equal(pp, bp)
        # the host packing of the separate arrays equals the device state
        hs = state.cpu().numpy()
        assert np.array_equal(hs.view(np.uint32), H.pack16_host(
            bw.cpu().numpy(), bm.cpu().numpy().view(np.uint16),
            bv.cpu().numpy().view(np.uint16)).view(np.uint32))
