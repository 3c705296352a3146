"""GPU parity of the step variants (through the C ABI) against the oracle:
the int8 all-gather payload (zs_shard_step_q8ag), int8 block-quantized
partials (zs_shard_step_q8grad) and bf16 moments (zs_shard_step_bf16mv).
Same bar as the ordinary step; int8 codes and scales must match exactly."""
import numpy as np
import pytest

import oracle
import sharded_mixed_precision_shard_amd as zs
import synth
from tests import _gpu_harness as H

pytestmark = pytest.mark.gpu

F32 = np.float32
BLOCK = zs.ZS_Q8_BLOCK
SIZES = [1, 7, 255, 256, 257, 511, 512, 513, 2047, 2049, 4096, 10007, 65539]


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


def _segments(rng, n):
    segs, a = [], 0
    while a < n:
        segs.append((a, bool(rng.random() < 0.5)))
        a += int(rng.integers(1, 8)) if rng.random() < 0.4 else int(rng.integers(8, 3000))
    return segs


def _bf16_partials(rng, k, n, sigma=1e-2):
    return [(rng.normal(0, sigma, n).astype(F32).view(np.uint32) >> 16).astype(np.uint16)
            for _ in range(k)]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("k", [1, 2, 5, 16])
def test_q8ag_matches_oracle(gpu, n, k):
    torch = gpu
    rng = np.random.default_rng(100 + n * 7 + k)
    segs = _segments(rng, n)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    ref = [w0.copy(), np.zeros(n, F32), np.zeros(n, F32), np.zeros(n, np.uint16)]
    dw, dm, dv = _dev(torch, w0), _dev(torch, ref[1]), _dev(torch, ref[2])
    dp = torch.zeros(n, dtype=torch.int16, device="cuda")
    nb = -(-n // BLOCK)
    dq = torch.full((n,), 99, dtype=torch.int8, device="cuda")
    ds = torch.full((nb,), -1.0, dtype=torch.float32, device="cuda")
    table = H.segment_tensor(segs, "cuda")
    for t in (1, 2, 3):
        gs = _bf16_partials(rng, k, n)
        if t == 3 and n > 300:
            gs[0][n // 2] = 0x7FC0  # a NaN partial poisons one element and its block
        zs.zs_shard_step_q8ag(dw, dm, dv, dp, dq, ds, [_dev(torch, g) for g in gs], k, n,
                              zs.seg_table(table), zs.hparams(), t, torch.cuda.current_stream())
        assert oracle.shard_step(*ref, gs, segs, oracle.hparams(), t) == 0
    torch.cuda.synchronize()
    q, s = oracle.q8_blocks(ref[3], BLOCK)
    got = (dw.cpu().numpy(), dm.cpu().numpy(), dv.cpu().numpy(),
           dp.cpu().numpy().view(np.uint16), dq.cpu().numpy(), ds.cpu().numpy())
    H.assert_parity(got, tuple(ref) + (q, s), "q8ag n=%d k=%d" % (n, k))
    if n > 300:
        assert np.isnan(got[5][(n // 2) // BLOCK])


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("k", [1, 3, 8, 16])
def test_q8grad_matches_oracle(gpu, n, k):
    torch = gpu
    rng = np.random.default_rng(200 + n * 7 + k)
    segs = _segments(rng, n)
    nb = -(-n // BLOCK)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    ref = [w0.copy(), np.zeros(n, F32), np.zeros(n, F32), np.zeros(n, np.uint16)]
    dw, dm, dv = _dev(torch, w0), _dev(torch, ref[1]), _dev(torch, ref[2])
    dp = torch.zeros(n, dtype=torch.int16, device="cuda")
    table = H.segment_tensor(segs, "cuda")
    for t in (1, 2, 3):
        qs = [rng.integers(-127, 128, n).astype(np.int8) for _ in range(k)]
        ss = [(rng.random(nb) * 1e-4).astype(F32) for _ in range(k)]
        zs.zs_shard_step_q8grad(dw, dm, dv, dp, [_dev(torch, q) for q in qs],
                                [_dev(torch, s) for s in ss], k, n, zs.seg_table(table),
                                zs.hparams(), t, torch.cuda.current_stream())
        assert oracle.shard_step_q8grad(*ref, qs, ss, segs, oracle.hparams(), t) == 0
    torch.cuda.synchronize()
    got = (dw.cpu().numpy(), dm.cpu().numpy(), dv.cpu().numpy(),
           dp.cpu().numpy().view(np.uint16))
    H.assert_parity(got, ref, "q8grad n=%d k=%d" % (n, k))


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("k", [1, 2, 8, 16])
def test_bf16mv_matches_oracle(gpu, n, k):
    torch = gpu
    rng = np.random.default_rng(300 + n * 7 + k)
    segs = _segments(rng, n)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    ref = [w0.copy(), np.zeros(n, np.uint16), np.zeros(n, np.uint16), np.zeros(n, np.uint16)]
    dw = _dev(torch, w0)
    dm = torch.zeros(n, dtype=torch.int16, device="cuda")
    dv = torch.zeros(n, dtype=torch.int16, device="cuda")
    dp = torch.zeros(n, dtype=torch.int16, device="cuda")
    table = H.segment_tensor(segs, "cuda")
    for t in range(1, 11):
        gs = _bf16_partials(rng, k, n, 1e-3)
        zs.zs_shard_step_bf16mv(dw, dm, dv, dp, [_dev(torch, g) for g in gs], k, n,
                                zs.seg_table(table), zs.hparams(), t,
                                torch.cuda.current_stream())
        assert oracle.shard_step_bf16mv(*ref, gs, segs, oracle.hparams(), t) == 0
    torch.cuda.synchronize()
    got = (dw.cpu().numpy(), dm.cpu().numpy().view(np.uint16), dv.cpu().numpy().view(np.uint16),
           dp.cpu().numpy().view(np.uint16))
    H.assert_parity(got, ref, "bf16mv n=%d k=%d" % (n, k))


def test_variant_argument_errors(gpu):
    torch = gpu
    n = 1024
    f = [torch.zeros(n, dtype=torch.float32, device="cuda") for _ in range(3)]
    p = torch.zeros(n, dtype=torch.int16, device="cuda")
    g = [torch.zeros(n, dtype=torch.int16, device="cuda")]
    q = torch.zeros(n, dtype=torch.int8, device="cuda")
    s = torch.zeros(4, dtype=torch.float32, device="cuda")
    st = zs.seg_table(H.segment_tensor([(0, True)], "cuda"))
    hp = zs.hparams()
    ok = zs.ZS_OK
    assert zs.zs_shard_step_q8ag(*f, p, q, s, g, 1, n, st, hp, 1, None, check=False) == ok
    assert zs.zs_shard_step_q8ag(*f, p, 0, s, g, 1, n, st, hp, 1, None, check=False) == \
        zs.ZS_ERR_INVALID_ARGUMENT
    assert zs.zs_shard_step_q8ag(*f, p, q.data_ptr() + 4, s, g, 1, n - 8, st, hp, 1, None,
                                 check=False) == zs.ZS_ERR_MISALIGNED
    assert zs.zs_shard_step_q8ag(*f, p, q, s.data_ptr() + 2, g, 1, n, st, hp, 1, None,
                                 check=False) == zs.ZS_ERR_MISALIGNED
    assert zs.zs_shard_step_q8ag(*f, p, p, s, g, 1, n, st, hp, 1, None, check=False) == \
        zs.ZS_ERR_ALIASING
    assert zs.zs_shard_step_q8ag(*f, p, q, f[0], g, 1, n, st, hp, 1, None, check=False) == \
        zs.ZS_ERR_ALIASING
    assert zs.zs_shard_step_q8grad(*f, p, [q], [s], 1, n, st, hp, 1, None, check=False) == ok
    assert zs.zs_shard_step_q8grad(*f, p, [q], [0], 1, n, st, hp, 1, None, check=False) == \
        zs.ZS_ERR_INVALID_ARGUMENT
    assert zs.zs_shard_step_q8grad(*f, p, [q], [s], 1, n, st, hp, 0, None, check=False) == \
        zs.ZS_ERR_INVALID_ARGUMENT
    assert zs.zs_shard_step_q8grad(*f, p, [f[0]], [s], 1, n, st, hp, 1, None, check=False) == \
        zs.ZS_ERR_ALIASING
    mb = torch.zeros(n, dtype=torch.int16, device="cuda")
    vb = torch.zeros(n, dtype=torch.int16, device="cuda")
    assert zs.zs_shard_step_bf16mv(f[0], mb, vb, p, g, 1, n, st, hp, 1, None, check=False) == ok
    assert zs.zs_shard_step_bf16mv(f[0], mb, mb, p, g, 1, n, st, hp, 1, None, check=False) == \
        zs.ZS_ERR_ALIASING
    torch.cuda.synchronize()


def test_device_int8_generator_matches_host(gpu):
    torch = gpu
    n, nb = 100_003, 400
    key = synth.stream_key(5, synth.ROLE_QGRAD, 2, 7)
    skey = synth.stream_key(5, synth.ROLE_QSCALE, 2, 7)
    dq = torch.empty(n, dtype=torch.int8, device="cuda")
    ds = torch.empty(nb, dtype=torch.float32, device="cuda")
    synth.dev_q8(dq, n, key, 777, 90_000)
    synth.dev_q8_scales(ds, nb, skey, 3, synth.q8_base_scale(1e-3))
    torch.cuda.synchronize()
    assert np.array_equal(dq.cpu().numpy(), synth.host_q8(n, key, 777, 90_000))
    assert np.array_equal(ds.cpu().numpy(),
                          synth.host_q8_scales(nb, skey, 3, synth.q8_base_scale(1e-3)))


def _large_variant(torch, name, variant, window, max_boundaries, step_ts=None):
    w = synth.workload(name)
    free, _ = torch.cuda.mem_get_info()
    per = {"base": 14 + 2 * w.k, "q8ag": 15 + 2 * w.k, "q8grad": 14 + w.k,
           "bf16mv": 10 + 2 * w.k}[variant]
    if free < w.n * per + (2 << 30):
        pytest.skip("needs %.1f GB of free device memory" % (w.n * per / 1e9))
    print("%s %s: n=%d k=%d" % (name, variant, w.n, w.k), flush=True)
    ds = H.DeviceShard(w, variant)
    ts = list(range(1, w.prewarm_steps + 1)) + w.step_ts() if step_ts is None else list(step_ts)
    for t in ts:
        ds.fill_grads(t)
        ds.step(t)
    torch.cuda.synchronize()
    wins = H.boundary_windows(w, window, max_boundaries=max_boundaries, n_random=3, seed=2,
                              align=BLOCK)
    got = [ds.window(lo, hi) for lo, hi in wins]
    ds.free()
    for (lo, hi), g in zip(wins, got):
        H.assert_parity(g, H.oracle_window(w, lo, hi, ts, variant),
                        "%s %s [%d,%d)" % (name, variant, lo, hi))


@pytest.mark.parametrize("variant", ["q8ag", "q8grad", "bf16mv"])
def test_variants_on_70b_shard_windows(gpu, variant):
    """The full 70B-shaped rank-0 shard (8.05e9 elements, 1970 segments,
    t = 10000..10002) in each variant's default launch, compared on windows
    around segment boundaries and at the ragged ends."""
    _large_variant(gpu, "70b", variant, 1 << 14, 48)


@pytest.mark.parametrize("ts", [(1, 2, 3), (200, 201, 202)], ids=["t1", "t200"])
def test_bf16mv_wide_kernel_other_corrections(gpu, ts):
    """The 70B-shaped shard takes the bf16-moment step's wide launch (two
    sub-windows per wave, occupancy cap 5); at t = 10000 both bias corrections
    are 1.0f, here neither (t = 1..3) and only the first (t = 200..202)."""
    plan = zs.zs_launch_plan(2, synth.workload("70b").n, "bf16mv")
    assert plan["window_quads"] == 2
    _large_variant(gpu, "70b", "bf16mv", 1 << 14, 24, step_ts=ts)


@pytest.mark.parametrize("variant", ["q8ag", "q8grad", "bf16mv"])
def test_variants_on_gpt2_shard_windows(gpu, variant):
    _large_variant(gpu, "gpt2-small", variant, 1 << 14, 30)


@pytest.mark.parametrize("variant", ["base", "cfg", "q8ag", "q8grad", "bf16mv"])
def test_prepared_call_matches_the_plain_call(gpu, variant):
    """zs.ShardStep (arguments checked and marshalled once) gives the same bits
    as the plain entry-point call on twin buffers, over three steps."""
    torch = gpu
    n, k = 70_001, 3
    rng = np.random.default_rng(7)
    segs = _segments(rng, n)
    nb = -(-n // BLOCK)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    mvt = torch.int16 if variant == "bf16mv" else torch.float32

    def twin():
        d = dict(w=_dev(torch, w0), m=torch.zeros(n, dtype=mvt, device="cuda"),
                 v=torch.zeros(n, dtype=mvt, device="cuda"),
                 p=torch.zeros(n, dtype=torch.int16, device="cuda"),
                 q8=torch.zeros(n, dtype=torch.int8, device="cuda"),
                 q8s=torch.zeros(nb, dtype=torch.float32, device="cuda"))
        return d

    a, b = twin(), twin()
    table = H.segment_tensor(segs, "cuda")
    st, hp = zs.seg_table(table), zs.hparams()
    qs = [_dev(torch, rng.integers(-127, 128, n).astype(np.int8)) for _ in range(k)]
    ss = [_dev(torch, (rng.random(nb) * 1e-4).astype(F32)) for _ in range(k)]
    gs = [_dev(torch, g) for g in _bf16_partials(rng, k, n)]
    cfg = dict(chunk_tiles=3, block_order=2, groups_per_cu=4)
    if variant == "q8grad":
        call = zs.ShardStep(b["w"], b["m"], b["v"], b["p"], qs, n, st, hp, variant="q8grad",
                            qscales=ss)
    elif variant == "q8ag":
        call = zs.ShardStep(b["w"], b["m"], b["v"], b["p"], gs, n, st, hp, variant="q8ag",
                            param_q8=b["q8"], param_q8_scale=b["q8s"])
    elif variant == "bf16mv":
        call = zs.ShardStep(b["w"], b["m"], b["v"], b["p"], gs, n, st, hp, variant="bf16mv")
    else:
        call = zs.ShardStep(b["w"], b["m"], b["v"], b["p"], gs, n, st, hp,
                            cfg=cfg if variant == "cfg" else None)
    s = torch.cuda.current_stream()
    for t in (1, 2, 3):
        if variant == "q8grad":
            zs.zs_shard_step_q8grad(a["w"], a["m"], a["v"], a["p"], qs, ss, k, n, st, hp, t, s)
        elif variant == "q8ag":
            zs.zs_shard_step_q8ag(a["w"], a["m"], a["v"], a["p"], a["q8"], a["q8s"], gs, k, n,
                                  st, hp, t, s)
        elif variant == "bf16mv":
            zs.zs_shard_step_bf16mv(a["w"], a["m"], a["v"], a["p"], gs, k, n, st, hp, t, s)
        elif variant == "cfg":
            zs.zs_shard_step_cfg(a["w"], a["m"], a["v"], a["p"], gs, k, n, st, hp, t, s, **cfg)
        else:
            zs.zs_shard_step(a["w"], a["m"], a["v"], a["p"], gs, k, n, st, hp, t, s)
        call(t, s)
    torch.cuda.synchronize()
    for key in ("w", "m", "v", "p", "q8", "q8s"):
        assert torch.equal(a[key].view(torch.uint8), b[key].view(torch.uint8)), key


def test_bf16mv_wide_kernel_ragged_tail(gpu):
    """A bf16-moment shard above 2^32 elements whose length is not a multiple
    of the wide kernel's 2048-element tile (nor of 256): the last window runs
    the element-by-element tail.  The buffers are zero except three windows
    (the first, one across a segment boundary, the last) that get seeded
    values; those are compared with the oracle after three steps."""
    torch = gpu
    n, k = (1 << 32) + 2777, 2
    plan = zs.zs_launch_plan(k, n, "bf16mv")
    assert plan["window_quads"] == 2 and n % plan["chunk_elements"]
    need = n * (4 + 2 + 2 + 2 + 2 * k) + (2 << 30)
    free, _ = torch.cuda.mem_get_info()
    if free < need:
        pytest.skip("needs %.1f GB of free device memory" % (need / 1e9))
    L = 20_000
    bnd = 3_000_000_017
    segs = [(0, True), (bnd, False), (bnd + 5, True), (n - 1500, False)]
    wins = [(0, L), (bnd - L // 2, bnd + L // 2), (n - L, n)]
    rng = np.random.default_rng(41)
    w = torch.zeros(n, dtype=torch.float32, device="cuda")
    m = torch.zeros(n, dtype=torch.int16, device="cuda")
    v = torch.zeros(n, dtype=torch.int16, device="cuda")
    p = torch.zeros(n, dtype=torch.int16, device="cuda")
    grads = [torch.zeros(n, dtype=torch.int16, device="cuda") for _ in range(k)]
    ref = []
    for lo, hi in wins:
        w0 = rng.normal(0, 0.02, hi - lo).astype(F32)
        w[lo:hi] = torch.from_numpy(w0).cuda()
        ref.append([w0, np.zeros(hi - lo, np.uint16), np.zeros(hi - lo, np.uint16),
                    np.zeros(hi - lo, np.uint16)])
    table = H.segment_tensor(segs, "cuda")
    st, hpz, hpo = zs.seg_table(table), zs.hparams(), oracle.hparams()
    for t in (1, 2, 3):
        gs = [[_bf16_partials(rng, 1, hi - lo, 1e-3)[0] for _ in range(k)] for lo, hi in wins]
        for (lo, hi), gw in zip(wins, gs):
            for j in range(k):
                grads[j][lo:hi] = _dev(torch, gw[j])
        zs.zs_shard_step_bf16mv(w, m, v, p, grads, k, n, st, hpz, t, torch.cuda.current_stream())
        for (lo, hi), gw, r in zip(wins, gs, ref):
            assert oracle.shard_step_bf16mv(*r, gw, synth.clip_segments(segs, lo, hi), hpo,
                                            t) == 0
    torch.cuda.synchronize()
    for (lo, hi), r in zip(wins, ref):
        got = (w[lo:hi].cpu().numpy(), m[lo:hi].cpu().numpy().view(np.uint16),
               v[lo:hi].cpu().numpy().view(np.uint16), p[lo:hi].cpu().numpy().view(np.uint16))
        assert H.assert_parity(got, r, "wide tail [%d,%d)" % (lo, hi))
