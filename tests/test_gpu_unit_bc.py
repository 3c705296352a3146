"""GPU parity of the kernels that leave out a bias-correction division.

Once beta^t falls below 2^-25 the correction 1 - beta^t rounds to exactly
1.0f (beta1 = 0.9: t >= 165; beta2 = 0.95: t >= 338), and x / 1.0f == x for
every x, so the library launches a kernel without that division.  These runs
cross both thresholds on every entry point, from non-zero moments, and must
stay bitwise equal to the oracle, which always divides.
"""
import zlib

import numpy as np
import pytest

import oracle
import sharded_mixed_precision_shard_amd as zs
from tests import _gpu_harness as H

pytestmark = pytest.mark.gpu

F32 = np.float32
HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)

# step ranges: no unit correction, across bc1 -> 1, bc1 only, across bc2 -> 1, both
# (tests/test_unit_correction_thresholds.py checks where the thresholds fall)
RANGES = {"none": range(1, 6), "bc1_switch": range(162, 168), "bc1": range(200, 205),
          "bc2_switch": range(335, 341), "both": range(10000, 10005)}


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
    return (x.astype(F32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("variant", H.VARIANTS)
@pytest.mark.parametrize("span", list(RANGES))
def test_unit_correction_kernels_are_bitwise(gpu, variant, span):
    torch = gpu
    rng = np.random.default_rng(zlib.crc32(("%s/%s" % (variant, span)).encode()))
    n, k = 70_001, 2
    nb = -(-n // zs.ZS_Q8_BLOCK)
    segs, a = [], 0
    while a < n:
        segs.append((a, bool(rng.random() < 0.5)))
        a += int(rng.integers(1, 8)) if rng.random() < 0.3 else int(rng.integers(8, 4000))
    w0 = rng.normal(0, 0.02, n).astype(F32)
    m0 = rng.normal(0, 1e-3, n).astype(F32)
    v0 = (rng.normal(0, 1e-3, n) ** 2).astype(F32)
    mv16 = variant in ("bf16mv", "packed_bf16mv", "bf16mv_sr", "packed_bf16mv_sr")
    seed = 0x5EED + len(variant)
    if mv16:
        m0, v0 = _bf16(m0), _bf16(v0)
    ref = [w0.copy(), m0.copy(), v0.copy(), np.zeros(n, np.uint16)]
    dw, dm, dv = _dev(torch, w0), _dev(torch, m0), _dev(torch, v0)
    packed = variant.startswith("packed")
    pack = H.pack16_host if mv16 else H.pack_host
    dstate = _dev(torch, pack(w0, m0, v0)) if packed else None
    dp = torch.zeros(n, dtype=torch.int16, device="cuda")
    dq = torch.zeros(n, dtype=torch.int8, device="cuda")
    ds = torch.zeros(nb, dtype=torch.float32, device="cuda")
    table = H.segment_tensor(segs, "cuda")
    st = zs.seg_table(table)
    hpz, hpo = zs.hparams(**HP), oracle.hparams(**HP)
    s = torch.cuda.current_stream()
    for t in RANGES[span]:
        if variant in ("q8grad", "packed_q8grad"):
            qs = [rng.integers(-127, 128, n).astype(np.int8) for _ in range(k)]
            ss = [(rng.random(nb) * 1e-4).astype(F32) for _ in range(k)]
            dqs, dss = [_dev(torch, q) for q in qs], [_dev(torch, x) for x in ss]
            if packed:
                zs.zs_shard_step_packed_q8grad(dstate, dp, dqs, dss, k, n, st, hpz, t, s)
            else:
                zs.zs_shard_step_q8grad(dw, dm, dv, dp, dqs, dss, k, n, st, hpz, t, s)
            assert oracle.shard_step_q8grad(*ref, qs, ss, segs, hpo, t) == 0
            continue
        gs = [_bf16(rng.normal(0, 1e-3, n)) for _ in range(k)]
        dgs = [_dev(torch, g) for g in gs]
        if variant == "q8ag":
            zs.zs_shard_step_q8ag(dw, dm, dv, dp, dq, ds, dgs, k, n, st, hpz, t, s)
        elif variant == "packed_q8ag":
            zs.zs_shard_step_packed_q8ag(dstate, dp, dq, ds, dgs, k, n, st, hpz, t, s)
        elif variant == "bf16mv":
            zs.zs_shard_step_bf16mv(dw, dm, dv, dp, dgs, k, n, st, hpz, t, s)
        elif variant == "packed":
            zs.zs_shard_step_packed(dstate, dp, dgs, k, n, st, hpz, t, s)
        elif variant == "packed_bf16mv":
            zs.zs_shard_step_packed_bf16mv(dstate, dp, dgs, k, n, st, hpz, t, s)
        elif variant == "bf16mv_sr":
            zs.zs_shard_step_bf16mv_sr(dw, dm, dv, dp, dgs, k, n, st, hpz, t, seed, s)
        elif variant == "packed_bf16mv_sr":
            zs.zs_shard_step_packed_bf16mv_sr(dstate, dp, dgs, k, n, st, hpz, t, seed, s)
        else:
            zs.zs_shard_step(dw, dm, dv, dp, dgs, k, n, st, hpz, t, s)
        if variant.endswith("_sr"):
            assert oracle.shard_step_bf16mv_sr(*ref, gs, segs, hpo, t, seed) == 0
        else:
            step = oracle.shard_step_bf16mv if mv16 else oracle.shard_step
            assert step(*ref, gs, segs, hpo, t) == 0
    torch.cuda.synchronize()
    mv = (lambda x: x.cpu().numpy().view(np.uint16)) if mv16 else (lambda x: x.cpu().numpy())
    got = (dw.cpu().numpy(), mv(dm), mv(dv), dp.cpu().numpy().view(np.uint16))
    if packed:
        unpack = H.unpack16_host if mv16 else H.unpack_host
        got = unpack(dstate.cpu().numpy(), n) + got[3:]
    want = tuple(ref)
    if variant in ("q8ag", "packed_q8ag"):
        got += (dq.cpu().numpy(), ds.cpu().numpy())
        want += oracle.q8_blocks(ref[3], zs.ZS_Q8_BLOCK)
    assert H.assert_parity(got, want, "%s %s" % (variant, span)), \
        "%s over %s: within tolerance but not bitwise equal" % (variant, span)
