"""A thousand steps in a row, each compared with the oracle bit for bit.

Ten steps show the recurrences; a long run shows that nothing drifts: the
moments and master weights carry every earlier step's rounding, both bias
corrections cross to exactly 1.0f on the way (t = 165 and 338), and the
state stays bitwise the oracle's throughout.  One small shard with short and
long segments, fresh seeded partials every step, checked every 100 steps.
"""
import numpy as np
import pytest

import oracle
import sharded_mixed_precision_shard_amd as zs
from tests import _gpu_harness as H

pytestmark = pytest.mark.gpu

F32 = np.float32
STEPS = 1000


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


@pytest.mark.parametrize("variant", ["base", "bf16mv", "q8grad", "packed", "packed_bf16mv",
                                     "bf16mv_sr", "packed_bf16mv_sr"])
def test_thousand_steps_stay_bitwise(gpu, variant):
    torch = gpu
    rng = np.random.default_rng(4242)
    n, k = 20_011, 2
    nb = -(-n // zs.ZS_Q8_BLOCK)
    segs, a = [], 0
    while a < n:
        segs.append((a, bool(rng.random() < 0.6)))
        a += int(rng.integers(1, 9)) if rng.random() < 0.3 else int(rng.integers(9, 3000))
    mv16 = variant in ("bf16mv", "packed_bf16mv", "bf16mv_sr", "packed_bf16mv_sr")
    seed = 987654321
    packed = variant.startswith("packed")
    w0 = rng.normal(0, 0.02, n).astype(F32)
    mz = np.zeros(n, np.uint16 if mv16 else F32)
    ref = [w0.copy(), mz.copy(), mz.copy(), np.zeros(n, np.uint16)]
    if packed:
        state = _dev(torch, (H.pack16_host if mv16 else H.pack_host)(w0, mz, mz))
    else:
        dw, dm, dv = _dev(torch, w0), _dev(torch, mz), _dev(torch, mz)
    dp = torch.zeros(n, dtype=torch.int16, device="cuda")
    table = H.segment_tensor(segs, "cuda")
    st = zs.seg_table(table)
    hpz = zs.hparams(3e-4, 0.9, 0.95, 1e-8, 0.1, 1.0)
    hpo = oracle.hparams(3e-4, 0.9, 0.95, 1e-8, 0.1, 1.0)
    s = torch.cuda.current_stream()
    for t in range(1, STEPS + 1):
        if variant == "q8grad":
            qs = [rng.integers(-127, 128, n).astype(np.int8) for _ in range(k)]
            ss = [(rng.random(nb) * 1e-4).astype(F32) for _ in range(k)]
            zs.zs_shard_step_q8grad(dw, dm, dv, dp, [_dev(torch, q) for q in qs],
                                    [_dev(torch, x) for x in ss], k, n, st, hpz, t, s)
            assert oracle.shard_step_q8grad(*ref, qs, ss, segs, hpo, t) == 0
        else:
            gs = [_bf16(rng.normal(0, 1e-3, n)) for _ in range(k)]
            dgs = [_dev(torch, g) for g in gs]
            if variant == "base":
                zs.zs_shard_step(dw, dm, dv, dp, dgs, k, n, st, hpz, t, s)
            elif variant == "bf16mv":
                zs.zs_shard_step_bf16mv(dw, dm, dv, dp, dgs, k, n, st, hpz, t, s)
            elif variant == "packed":
                zs.zs_shard_step_packed(state, dp, dgs, k, n, st, hpz, t, s)
            elif variant == "bf16mv_sr":
                zs.zs_shard_step_bf16mv_sr(dw, dm, dv, dp, dgs, k, n, st, hpz, t, seed, s)
            elif variant == "packed_bf16mv_sr":
                zs.zs_shard_step_packed_bf16mv_sr(state, dp, dgs, k, n, st, hpz, t, seed, s)
            else:
                zs.zs_shard_step_packed_bf16mv(state, dp, dgs, k, n, st, hpz, t, s)
            if variant.endswith("_sr"):
                assert oracle.shard_step_bf16mv_sr(*ref, gs, segs, hpo, t, seed) == 0
            else:
                step = oracle.shard_step_bf16mv if mv16 else oracle.shard_step
                assert step(*ref, gs, segs, hpo, t) == 0
        if t % 100 == 0:
            torch.cuda.synchronize()
            if packed:
                got = (H.unpack16_host if mv16 else H.unpack_host)(state.cpu().numpy(), n)
            else:
                mv = (lambda x: x.cpu().numpy().view(np.uint16)) if mv16 \
                    else (lambda x: x.cpu().numpy())
                got = (dw.cpu().numpy(), mv(dm), mv(dv))
            got = tuple(got) + (dp.cpu().numpy().view(np.uint16),)
            assert H.assert_parity(got, ref, "%s t=%d" % (variant, t)), \
                "%s: not bitwise at t=%d" % (variant, t)
