"""The kernel's fp32 -> bf16 cast over all 2^32 fp32 bit patterns, pinned to
torch's CPU conversion (a library routine, not the oracle).

With lr = 0, weight_decay = 0, zero gradients, zero moments and eps = 1 the
update is the identity (u = 0 / (0 + 1) = 0, w' = w * 1 - 0), so after one
step master must hold its input bit for bit (denormals, signed zeros and
infinities included; NaNs stay NaN), m and v must stay 0, and param must be
round-to-nearest-even of the input, every NaN giving 0x7FC0."""
import numpy as np
import pytest

import sharded_mixed_precision_shard_amd as zs
from tests import _gpu_harness as H

pytestmark = pytest.mark.gpu

CHUNK = 1 << 28


@pytest.fixture(scope="module")
def gpu():
    import torch
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    assert zs.zs_init(0) == zs.ZS_OK
    yield torch
    torch.cuda.synchronize()


def test_every_fp32_pattern(gpu):
    torch = gpu
    n = CHUNK
    dw = torch.empty(n, dtype=torch.int32, device="cuda")
    dm = torch.zeros(n, dtype=torch.float32, device="cuda")
    dv = torch.zeros(n, dtype=torch.float32, device="cuda")
    dp = torch.empty(n, dtype=torch.int16, device="cuda")
    dg = [torch.zeros(n, dtype=torch.int16, device="cuda") for _ in range(2)]
    # both decay branches (df = 1 - 0 * 0 = 1 either way)
    table = H.segment_tensor([(0, True), (n // 3, False), (n // 2, True), (n // 2 + 1, False)],
                             "cuda")
    hp = zs.hparams(lr=0.0, beta1=0.9, beta2=0.95, eps=1.0, weight_decay=0.0)
    base = torch.arange(n, dtype=torch.int64, device="cuda")
    for c in range(1 << 32 >> 28):
        lo = c * n
        vals = base + lo  # the uint32 patterns lo .. lo + n - 1, as int32 bit patterns
        dw.copy_(torch.where(vals >= 1 << 31, vals - (1 << 32), vals).to(torch.int32))
        del vals
        dm.zero_()
        dv.zero_()
        zs.zs_shard_step(dw.view(torch.float32), dm, dv, dp, dg, 2, n, zs.seg_table(table), hp,
                         1, torch.cuda.current_stream())
        torch.cuda.synchronize()
        w_in = np.arange(lo, lo + n, dtype=np.uint32)
        w_out = dw.cpu().numpy().view(np.uint32)
        p_out = dp.cpu().numpy().view(np.uint16)
        f_in = w_in.view(np.float32)
        nan = np.isnan(f_in)
        assert np.array_equal(w_out[~nan], w_in[~nan]), "chunk %d: master changed" % c
        assert np.isnan(w_out.view(np.float32)[nan]).all(), "chunk %d: NaN lost" % c
        assert not dm.any().item() and not dv.any().item(), "chunk %d: moments moved" % c
        want = torch.from_numpy(f_in.copy()).to(torch.bfloat16).view(torch.int16).numpy()
        want = want.view(np.uint16).copy()
        want[nan] = 0x7FC0
        bad = p_out != want
        assert not bad.any(), "chunk %d: %d patterns cast differently, first %#010x" % (
            c, int(bad.sum()), int(w_in[np.argmax(bad)]))


def test_every_pair_of_bf16_partials(gpu):
    """The reduce over all 2^32 pairs (G0, G1) of bf16 partials, pinned to
    numpy's binary32 addition: with beta1 = 0 and zero moments the new first
    moment is 0 + 1 * g, so m exposes fp32(G0) + fp32(G1) (NaNs compared as
    NaN).  lr = 0 keeps the weights finite."""
    torch = gpu
    n = CHUNK
    dw = torch.zeros(n, dtype=torch.float32, device="cuda")
    dm = torch.empty(n, dtype=torch.float32, device="cuda")
    dv = torch.empty(n, dtype=torch.float32, device="cuda")
    dp = torch.empty(n, dtype=torch.int16, device="cuda")
    g0 = torch.empty(n, dtype=torch.int16, device="cuda")
    g1 = torch.empty(n, dtype=torch.int16, device="cuda")
    table = H.segment_tensor([(0, False)], "cuda")
    hp = zs.hparams(lr=0.0, beta1=0.0, beta2=0.5, eps=1.0, weight_decay=0.0)
    low = torch.arange(1 << 16, dtype=torch.int32, device="cuda")
    low16 = torch.where(low >= 1 << 15, low - (1 << 16), low).to(torch.int16)
    for c in range(1 << 32 >> 28):
        hi0 = c << 12  # G0 takes the values hi0 .. hi0 + 4095, each against every G1
        h = torch.arange(hi0, hi0 + (n >> 16), dtype=torch.int32, device="cuda")
        h16 = torch.where(h >= 1 << 15, h - (1 << 16), h).to(torch.int16)
        g0.copy_(h16.repeat_interleave(1 << 16))
        g1.copy_(low16.repeat(n >> 16))
        dm.zero_()
        dv.zero_()
        zs.zs_shard_step(dw, dm, dv, dp, [g0, g1], 2, n, zs.seg_table(table), hp, 1,
                         torch.cuda.current_stream())
        torch.cuda.synchronize()
        a = np.repeat(np.arange(hi0, hi0 + (n >> 16), dtype=np.uint32) << 16, 1 << 16)
        b = np.tile(np.arange(1 << 16, dtype=np.uint32) << 16, n >> 16)
        with np.errstate(invalid="ignore", over="ignore"):
            want = np.float32(0.0) + (a.view(np.float32) + b.view(np.float32))
        got = dm.cpu().numpy()
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), "chunk %d: NaN pattern differs" % c
        same = got.view(np.uint32)[~nan] == want.view(np.uint32)[~nan]
        assert same.all(), "chunk %d: %d sums differ" % (c, int((~same).sum()))


def test_int8_payload_of_every_bf16_pattern(gpu):
    """zs_shard_step_q8ag's int8 payload for parameters taking every bf16 bit
    pattern (in order, shuffled and sign-flipped, so blocks mix magnitudes,
    NaNs and infinities), pinned to torch's formula on the CPU: per block of
    256, scale = max |x| / 127 in binary32 (NaN if any x is NaN), q =
    clamp(round-half-even(x / scale), -127, 127), q = 0 where the scale is 0
    or not finite.  The identity update makes param equal the patterns."""
    torch = gpu
    rng = np.random.default_rng(33)
    pats = np.arange(1 << 16, dtype=np.uint32)
    order = np.concatenate([pats, rng.permutation(pats), rng.permutation(pats) ^ 0x8000,
                            rng.permutation(pats)[: 40_000]]).astype(np.uint32)
    n = order.shape[0]
    w0 = (order << 16).view(np.float32)
    nb = -(-n // zs.ZS_Q8_BLOCK)
    dw = torch.from_numpy(w0.copy()).cuda()
    dm = torch.zeros(n, device="cuda")
    dv = torch.zeros(n, device="cuda")
    dp = torch.zeros(n, dtype=torch.int16, device="cuda")
    dq = torch.zeros(n, dtype=torch.int8, device="cuda")
    ds = torch.zeros(nb, dtype=torch.float32, device="cuda")
    dg = [torch.zeros(n, dtype=torch.int16, device="cuda")]
    table = H.segment_tensor([(0, True)], "cuda")
    hp = zs.hparams(lr=0.0, beta1=0.9, beta2=0.95, eps=1.0, weight_decay=0.0)
    zs.zs_shard_step_q8ag(dw, dm, dv, dp, dq, ds, dg, 1, n, zs.seg_table(table), hp, 1,
                          torch.cuda.current_stream())
    torch.cuda.synchronize()
    p = dp.cpu().numpy().view(np.uint16)
    want_p = (order & 0xFFFF).astype(np.uint16)
    nan_in = np.isnan(w0)
    assert np.array_equal(p[~nan_in], want_p[~nan_in]) and (p[nan_in] == 0x7FC0).all()
    x = torch.from_numpy((p.astype(np.uint32) << 16).view(np.float32).copy())
    pad = torch.zeros(nb * zs.ZS_Q8_BLOCK - n)
    blocks = torch.cat([x, pad]).view(nb, zs.ZS_Q8_BLOCK)
    amax = blocks.abs().amax(dim=1)
    scale = amax / 127.0
    usable = torch.isfinite(scale) & (scale > 0)
    safe = torch.where(usable, scale, torch.ones_like(scale))
    q = torch.clamp(torch.round(blocks / safe[:, None]), -127, 127)
    q = torch.where(usable[:, None], q, torch.zeros_like(q)).to(torch.int8).view(-1)[:n]
    got_s = ds.cpu().numpy()
    want_s = scale.numpy()
    assert np.array_equal(got_s, want_s, equal_nan=True), "block scales differ"
    got_q = dq.cpu().numpy()
    bad = got_q != q.numpy()
    assert not bad.any(), "%d codes differ, first at %d" % (int(bad.sum()), int(np.argmax(bad)))


def test_int8_partials_every_pair(gpu):
    """zs_shard_step_q8grad's dequantize-and-reduce for every pair (q0, q1) of
    int8 codes under 64 random (not power-of-two) block scales each, pinned to
    numpy's binary32 arithmetic: with beta1 = 0 the new m is
    0 + (fl(q0 * s0) + fl(q1 * s1))."""
    torch = gpu
    rng = np.random.default_rng(34)
    reps = 64
    q = np.arange(-128, 128, dtype=np.int32)
    q0 = np.tile(np.repeat(q, 256), reps).astype(np.int8)
    q1 = np.tile(np.tile(q, 256), reps).astype(np.int8)
    n = q0.shape[0]
    nb = -(-n // zs.ZS_Q8_BLOCK)
    s0 = (rng.random(nb) * 1e-2 + 1e-6).astype(np.float32)
    s1 = (rng.random(nb) * 1e-3 + 1e-7).astype(np.float32)
    dm = torch.zeros(n, device="cuda")
    dv = torch.zeros(n, device="cuda")
    dw = torch.zeros(n, device="cuda")
    dp = torch.zeros(n, dtype=torch.int16, device="cuda")
    table = H.segment_tensor([(0, False)], "cuda")
    hp = zs.hparams(lr=0.0, beta1=0.0, beta2=0.5, eps=1.0, weight_decay=0.0)
    dq = [torch.from_numpy(q0.copy()).cuda(), torch.from_numpy(q1.copy()).cuda()]
    dsc = [torch.from_numpy(s0.copy()).cuda(), torch.from_numpy(s1.copy()).cuda()]
    zs.zs_shard_step_q8grad(dw, dm, dv, dp, dq, dsc, 2, n, zs.seg_table(table), hp, 1,
                            torch.cuda.current_stream())
    torch.cuda.synchronize()
    b = np.arange(n) // zs.ZS_Q8_BLOCK
    want = np.float32(0.0) + (q0.astype(np.float32) * s0[b] + q1.astype(np.float32) * s1[b])
    got = dm.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.astype(np.float32).view(np.uint32))


def test_bf16_moments_of_every_pair(gpu):
    """zs_shard_step_bf16mv's moment rounding over all 2^32 pairs of bf16
    partials, pinned to torch's bf16 conversion: with beta1 = beta2 = 0 the
    stored moments are bf16(0 + g) and bf16(0 + g * g), g = fp32(G0) + fp32(G1)."""
    torch = gpu
    n = CHUNK
    dw = torch.zeros(n, dtype=torch.float32, device="cuda")
    dm = torch.empty(n, dtype=torch.int16, device="cuda")
    dv = torch.empty(n, dtype=torch.int16, device="cuda")
    dp = torch.empty(n, dtype=torch.int16, device="cuda")
    g0 = torch.empty(n, dtype=torch.int16, device="cuda")
    g1 = torch.empty(n, dtype=torch.int16, device="cuda")
    table = H.segment_tensor([(0, False)], "cuda")
    hp = zs.hparams(lr=0.0, beta1=0.0, beta2=0.0, eps=1.0, weight_decay=0.0)
    low = torch.arange(1 << 16, dtype=torch.int32, device="cuda")
    low16 = torch.where(low >= 1 << 15, low - (1 << 16), low).to(torch.int16)
    for c in range(1 << 32 >> 28):
        hi0 = c << 12
        h = torch.arange(hi0, hi0 + (n >> 16), dtype=torch.int32, device="cuda")
        g0.copy_(torch.where(h >= 1 << 15, h - (1 << 16), h).to(torch.int16)
                 .repeat_interleave(1 << 16))
        g1.copy_(low16.repeat(n >> 16))
        dm.zero_()
        dv.zero_()
        zs.zs_shard_step_bf16mv(dw, dm, dv, dp, [g0, g1], 2, n, zs.seg_table(table), hp, 1,
                                torch.cuda.current_stream())
        torch.cuda.synchronize()
        a = np.repeat(np.arange(hi0, hi0 + (n >> 16), dtype=np.uint32) << 16, 1 << 16)
        b = np.tile(np.arange(1 << 16, dtype=np.uint32) << 16, n >> 16)
        with np.errstate(invalid="ignore", over="ignore"):
            g = a.view(np.float32) + b.view(np.float32)
            m_ref = np.float32(0.0) + g
            v_ref = np.float32(0.0) + g * g
        for name, dev, ref in (("m", dm, m_ref), ("v", dv, v_ref)):
            want = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy()
            want = want.view(np.uint16).copy()
            want[np.isnan(ref)] = 0x7FC0
            got = dev.cpu().numpy().view(np.uint16)
            bad = got != want
            assert not bad.any(), "chunk %d %s: %d values differ" % (c, name, int(bad.sum()))
