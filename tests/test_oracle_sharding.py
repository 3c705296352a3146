"""Sharding invariants of the oracle (CPU).

FlatZeRO1 ("Lecture 7: Parallelism I", section 8.1) splits one flat,
zero-padded buffer evenly over p ranks; each rank updates only its slice.
Because AdamW is elementwise, running every rank's shard step and
concatenating the slices must give, bit for bit, plain AdamW over the whole
padded buffer on the reduced gradient -- the analogue of the page's
observation that the sharded optimizer matches DDP bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from synth.layouts import decay_mask_full, shard_of

F32 = np.float32


def _random_tensors(rng, total):
    out, a = [], 0
    while a < total:
        size = int(rng.integers(1, 8)) if rng.random() < 0.7 else int(rng.integers(8, 300))
        size = min(size, total - a)
        out.append(("t%d" % len(out), size, bool(rng.random() < 0.6)))
        a += size
    return out


def _fold(parts):
    g = oracle.bf16_to_f32(parts[0]).copy()
    for h in parts[1:]:
        g = g + oracle.bf16_to_f32(h)
    return g


@pytest.mark.parametrize("p", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("k", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("total", [1, 7, 64, 1000, 4099])
def test_concatenated_shards_equal_unsharded(p, k, total):
    rng = np.random.default_rng(1000 * p + 10 * k + total)
    tensors = _random_tensors(rng, total)
    seed = int(rng.integers(1 << 62))
    sh0 = shard_of(tensors, p, 0)
    padded = sh0.padded
    key_w = synth.stream_key(seed, synth.ROLE_MASTER, 0, 0)
    w_full = synth.host_normal_f32(padded, key_w, 0, total, 0.02)
    m_full = np.zeros(padded, F32)
    v_full = np.zeros(padded, F32)
    p_full = np.zeros(padded, np.uint16)
    mask = decay_mask_full(tensors, padded)
    shards = []
    for r in range(p):
        sh = shard_of(tensors, p, r)
        lo, hi = sh.index0, sh.index0 + sh.n
        shards.append((sh, w_full[lo:hi].copy(), np.zeros(sh.n, F32), np.zeros(sh.n, F32),
                       np.zeros(sh.n, np.uint16)))
    hp = oracle.hparams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    for t in range(1, 11):
        parts = [synth.host_normal_bf16(padded, synth.stream_key(seed, synth.ROLE_GRAD, j, t), 0,
                                        total, 0.01) for j in range(k)]
        assert oracle.adamw_unsharded(w_full, m_full, v_full, p_full, _fold(parts), mask, hp,
                                      t) == 0
        for sh, w, m, v, pb in shards:
            lo, hi = sh.index0, sh.index0 + sh.n
            rc = oracle.shard_step(w, m, v, pb, [x[lo:hi].copy() for x in parts], sh.segments,
                                   hp, t)
            assert rc == 0
    cat = [np.concatenate([s[i] for s in shards]) for i in range(1, 5)]
    assert np.array_equal(cat[0].view(np.uint32), w_full.view(np.uint32))
    assert np.array_equal(cat[1].view(np.uint32), m_full.view(np.uint32))
    assert np.array_equal(cat[2].view(np.uint32), v_full.view(np.uint32))
    assert np.array_equal(cat[3], p_full)
    # padding stays exactly +0
    assert not w_full[total:].view(np.uint32).any() and not p_full[total:].any()


def test_k1_is_unsharded_adamw():
    rng = np.random.default_rng(11)
    n = 5000
    w0 = rng.normal(0, 0.02, n).astype(F32)
    segs = [(0, True), (17, False), (18, True), (3000, False)]
    mask = np.zeros(n, np.uint8)
    mask[:17] = 1
    mask[18:3000] = 1
    a = [w0.copy(), np.zeros(n, F32), np.zeros(n, F32), np.zeros(n, np.uint16)]
    b = [w0.copy(), np.zeros(n, F32), np.zeros(n, F32), np.zeros(n, np.uint16)]
    hp = oracle.hparams()
    for t in range(1, 11):
        g = (rng.normal(0, 0.01, n).astype(F32).view(np.uint32) >> 16).astype(np.uint16)
        oracle.shard_step(*a, [g], segs, hp, t)
        oracle.adamw_unsharded(*b, oracle.bf16_to_f32(g).copy(), mask, hp, t)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_segment_lookup_semantics():
    """Element i takes the flag of the LAST entry with start <= i: duplicate
    starts (empty segments) and entries past the end are allowed."""
    n = 40
    segs = [(0, False), (5, True), (5, False), (5, True), (9, False), (9, True), (33, False),
            (40, True), (100, True)]
    want = np.zeros(n, np.uint8)
    want[5:9] = 1
    want[9:33] = 1
    rng = np.random.default_rng(12)
    w0 = rng.normal(0, 0.02, n).astype(F32)
    g = (rng.normal(0, 0.01, n).astype(F32).view(np.uint32) >> 16).astype(np.uint16)
    hp = oracle.hparams(weight_decay=0.5)
    a = [w0.copy(), np.zeros(n, F32), np.zeros(n, F32), np.zeros(n, np.uint16)]
    b = [w0.copy(), np.zeros(n, F32), np.zeros(n, F32), np.zeros(n, np.uint16)]
    oracle.shard_step(*a, [g], segs, hp, 1)
    oracle.adamw_unsharded(*b, oracle.bf16_to_f32(g).copy(), want, hp, 1)
    assert np.array_equal(a[0], b[0])


def test_padding_segment_layout():
    """Length not divisible by p: the tail is zero padding in a decay-free
    segment (exercise 1(e) of the lecture notes: pad with zeros)."""
    tensors = [("a", 2, True)]
    shards = [shard_of(tensors, 4, r) for r in range(4)]
    assert [s.n for s in shards] == [1, 1, 1, 1]
    assert shards[0].segments == [(0, True)]
    assert shards[2].segments == [(0, False)] and shards[3].segments == [(0, False)]
