"""The seeded generator and the model layouts (CPU)."""
import numpy as np

import synth
from oracle import accounting
from synth.layouts import gpt2_small, shard_of, transformer_12d2, workload


def test_splitmix64_published_sequence():
    """SplitMix64 seeded with 0 (Steele, Lea and Flood 2014): the first three
    outputs of the reference generator."""
    assert [synth.splitmix_output(0, i) for i in range(3)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_windows_are_slices_of_the_stream():
    key = synth.stream_key(123, synth.ROLE_GRAD, 3, 7)
    hkey = synth.stream_key(123, synth.ROLE_HEAVY, 3, 7)
    full = synth.host_normal_bf16(10000, key, 5000, 14000, 1e-3, hkey, 0.01, 1.0)
    win = synth.host_normal_bf16(777, key, 5000 + 4321, 14000, 1e-3, hkey, 0.01, 1.0)
    assert np.array_equal(full[4321:4321 + 777], win)
    # padding past valid_end is zero
    assert not full[9000:].any() and full[:9000].any()


def test_normal_statistics():
    key = synth.stream_key(1, synth.ROLE_MASTER, 0, 0)
    x = synth.host_normal_f32(1 << 20, key, 0, 1 << 20, 0.02).astype(np.float64)
    assert abs(x.mean()) < 1e-4
    assert abs(x.std() - 0.02) < 2e-4
    assert np.abs(x).max() < 6.0 * 0.02 + 1e-9  # Irwin-Hall(12) support is +-6 sigma
    # heavy tail: about 1% of the elements carry sigma = 1
    hkey = synth.stream_key(1, synth.ROLE_HEAVY, 0, 1)
    y = synth.host_normal_f32(1 << 20, key, 0, 1 << 20, 1e-3, hkey, 0.01, 1.0)
    frac = np.mean(np.abs(y) > 0.01)
    assert 0.007 < frac < 0.011


def test_streams_differ_by_role_partial_and_step():
    keys = {synth.stream_key(9, r, j, t) for r in (1, 2, 3) for j in range(4) for t in range(4)}
    assert len(keys) == 48


def test_layout_sizes():
    g2 = gpt2_small()
    assert sum(t[1] for t in g2) == 124_439_808
    s = shard_of(g2, 8, 0)
    assert s.n == 15_554_976 and len(s.segments) == 27 and s.padded == s.total
    s7 = shard_of(transformer_12d2(32, 4096), 8, 0)
    assert s7.n == 805_388_288 and len(s7.segments) == 32
    s175 = shard_of(transformer_12d2(96, 12288), 64, 0)
    assert s175.n == 2_718_001_152 and len(s175.segments) == 13
    s70 = shard_of(transformer_12d2(80, 8192, n_heads=64), 8, 0)
    assert s70.n == 8_053_473_280 and len(s70.segments) == 1970
    assert s70.total == accounting.transformer_params(80, 8192)
    assert s175.total == accounting.transformer_params(96, 12288)


def test_every_shard_is_covered_and_sorted():
    for name in ("gpt2-small",):
        w = workload(name)
        for r in range(w.p):
            sh = w.with_rank(r).shard
            starts = [a for a, _ in sh.segments]
            assert starts[0] == 0 and starts == sorted(starts) and starts[-1] < sh.n


def test_decay_off_for_biases_and_norms():
    for name, _, wd in gpt2_small():
        assert wd == (name.split(".")[-1].startswith("w") or name in ("wpe", "wte"))
    for name, _, wd in transformer_12d2(2, 64, n_heads=4):
        assert wd == (".w_" in name)


def test_int8_partials_and_scales():
    key = synth.stream_key(3, synth.ROLE_QGRAD, 1, 2)
    q = synth.host_q8(1 << 18, key, 1000, 1000 + (1 << 18) - 50)
    assert q.dtype == np.int8 and abs(q[:-50].astype(np.float64).std() - synth.Q8_SD) < 1.0
    assert not q[-50:].any()  # padding
    win = synth.host_q8(333, key, 1000 + 4096, 1000 + (1 << 18) - 50)
    assert np.array_equal(win, q[4096:4096 + 333])
    s = synth.host_q8_scales(64, synth.stream_key(3, synth.ROLE_QSCALE, 1, 2), 0, 0.5)
    assert np.all((s >= 0.5) & (s < 1.0))
    s2 = synth.host_q8_scales(10, synth.stream_key(3, synth.ROLE_QSCALE, 1, 2), 20, 0.5)
    assert np.array_equal(s2, s[20:30])
