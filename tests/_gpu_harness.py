"""Helpers shared by the GPU parity tests: device state for a workload, the
oracle run over windows of a shard, and the tolerance check.

Inputs on both sides come from the seeded generator: the GPU fills its
buffers with the device twin, the oracle regenerates the same windows with
the host twin (the two are checked bit-identical).  Nothing the oracle sees
comes from the HIP path.
"""
from __future__ import annotations

import numpy as np

import oracle
import sharded_mixed_precision_shard_amd as zs
import synth

F32 = np.float32


def torch():
    import torch as _t
    return _t


class DeviceShard:
    """Device buffers of one rank's shard for a synth Workload."""

    def __init__(self, w: synth.Workload, device="cuda:0"):
        t = torch()
        self.w = w
        n = w.n
        dev = t.device(device)
        self.master = t.empty(n, dtype=t.float32, device=dev)
        self.m = t.zeros(n, dtype=t.float32, device=dev)
        self.v = t.zeros(n, dtype=t.float32, device=dev)
        self.param = t.zeros(n, dtype=t.int16, device=dev)
        self.grads = [t.empty(n, dtype=t.int16, device=dev) for _ in range(w.k)]
        self.table = segment_tensor(w.shard.segments, dev)
        synth.dev_master(w, self.master)

    def fill_grads(self, step):
        synth.dev_grads(self.w, step, self.grads)

    def step(self, t_step, **cfg):
        t = torch()
        w = self.w
        hp = zs.hparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1.0)
        if cfg:
            zs.zs_shard_step_cfg(self.master, self.m, self.v, self.param, self.grads, w.k, w.n,
                                 zs.seg_table(self.table), hp, t_step,
                                 t.cuda.current_stream(), **cfg)
        else:
            zs.zs_shard_step(self.master, self.m, self.v, self.param, self.grads, w.k, w.n,
                             zs.seg_table(self.table), hp, t_step, t.cuda.current_stream())

    def window(self, lo, hi):
        return (self.master[lo:hi].cpu().numpy(), self.m[lo:hi].cpu().numpy(),
                self.v[lo:hi].cpu().numpy(), self.param[lo:hi].cpu().numpy().view(np.uint16))

    def free(self):
        for name in ("master", "m", "v", "param", "grads", "table"):
            setattr(self, name, None)
        torch().cuda.empty_cache()


def segment_tensor(segments, device):
    t = torch()
    rows = [[int(s), 1 if f else 0] for s, f in segments]
    return t.tensor(rows, dtype=t.int64, device=device)


def oracle_window(w: synth.Workload, lo, hi, steps):
    """Run the oracle over shard elements [lo, hi) for the given optimizer
    steps (inputs regenerated on the host).  Returns (master, m, v, param)."""
    n = hi - lo
    master = synth.host_master(w, lo, hi)
    m = np.zeros(n, F32)
    v = np.zeros(n, F32)
    p = np.zeros(n, np.uint16)
    segs = synth.clip_segments(w.shard.segments, lo, hi)
    hp = oracle.hparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1.0)
    for t in steps:
        rc = oracle.shard_step(master, m, v, p, synth.host_grads(w, t, lo, hi), segs, hp, t)
        assert rc == 0
    return master, m, v, p


def bf16_ulp_distance(a, b):
    """Distance in representable bf16 steps between two bit-pattern arrays."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7fff), 0x8000 + x)
    return np.abs(ordered(a) - ordered(b))


def assert_parity(got, ref, where=""):
    """|d| <= 1e-6 * max(1, |x|) on master, m, v; <= 1 bf16 ulp on the param.
    NaN must meet NaN.  Returns True if every output is bitwise equal."""
    bitwise = True
    for name, g, r in zip(("master", "m", "v"), got[:3], ref[:3]):
        gd, rd = g.astype(np.float64), r.astype(np.float64)
        nan_g, nan_r = np.isnan(gd), np.isnan(rd)
        assert np.array_equal(nan_g, nan_r), "%s %s: NaN pattern differs" % (where, name)
        ok = ~nan_r
        err = np.abs(gd[ok] - rd[ok])
        bound = 1e-6 * np.maximum(1.0, np.abs(rd[ok]))
        inf_same = np.isinf(rd[ok]) & (gd[ok] == rd[ok])
        bad = (err > bound) & ~inf_same
        assert not bad.any(), "%s %s: %d elements off, max err %g" % (
            where, name, int(bad.sum()), float(err[bad].max()))
        bitwise &= bool(np.array_equal(g.view(np.uint32), r.view(np.uint32)))
    d = bf16_ulp_distance(got[3], ref[3])
    nan_p = ((ref[3] & 0x7fff) > 0x7f80)
    d = np.where(nan_p & (got[3] == ref[3]), 0, d)
    assert d.max(initial=0) <= 1, "%s param: %d bf16 ulp" % (where, int(d.max()))
    bitwise &= bool(np.array_equal(got[3], ref[3]))
    return bitwise


def boundary_windows(w: synth.Workload, size, max_boundaries=64, n_random=4, seed=0):
    """Windows [lo, hi) of the shard: first, last (ragged tail), ones that
    straddle segment boundaries, and random ones.  Deduplicated, sorted."""
    n = w.n
    size = min(size, n)
    starts = {0, max(0, n - size)}
    bounds = [s for s, _ in w.shard.segments[1:]]
    if len(bounds) > max_boundaries:
        idx = np.linspace(0, len(bounds) - 1, max_boundaries).astype(int)
        bounds = [bounds[i] for i in idx]
    for b in bounds:
        starts.add(int(min(max(0, b - size // 2), n - size)))
    rng = np.random.default_rng(seed)
    for _ in range(n_random):
        starts.add(int(rng.integers(0, n - size + 1)))
    return [(s, s + size) for s in sorted(starts)]
