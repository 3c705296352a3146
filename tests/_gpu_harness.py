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


VARIANTS = ("base", "q8ag", "q8grad", "bf16mv", "packed", "packed_q8ag", "packed_q8grad",
            "packed_bf16mv", "bf16mv_sr", "packed_bf16mv_sr")


def sr_seed(w: synth.Workload) -> int:
    """The random-stream seed the stochastic-rounding steps use for a workload."""
    return (w.seed * 0x9E3779B1 + 17) & (2 ** 64 - 1)


def pack_host(w, m, v):
    """Packed optimizer state on the host, by reshaping: block b holds the
    master values, then m, then v of elements 256b .. 256b + 255; the slots
    past n are +0."""
    n = w.size
    nb = -(-n // 256)
    out = np.zeros((nb, 3, 256), np.float32)
    for j, x in enumerate((w, m, v)):
        pad = np.zeros(nb * 256, np.float32)
        pad[:n] = x
        out[:, j, :] = pad.reshape(nb, 256)
    return out.reshape(-1)


def unpack_host(state, n):
    """(master, m, v) [n] from a packed state (the inverse of pack_host)."""
    blk = np.asarray(state).reshape(-1, 3, 256)
    return tuple(blk[:, j, :].reshape(-1)[:n].copy() for j in range(3))


def pack16_host(w, m16, v16):
    """Packed bf16-moment state on the host, by byte slices: block b is 2048
    bytes, the fp32 master values of elements 256b .. 256b + 255 (1024
    bytes), then their bf16 m (512 bytes), then their bf16 v; zero bytes past
    n.  Returned as float32 (the state's declared type)."""
    n = w.size
    nb = -(-n // 256)
    out = np.zeros((nb, 2048), np.uint8)
    for x, dt, a, z in ((w, np.float32, 0, 1024), (m16, np.uint16, 1024, 1536),
                        (v16, np.uint16, 1536, 2048)):
        pad = np.zeros(nb * 256, dt)
        pad[:n] = x
        out[:, a:z] = pad.view(np.uint8).reshape(nb, z - a)
    return out.reshape(-1).view(np.float32)


def unpack16_host(state, n):
    """(master fp32, m bf16 bits, v bf16 bits) [n] from a packed bf16-moment
    state (the inverse of pack16_host)."""
    blk = np.ascontiguousarray(state).view(np.uint8).reshape(-1, 2048)
    w = np.ascontiguousarray(blk[:, :1024]).reshape(-1).view(np.float32)[:n].copy()
    m = np.ascontiguousarray(blk[:, 1024:1536]).reshape(-1).view(np.uint16)[:n].copy()
    v = np.ascontiguousarray(blk[:, 1536:]).reshape(-1).view(np.uint16)[:n].copy()
    return w, m, v


class DeviceShard:
    """Device buffers of one rank's shard for a synth Workload, for one of the
    entry points: base (zs_shard_step), q8ag (also the int8 parameter copy),
    q8grad (int8 partials), bf16mv (bf16 moments), packed (master, m and v
    in one array, per 256-element block) or packed_bf16mv (the same with bf16
    moments); packed states are filled and read back here with torch views,
    not with the library's conversion calls."""

    def __init__(self, w: synth.Workload, variant="base", device="cuda:0"):
        t = torch()
        self.w = w
        self.variant = variant
        n = w.n
        nb = -(-n // zs.ZS_Q8_BLOCK)
        dev = t.device(device)
        self.seed = sr_seed(w)
        mv_dtype = t.int16 if variant in ("bf16mv", "bf16mv_sr") else t.float32
        self.param = t.zeros(n, dtype=t.int16, device=dev)
        if variant in ("packed", "packed_bf16mv", "packed_bf16mv_sr"):
            # a block is 768 floats (master, m, v), or 512 floats' room
            # (256 fp32 master values, then 256 bf16 m and 256 bf16 v)
            mv16 = variant != "packed"
            floats = zs.packed_bf16mv_floats(n) if mv16 else zs.packed_floats(n)
            self.state = t.zeros(floats, dtype=t.float32, device=dev)
            master = t.empty(n, dtype=t.float32, device=dev)
            synth.dev_master(w, master)
            blocks = self.state.view(-1, 512 if mv16 else 768)
            full = n // 256
            blocks[:full, :256] = master[:full * 256].view(-1, 256)
            if n % 256:
                blocks[full, :n % 256] = master[full * 256:]
            del master
            self.master = self.m = self.v = None
        else:
            self.master = t.empty(n, dtype=t.float32, device=dev)
            self.m = t.zeros(n, dtype=mv_dtype, device=dev)
            self.v = t.zeros(n, dtype=mv_dtype, device=dev)
        self.grads = self.qgrads = self.qscales = self.q8 = self.q8s = None
        if variant == "q8grad":
            self.qgrads = [t.empty(n, dtype=t.int8, device=dev) for _ in range(w.k)]
            self.qscales = [t.empty(nb, dtype=t.float32, device=dev) for _ in range(w.k)]
        else:
            self.grads = [t.empty(n, dtype=t.int16, device=dev) for _ in range(w.k)]
        if variant == "q8ag":
            self.q8 = t.zeros(n, dtype=t.int8, device=dev)
            self.q8s = t.zeros(nb, dtype=t.float32, device=dev)
        self.table = segment_tensor(w.shard.segments, dev)
        if self.master is not None:
            synth.dev_master(w, self.master)

    def fill_grads(self, step):
        if self.variant == "q8grad":
            synth.dev_qgrads(self.w, step, self.qgrads, self.qscales)
        else:
            synth.dev_grads(self.w, step, self.grads)

    def step(self, t_step, **cfg):
        t = torch()
        w = self.w
        hp = zs.hparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1.0)
        st = zs.seg_table(self.table)
        s = t.cuda.current_stream()
        if self.variant == "q8ag":
            zs.zs_shard_step_q8ag(self.master, self.m, self.v, self.param, self.q8, self.q8s,
                                  self.grads, w.k, w.n, st, hp, t_step, s)
        elif self.variant == "q8grad":
            zs.zs_shard_step_q8grad(self.master, self.m, self.v, self.param, self.qgrads,
                                    self.qscales, w.k, w.n, st, hp, t_step, s)
        elif self.variant == "packed":
            zs.zs_shard_step_packed(self.state, self.param, self.grads, w.k, w.n, st, hp, t_step,
                                    s)
        elif self.variant == "packed_bf16mv_sr":
            zs.zs_shard_step_packed_bf16mv_sr(self.state, self.param, self.grads, w.k, w.n, st,
                                              hp, t_step, self.seed, s)
        elif self.variant == "bf16mv_sr":
            zs.zs_shard_step_bf16mv_sr(self.master, self.m, self.v, self.param, self.grads, w.k,
                                       w.n, st, hp, t_step, self.seed, s)
        elif self.variant == "packed_bf16mv":
            zs.zs_shard_step_packed_bf16mv(self.state, self.param, self.grads, w.k, w.n, st, hp,
                                           t_step, s)
        elif self.variant == "bf16mv":
            zs.zs_shard_step_bf16mv(self.master, self.m, self.v, self.param, self.grads, w.k,
                                    w.n, st, hp, t_step, s)
        elif cfg:
            zs.zs_shard_step_cfg(self.master, self.m, self.v, self.param, self.grads, w.k, w.n,
                                 st, hp, t_step, s, **cfg)
        else:
            zs.zs_shard_step(self.master, self.m, self.v, self.param, self.grads, w.k, w.n, st,
                             hp, t_step, s)

    def window(self, lo, hi):
        """(master, m, v, param[, q8, q8 scales of the covered blocks]) on [lo, hi)."""
        if self.variant == "packed":
            b0, b1 = lo // 256, (hi - 1) // 256 + 1
            blk = self.state.view(-1, 3, 256)[b0:b1].cpu().numpy()
            a, z = lo - b0 * 256, hi - b0 * 256
            return (blk[:, 0, :].reshape(-1)[a:z].copy(), blk[:, 1, :].reshape(-1)[a:z].copy(),
                    blk[:, 2, :].reshape(-1)[a:z].copy(),
                    self.param[lo:hi].cpu().numpy().view(np.uint16))
        if self.variant in ("packed_bf16mv", "packed_bf16mv_sr"):
            b0, b1 = lo // 256, (hi - 1) // 256 + 1
            blk = self.state.view(-1, 512)[b0:b1].cpu().numpy()
            a, z = lo - b0 * 256, hi - b0 * 256
            part = lambda c0, c1: np.ascontiguousarray(blk[:, c0:c1]).view(np.uint16)  # noqa
            return (blk[:, :256].reshape(-1)[a:z].copy(), part(256, 384).reshape(-1)[a:z].copy(),
                    part(384, 512).reshape(-1)[a:z].copy(),
                    self.param[lo:hi].cpu().numpy().view(np.uint16))
        mv = (lambda x: x[lo:hi].cpu().numpy().view(np.uint16)) \
            if self.variant in ("bf16mv", "bf16mv_sr") \
            else (lambda x: x[lo:hi].cpu().numpy())
        out = (self.master[lo:hi].cpu().numpy(), mv(self.m), mv(self.v),
               self.param[lo:hi].cpu().numpy().view(np.uint16))
        if self.variant == "q8ag":
            b0, b1 = lo // zs.ZS_Q8_BLOCK, -(-hi // zs.ZS_Q8_BLOCK)
            out = out + (self.q8[lo:hi].cpu().numpy(), self.q8s[b0:b1].cpu().numpy())
        return out

    def free(self):
        for name in ("master", "m", "v", "state", "param", "grads", "qgrads", "qscales", "q8",
                     "q8s", "table"):
            setattr(self, name, None)
        torch().cuda.empty_cache()


def segment_tensor(segments, device):
    t = torch()
    rows = [[int(s), 1 if f else 0] for s, f in segments]
    return t.tensor(rows, dtype=t.int64, device=device)


def oracle_window(w: synth.Workload, lo, hi, steps, variant="base"):
    """Run the oracle over shard elements [lo, hi) for the given optimizer
    steps (inputs regenerated on the host), with the arithmetic of `variant`.
    Quantized variants need lo on a block boundary and hi on one or at n."""
    n = hi - lo
    master = synth.host_master(w, lo, hi)
    mv_dtype = np.uint16 if variant in ("bf16mv", "bf16mv_sr") else F32
    m = np.zeros(n, mv_dtype)
    v = np.zeros(n, mv_dtype)
    p = np.zeros(n, np.uint16)
    segs = synth.clip_segments(w.shard.segments, lo, hi)
    hp = oracle.hparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1.0)
    for t in steps:
        if variant == "q8grad":
            qs, ss = synth.host_qgrads(w, t, lo, hi)
            rc = oracle.shard_step_q8grad(master, m, v, p, qs, ss, segs, hp, t)
        elif variant == "bf16mv":
            rc = oracle.shard_step_bf16mv(master, m, v, p, synth.host_grads(w, t, lo, hi), segs,
                                          hp, t)
        elif variant == "bf16mv_sr":
            rc = oracle.shard_step_bf16mv_sr(master, m, v, p, synth.host_grads(w, t, lo, hi),
                                             segs, hp, t, sr_seed(w), lo)
        else:
            rc = oracle.shard_step(master, m, v, p, synth.host_grads(w, t, lo, hi), segs, hp, t)
        assert rc == 0
    if variant == "q8ag":
        if lo % zs.ZS_Q8_BLOCK or (hi % zs.ZS_Q8_BLOCK and hi != w.n):
            raise ValueError("q8ag windows must be whole quantization blocks")
        q, s = oracle.q8_blocks(p, zs.ZS_Q8_BLOCK)
        return master, m, v, p, q, s
    return master, m, v, p


def bf16_ulp_distance(a, b):
    """Distance in representable bf16 steps between two bit-pattern arrays."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7fff), 0x8000 + x)
    return np.abs(ordered(a) - ordered(b))


def assert_parity(got, ref, where=""):
    """|d| <= 1e-6 * max(1, |x|) on fp32 master, m, v; <= 1 bf16 ulp on the
    param (and on m, v when they are bf16); int8 codes and their scales of the
    quantized parameter copy, when present, exactly (NaN meets NaN).
    Returns True if every output is bitwise equal."""
    bitwise = True
    for name, g, r in zip(("m", "v"), got[1:3], ref[1:3]):
        if g.dtype == np.uint16:
            d = bf16_ulp_distance(g, r)
            assert d.max(initial=0) <= 1, "%s %s: %d bf16 ulp" % (where, name, int(d.max()))
            bitwise &= bool(np.array_equal(g, r))
    if len(got) > 4:
        assert np.array_equal(got[4], ref[4]), "%s q8: %d codes differ" % (
            where, int((got[4] != ref[4]).sum()))
        assert np.array_equal(got[5], ref[5], equal_nan=True), "%s q8 scales differ" % where
    for name, g, r in zip(("master", "m", "v"), got[:3], ref[:3]):
        if g.dtype == np.uint16:
            continue
        gd, rd = g.astype(np.float64), r.astype(np.float64)
        nan_g, nan_r = np.isnan(gd), np.isnan(rd)
        assert np.array_equal(nan_g, nan_r), "%s %s: NaN pattern differs" % (where, name)
        ok = ~nan_r
        with np.errstate(invalid="ignore"):  # inf - inf where both sides hold the same inf
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


def boundary_windows(w: synth.Workload, size, max_boundaries=64, n_random=4, seed=0, align=1):
    """Windows [lo, hi) of the shard: first, last (ragged tail), ones that
    straddle segment boundaries, and random ones.  Deduplicated, sorted.
    With align > 1 every window starts on a multiple of align and has a
    multiple of align elements, except a last window that ends at n."""
    n = w.n
    size = min(size, n)
    if align > 1:
        out = set()
        for lo, hi in boundary_windows(w, size, max_boundaries, n_random, seed):
            a = lo // align * align
            b = min(n, -(-hi // align) * align)
            out.add((a, b))
        return sorted(out)
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
