#!/usr/bin/env python3
"""Benchmark of one rank's fused ZeRO-shard AdamW step on one MI355X.

A step is one zs_shard_step call over the whole shard: sum the k bf16
partials, AdamW on the fp32 master/m/v, write the bf16 parameter copy.
Inputs are seeded and synthetic, shaped like the model shards of the
workload (see synth/layouts.py), resident in HBM before timing starts.

Default workload: the 70B-shaped shard (80 layers, d = 8192, rank 0 of 8,
8,053,473,280 elements, 1,970 weight-decay segments, k = 2 partials,
t = 10000...), the largest shard of the set and one of the >= 1e9-element
shards.  Other workloads: --config {tiny,gpt2-small,7b,175b,70b}.

Prints ONE JSON line on stdout (rank 0): the metric (achieved HBM GB/s by
the algorithmic byte count, and params/s), the roofline of the kernel
measured with HIP events on the launch stream, and the CPU oracle timed on
a bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD's published figure
KERNEL_SRCS = [os.path.join(ROOT, "sharded_mixed_precision_shard_amd", "csrc", f)
               for f in ("zs_kernels.hip", "zs_kernels.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C++ source without comments and with runs of white space collapsed
    (the kernel sources hold no string literal with comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """sha256[:16] over the code of the kernel sources (device code and the
    argument block it reads), comments and layout ignored, in a fixed order;
    host-side changes leave it alone."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(config: str, launch_key: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source and launch configuration."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(config)
    if not ent or ent.get("kernel_sha") != kernel_source_hash() or \
            ent.get("launch") != launch_key:
        return None
    return ent.get("bytes_per_launch")


def launch_key(plan: dict) -> str:
    """The launch a step resolves to (zs_launch_plan), as the key under which
    measured traffic is stored: any change of the library's defaults that
    changes grid, chunk, chunk order, occupancy cap or cache policy changes it."""
    key = "wg=%d,chunk=%d,order=%d,cap=%d,nt=%d" % (
        plan["workgroups"], plan["chunk_elements"], plan["block_order"],
        plan["groups_per_cu"], plan["nontemporal"])
    if plan.get("window_quads", 1) != 1:
        key += ",quads=%d" % plan["window_quads"]
    return key


def host_info():
    """CPU model, online CPUs and the CPUs this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "online_cpus": os.cpu_count(),
            "usable_cpus": len(os.sched_getaffinity(0))}


# The threaded oracle uses at most 16 threads, one GPU's share of the CPUs of
# an eight-GPU MI355X host, whatever the host has online.
HOST_THREAD_CAP = 16


def oracle_threads() -> int:
    return max(1, min(len(os.sched_getaffinity(0)), HOST_THREAD_CAP))


# the arithmetic families with bf16 moments
MV16 = ("bf16mv", "bf16mv_sr")


def sr_seed(w) -> int:
    """The random-stream seed the stochastic-rounding steps use on a workload."""
    return (w.seed * 0x9E3779B1 + 17) & (2 ** 64 - 1)


# ---------------------------------------------------------------- parity windows

PARITY_WINDOW = 1 << 20


def parity_windows(w, n: int, count: int = 10):
    """Windows [a, b) of the shard that the cpu_baseline leg replays with the
    oracle: the first, the last (the tail), up to six around segment
    boundaries and random ones; starts on 256-element block boundaries."""
    import random
    L = min(PARITY_WINDOW, n)

    def at(a):
        a = max(0, min(a, n - L)) // 256 * 256
        return (a, min(a + L, n))

    wins = [at(0), at(n - L)]
    starts = [s for s, _ in w.shard.segments[1:] if 0 < s < n]
    if starts:
        pick = sorted(set(starts[i * len(starts) // 6] for i in range(min(6, len(starts)))))
        wins += [at(s - L // 2) for s in pick]
    rng = random.Random(w.seed)
    while len(wins) < count:
        wins.append(at(rng.randrange(0, max(1, n - L))))
    out = []
    for x in sorted(set(wins)):
        if not out or x[0] >= out[-1][1]:
            out.append(x)
    return out


def snapshot(tensors, wins):
    """D2H copies of the windows of each tensor: {name: [np.ndarray per window]}."""
    out = {}
    for name, t in tensors.items():
        if t is None:
            continue
        out[name] = [t[a:b].cpu().numpy().copy() for a, b in wins]
    return out


def snapshot_packed(state, wins, mv16=False):
    """The windows' master, m and v read out of a packed state (block b of 256
    elements: their master values, then m, then v; with mv16 a block is 512
    floats' room, 256 fp32 master values then 256 bf16 m and 256 bf16 v), as
    snapshot() gives them."""
    import numpy as np
    blocks = state.view(-1, 512 if mv16 else 768)
    cols = ((0, 256), (256, 384), (384, 512)) if mv16 else ((0, 256), (256, 512), (512, 768))
    out = {"master": [], "m": [], "v": []}
    for a, b in wins:
        b0, b1 = a // 256, (b - 1) // 256 + 1
        blk = blocks[b0:b1].cpu().numpy()
        lo, hi = a - b0 * 256, b - b0 * 256
        for j, name in enumerate(("master", "m", "v")):
            part = np.ascontiguousarray(blk[:, cols[j][0]:cols[j][1]])
            if mv16 and j:
                part = part.view(np.int16)  # as a bf16 array's snapshot reads
            out[name].append(part.reshape(-1)[lo:hi].copy())
    return out


# the packed-state form of each entry point that has one
PACKED_FORM = {"base": "packed", "q8ag": "packed_q8ag", "q8grad": "packed_q8grad",
               "bf16mv": "packed_bf16mv", "bf16mv_sr": "packed_bf16mv_sr"}


def packed_state_floats(var, n):
    """Floats (or floats' room) of the packed state of entry point `var`."""
    import sharded_mixed_precision_shard_amd as zs
    return zs.packed_bf16mv_floats(n) if "bf16mv" in var else zs.packed_floats(n)


def packed_leg(torch, w, var, pstate, bufs, st, hp, stream, args, bytes_per_step):
    """The packed-state form of entry point `var` on `pstate` (packed from the
    separate-array step's state before its warm-up), over the same steps with
    the same partials: GB/s per launch (HIP events on the launch stream), its
    twin in its own launch, and whether its final state and outputs equal the
    separate-array step's bit for bit on the parity windows."""
    import numpy as np
    import sharded_mixed_precision_shard_amd as zs
    n, k = w.n, w.k
    pvar = PACKED_FORM[var]
    param, q8, q8s = bufs["param"], bufs["q8"], bufs["q8s"]
    wins = parity_windows(w, n)
    want = snapshot({name: bufs[name] for name in ("master", "m", "v", "param", "q8")}, wins)
    if q8s is not None:
        want["q8s"] = [block_slice(q8s, a, b).cpu().numpy().copy() for a, b in wins]
    partials = bufs["qgrads"] if pvar == "packed_q8grad" else bufs["grads"]
    call = zs.ShardStep(pstate, None, None, param, partials, n, st, hp, variant=pvar,
                        param_q8=q8, param_q8_scale=q8s, qscales=bufs["qscales"],
                        seed=sr_seed(w) if pvar.endswith("_sr") else None)
    t = w.t0
    for _ in range(args.warmup):
        call(t, stream)
        t += 1
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record(stream)
        call(t, stream)
        ends[i].record(stream)
        t += 1
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    avg = sum(ms) / len(ms)
    got = snapshot_packed(pstate, wins, mv16="bf16mv" in pvar)
    got.update(snapshot({"param": param, "q8": q8}, wins))
    if q8s is not None:
        got["q8s"] = [block_slice(q8s, a, b).cpu().numpy().copy() for a, b in wins]
    same = all(np.array_equal(x.view(np.uint8), y.view(np.uint8))
               for name in want for x, y in zip(got[name], want[name]))
    plan = zs.zs_launch_plan(k, n, pvar)
    achieved = bytes_per_step / (avg * 1e-3) / 1e9
    out = {"entry_point": "zs_shard_step_" + pvar, "launch": launch_key(plan),
           "achieved": round(achieved, 2), "frac": round(achieved / HBM_PEAK_GBPS, 4),
           "avg_launch_ms": round(avg, 4), "steps": args.steps,
           "separate_arrays_entry_point": "zs_shard_step" + ("" if var == "base" else "_" + var),
           "bitwise_equal_to_separate_arrays": bool(same)}
    if not args.no_twin:
        twin = Twin(torch, pvar, dict(bufs, master=pstate, m=None, v=None), k, n, plan)
        if twin.ok:
            r = twin.rate("step", stream)
            out["twin_step_gbps"] = round(r, 1)
            out["pct_of_twin"] = round(100.0 * achieved / r, 2)
    return out


def _fill_packed_master(state, master, n, mv16=False):
    """Write fp32 master [n] into the master slots of a packed state (the
    first 256 floats of each block of 768, or of 512 with bf16 moments; torch
    copies into strided views; m, v and the padding keep what they hold)."""
    blocks = state.view(-1, 512 if mv16 else 768)
    full = n // 256
    blocks[:full, :256] = master[:full * 256].view(-1, 256)
    if n % 256:
        blocks[full, :n % 256] = master[full * 256:]


def block_slice(t, a, b):
    return t[a // 256:-(-b // 256)]


def _rel_err(got, ref):
    import numpy as np
    g = got.astype(np.float64)
    r = ref.astype(np.float64)
    both_nan = np.isnan(g) & np.isnan(r)
    d = np.where(both_nan, 0.0, np.abs(g - r) / np.maximum(1.0, np.abs(r)))
    d = np.where(np.isnan(d), np.inf, d)
    return float(d.max()) if d.size else 0.0


def _bf16_ulp(got, ref):
    import numpy as np
    g = got.view(np.uint16).astype(np.int64)
    r = ref.view(np.uint16).astype(np.int64)
    nan = lambda x: ((x & 0x7fff) > 0x7f80)  # noqa: E731
    same = (g == r) | (nan(g) & nan(r))
    # signed-magnitude order of the bit patterns
    key = lambda x: np.where(x & 0x8000, -(x & 0x7fff), x)  # noqa: E731
    d = np.where(same, 0, np.abs(key(g) - key(r)))
    return int(d.max()) if d.size else 0


def cpu_baseline(w, seconds: float, variant: str, bytes_per_elem: float, parity=None):
    """The CPU oracle, as it stands, on bounded samples of the same workload.

    1. Parity (when `parity` holds the GPU run's windows): the oracle replays
       the timed run's step sequence on the windows' initial state and the
       resident partials, and its results are compared with the GPU's state
       after the timed steps (the step is elementwise, so a window's result
       depends only on that window's inputs).
    2. Throughput: the oracle, single-threaded, on the first min(n, 2^27)
       elements of the shard for about `seconds`, and the same oracle driven
       from T threads over T contiguous ranges of that window."""
    par = _parity_replay(w, variant, parity) if parity else None
    res = _throughput_sample(w, seconds, variant, bytes_per_elem)
    res["parity"] = par
    return res


def _parity_replay(w, variant, par):
    import numpy as np

    import oracle
    import synth

    wins, before, after, ts = par["windows"], par["before"], par["after"], par["ts"]
    hp = oracle.hparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1.0)
    errs = {"master": 0.0, "m": 0.0, "v": 0.0}
    ulp_p = ulp_mv = dq = 0
    exact = True
    elems = 0
    t_start = time.perf_counter()
    for i, (a, b) in enumerate(wins):
        n = b - a
        elems += n
        master = before["master"][i].copy()
        m = before["m"][i].copy()
        v = before["v"][i].copy()
        p = np.zeros(n, np.uint16)
        segs = synth.clip_segments(w.shard.segments, a, b)
        for t in ts:
            if variant == "q8grad":
                rc = oracle.shard_step_q8grad(master, m, v, p, [q[i] for q in par["qgrads"]],
                                              [s[i] for s in par["qscales"]], segs, hp, t)
            elif variant == "bf16mv":
                rc = oracle.shard_step_bf16mv(master, m.view(np.uint16), v.view(np.uint16), p,
                                              [g[i].view(np.uint16) for g in par["grads"]],
                                              segs, hp, t)
            elif variant == "bf16mv_sr":
                rc = oracle.shard_step_bf16mv_sr(master, m.view(np.uint16), v.view(np.uint16),
                                                 p, [g[i].view(np.uint16) for g in par["grads"]],
                                                 segs, hp, t, sr_seed(w), a)
            else:
                rc = oracle.shard_step(master, m, v, p,
                                       [g[i].view(np.uint16) for g in par["grads"]], segs, hp, t)
            assert rc == 0, rc
        gm, gmm, gv = after["master"][i], after["m"][i], after["v"][i]
        gp = after["param"][i].view(np.uint16)
        exact &= gm.tobytes() == master.tobytes() and gmm.tobytes() == m.tobytes() and \
            gv.tobytes() == v.tobytes() and gp.tobytes() == p.tobytes()
        errs["master"] = max(errs["master"], _rel_err(gm, master))
        if variant in MV16:
            ulp_mv = max(ulp_mv, _bf16_ulp(gmm, m), _bf16_ulp(gv, v))
        else:
            errs["m"] = max(errs["m"], _rel_err(gmm, m))
            errs["v"] = max(errs["v"], _rel_err(gv, v))
        ulp_p = max(ulp_p, _bf16_ulp(gp, p))
        if variant == "q8ag":
            q, sc = oracle.q8_blocks(p, 256)
            gq = after["q8"][i]
            gs = after["q8s"][i]
            exact &= gq.tobytes() == q.tobytes() and gs.tobytes() == sc.tobytes()
            dq = max(dq, int(np.abs(gq.astype(np.int32) - q.astype(np.int32)).max()))
    elapsed = time.perf_counter() - t_start
    out = {"windows": len(wins), "window_elements": elems, "steps_replayed": len(ts),
           "first_t": ts[0], "last_t": ts[-1],
           "max_rel_err": {k: float("%.3g" % e) for k, e in errs.items()
                           if not (variant in MV16 and k != "master")},
           "max_param_bf16_ulp": ulp_p, "bitwise_equal": bool(exact),
           "oracle_seconds": round(elapsed, 3)}
    if variant in MV16:
        out["max_moment_bf16_ulp"] = ulp_mv
    if variant == "q8ag":
        out["max_q8_code_diff"] = dq
    tol_ok = all(e <= 1e-6 for e in errs.values()) and ulp_p <= 1 and ulp_mv <= 1 and dq <= 1
    out["within_tolerance"] = bool(tol_ok)
    out["tolerance"] = "|d| <= 1e-6*max(1,|x|) on fp32 master/m/v, <= 1 bf16 ulp on bf16 outputs"
    return out


def _throughput_sample(w, seconds, variant, bytes_per_elem):
    import numpy as np

    import oracle
    import synth

    n = min(w.n, 1 << 27)
    threads = oracle_threads()
    master = synth.host_master(w, 0, n, threads=threads)
    mv_dtype = np.uint16 if variant in MV16 else np.float32
    m = np.zeros(n, mv_dtype)
    v = np.zeros(n, mv_dtype)
    p = np.zeros(n, np.uint16)
    if variant == "q8grad":
        qgrads, qscales = synth.host_qgrads(w, w.t0, 0, n)
    else:
        grads = synth.host_grads(w, w.t0, 0, n, threads=threads)
    segs = synth.clip_segments(w.shard.segments, 0, n)
    hp = oracle.hparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1.0)
    steps = 0
    elapsed = 0.0
    t = w.t0
    warm = True  # one untimed step first: the first touch of the fresh arrays
    while elapsed < seconds or steps == 0:
        t0 = time.perf_counter()
        if variant == "q8grad":
            rc = oracle.shard_step_q8grad(master, m, v, p, qgrads, qscales, segs, hp, t)
        elif variant == "bf16mv":
            rc = oracle.shard_step_bf16mv(master, m, v, p, grads, segs, hp, t)
        elif variant == "bf16mv_sr":
            rc = oracle.shard_step_bf16mv_sr(master, m, v, p, grads, segs, hp, t, sr_seed(w))
        else:
            rc = oracle.shard_step(master, m, v, p, grads, segs, hp, t)
            if variant == "q8ag":
                oracle.q8_blocks(p, 256)
        assert rc == 0
        t += 1
        if warm:
            warm = False
            continue
        elapsed += time.perf_counter() - t0
        steps += 1
    threaded = _threaded_oracle(master, m, v, p, grads if variant != "q8grad" else None,
                                segs, hp, t, variant, bytes_per_elem, threads,
                                qgrads if variant == "q8grad" else None,
                                qscales if variant == "q8grad" else None, seed=sr_seed(w))
    return {
        "value": round(n * steps * bytes_per_elem / elapsed / 1e9, 4),
        "unit": "GB/s",
        "params_per_s": round(n * steps / elapsed, 1),
        "cores": 1,
        "threaded": threaded,
        "kind": "oracle",
        "host": host_info(),
        "sample": "first %d elements of the %s shard (k=%d, %d segments in the window), "
                  "%d timed oracle steps after one untimed (%s arithmetic), single-threaded C, %.1f s" % (
                      n, w.name.split(":")[0].split(" (")[0], w.k, len(segs), steps, variant,
                      elapsed),
    }


def _threaded_oracle(master, m, v, p, grads, segs, hp, t, variant, bytes_per_elem, threads,
                     qgrads=None, qscales=None, seconds=3.0, seed=0):
    """The same oracle driven from T threads over T contiguous ranges of the
    window (the step is elementwise, so the split does not change a bit);
    T = the CPUs this process may use, at most HOST_THREAD_CAP."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import synth

    n = master.shape[0]
    # ranges on 256-element boundaries so that q8 blocks never straddle two threads
    per = -(-n // threads)
    per = -(-per // 256) * 256
    ranges = [(a, min(a + per, n)) for a in range(0, n, per)]
    tabs = [synth.clip_segments(segs, a, b) for a, b in ranges]

    def one(i, step):
        a, b = ranges[i]
        if variant == "q8grad":
            return oracle.shard_step_q8grad(master[a:b], m[a:b], v[a:b], p[a:b],
                                            [q[a:b] for q in qgrads],
                                            [s[a // 256:-(-b // 256)] for s in qscales],
                                            tabs[i], hp, step)
        if variant == "bf16mv":
            return oracle.shard_step_bf16mv(master[a:b], m[a:b], v[a:b], p[a:b],
                                            [g[a:b] for g in grads], tabs[i], hp, step)
        if variant == "bf16mv_sr":
            return oracle.shard_step_bf16mv_sr(master[a:b], m[a:b], v[a:b], p[a:b],
                                               [g[a:b] for g in grads], tabs[i], hp, step,
                                               seed, a)
        rc = oracle.shard_step(master[a:b], m[a:b], v[a:b], p[a:b], [g[a:b] for g in grads],
                               tabs[i], hp, step)
        if variant == "q8ag":
            oracle.q8_blocks(p[a:b], 256)
        return rc

    steps, elapsed = 0, 0.0
    with ThreadPoolExecutor(len(ranges)) as ex:
        while elapsed < seconds or steps == 0:
            t0 = time.perf_counter()
            assert all(rc == 0 for rc in ex.map(one, range(len(ranges)),
                                                [t] * len(ranges)))
            elapsed += time.perf_counter() - t0
            steps += 1
            t += 1
    return {"value": round(n * steps * bytes_per_elem / elapsed / 1e9, 4),
            "params_per_s": round(n * steps / elapsed, 1), "cores": len(ranges),
            "steps": steps,
            "thread_rule": "the CPUs this process may use, at most %d (one GPU's share of "
                           "the host)" % HOST_THREAD_CAP}


def _ceiling_lib():
    import ctypes
    path = os.path.join(ROOT, "sharded_mixed_precision_shard_amd", "libzs_ceiling.so")
    if not os.path.exists(path):
        raise ImportError("libzs_ceiling.so is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.zs_ceiling_copy.argtypes = [P, P, ctypes.c_int64, P]
    lib.zs_ceiling_copy.restype = ctypes.c_int
    lib.zs_ceiling_twin.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P, P, P, P, P,
                                    ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, P]
    lib.zs_ceiling_twin.restype = ctypes.c_int
    return lib


def twin_bytes(variant: str, k: int, n: int):
    """(read, written) bytes of the step's streams over n elements."""
    nb = -(-n // 256)
    return {"base": ((12 + 2 * k) * n, 14 * n),
            "packed": ((12 + 2 * k) * n, 14 * n),
            "packed_q8ag": ((12 + 2 * k) * n, 15 * n + 4 * nb),
            "packed_q8grad": (12 * n + k * (n + 4 * nb), 14 * n),
            "packed_bf16mv": ((8 + 2 * k) * n, 10 * n),
            "bf16mv_sr": ((8 + 2 * k) * n, 10 * n),
            "packed_bf16mv_sr": ((8 + 2 * k) * n, 10 * n),
            "q8ag": ((12 + 2 * k) * n, 15 * n + 4 * nb),
            "q8grad": (12 * n + k * (n + 4 * nb), 14 * n),
            "bf16mv": ((8 + 2 * k) * n, 10 * n)}[variant]


# launch shapes (chunk order, occupancy cap; 32 never binds) the bench also
# runs the twin in, besides the step's own
TWIN_SHAPES = [(2, 32), (2, 4), (2, 5), (2, 6), (1, 32)]


class Twin:
    """The step's traffic without its arithmetic (libzs_ceiling.so), on the
    step's own buffers and in the step's own launch."""
    MODES = {"step": 0, "read": 1, "write": 2}
    LAYOUT = {"base": 0, "q8ag": 1, "q8grad": 2, "bf16mv": 4, "packed": 8, "packed_q8ag": 9,
              "packed_q8grad": 10, "packed_bf16mv": 12, "bf16mv_sr": 4, "packed_bf16mv_sr": 12}

    def __init__(self, torch, variant, bufs, k, n, plan):
        import ctypes
        self.torch, self.variant, self.k = torch, variant, k
        self.bufs = bufs
        self.lib = _ceiling_lib()
        self.chunk = plan["chunk_elements"]
        self.quads = plan.get("window_quads", 1)
        self.n = n // self.chunk * self.chunk if self.chunk else 0
        self.ok = plan["nontemporal"] == 1 and self.n > 0 and \
            self.chunk % (1024 * self.quads) == 0
        self.plan = plan
        ptr = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else 0)  # noqa: E731
        self.head = [ptr(bufs["master"]), ptr(bufs.get("m")), ptr(bufs.get("v")),
                     ptr(bufs["param"]),
                     ptr(bufs.get("q8")), ptr(bufs.get("q8s"))]
        q8g = variant in ("q8grad", "packed_q8grad")
        gl = bufs.get("qgrads") if q8g else bufs["grads"]
        self.gp = (ctypes.c_void_p * k)(*[g.data_ptr() for g in gl])
        sl = bufs.get("qscales") if q8g else None
        self.sp = (ctypes.c_void_p * k)(*[s.data_ptr() for s in sl]) if sl else None

    def launch(self, mode, stream):
        import ctypes
        rc = self.lib.zs_ceiling_twin(
            self.MODES[mode], self.LAYOUT[self.variant], *self.head,
            ctypes.cast(self.gp, ctypes.c_void_p),
            ctypes.cast(self.sp, ctypes.c_void_p) if self.sp is not None else None,
            self.k, self.n, self.chunk, self.plan["block_order"], self.plan["groups_per_cu"],
            self.quads, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("zs_ceiling_twin(%s) failed: %d" % (mode, rc))

    def rate(self, mode, stream, reps=4):
        """GB/s of one mode: the bytes it moves over its mean HIP-event time."""
        torch = self.torch
        rb, wb = twin_bytes(self.variant, self.k, self.n)
        nbytes = {"step": rb + wb, "read": rb, "write": wb}[mode]
        self.launch(mode, stream)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(reps):
            self.launch(mode, stream)
        e.record(stream)
        torch.cuda.synchronize()
        return nbytes / (s.elapsed_time(e) / reps * 1e-3) / 1e9


def copy_ceiling(torch, nbytes: int):
    """Device-to-device copies of nbytes, read + write GB/s: torch's copy_ (the
    runtime's blit kernel, also the byte-counter calibration of the profiles)
    and the streaming copy of libzs_ceiling.so (the step's access pattern)."""
    lib = _ceiling_lib()
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    stream = torch.cuda.current_stream()
    copies = {
        "torch": lambda: dst.copy_(src),
        "stream": lambda: lib.zs_ceiling_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                                              stream.cuda_stream),
    }
    out = {}
    for name, f in copies.items():
        for _ in range(2):
            rc = f()
            assert not isinstance(rc, int) or rc == 0, rc
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        torch.cuda.synchronize()
        s.record(stream)
        for _ in range(reps):
            f()
        e.record(stream)
        torch.cuda.synchronize()
        out[name] = 2 * nbytes / (s.elapsed_time(e) / reps * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return out


def host_copy_ceiling(nbytes: int, threads: int):
    """Host memory copy bandwidth (read + write GB/s): `threads` threads each
    copying a contiguous slice with numpy (which releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    n = nbytes // 4
    src = np.ones(n, np.float32)
    dst = np.empty(n, np.float32)
    dst.fill(0.0)  # map every destination page before anything is timed
    step = -(-n // threads)
    parts = [(dst[a:a + step], src[a:a + step]) for a in range(0, n, step)]
    best = 0.0
    with ThreadPoolExecutor(threads) as ex:
        for _ in range(10):
            t0 = time.perf_counter()
            list(ex.map(lambda ds: np.copyto(ds[0], ds[1]), parts))
            best = max(best, 2 * nbytes / (time.perf_counter() - t0) / 1e9)
    return best


def offload_main(args):
    """The ZeRO-Offload host step on host memory: one shard step of the
    workload per timed step, all host threads.  The roofline reference is the
    host's measured copy bandwidth (no published peak for this host)."""
    import numpy as np

    import sharded_mixed_precision_shard_amd as zs
    import synth

    w = synth.workload(args.config)
    n, k = w.n, w.k
    threads = zs.zs_host_max_threads()
    bytes_per_step = zs.algorithmic_bytes("base", k, n)
    log("offload workload: %s  n=%d k=%d, %d host threads, %s" % (
        w.name, n, k, threads, zs.zs_host_isa()))
    ceiling = host_copy_ceiling(min(4 << 30, 4 * n), threads)
    log("host copy ceiling: %.1f GB/s" % ceiling)
    master = synth.host_master(w, threads=threads)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    p = np.zeros(n, np.uint16)
    for a in (m, v, p):  # np.zeros maps pages lazily: touch them before anything is timed
        a.fill(0)
    grads = synth.host_grads(w, w.t0, threads=threads)
    log("host inputs generated")
    segs = zs.host_segments(w.shard.segments)
    hp = zs.hparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1.0)
    # pre-warm steps reuse the resident partials (drawing fresh host partials
    # for each of them would dominate the run; traffic does not depend on values)
    for t in range(1, w.prewarm_steps + 1):
        zs.zs_host_shard_step(master, m, v, p, grads, k, n, segs, hp, t)
        if t % 20 == 0:
            log("pre-warm step %d" % t)
    t = w.t0
    for _ in range(args.warmup):
        zs.zs_host_shard_step(master, m, v, p, grads, k, n, segs, hp, t)
        t += 1
    times = []
    for _ in range(args.steps):
        t0 = time.perf_counter()
        zs.zs_host_shard_step(master, m, v, p, grads, k, n, segs, hp, t)
        times.append(time.perf_counter() - t0)
        t += 1
    log("host step: %.3f ms average over %d steps" % (1e3 * sum(times) / len(times), len(times)))
    elapsed = sum(times)
    value = bytes_per_step * args.steps / elapsed / 1e9
    cpu = cpu_baseline(w, args.cpu_seconds, "base", 26 + 2 * k) if args.cpu_seconds > 0 \
        else None
    out = {
        "metric": "achieved host DRAM GB/s and params/s for the ZeRO-Offload shard AdamW step",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 0,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage": "f32 master/m/v, bf16 partials and param",
        "data": "synthetic (seeded SplitMix64 / Irwin-Hall draws)",
        "config": {"workload": w.name, "entry_point": "zs_host_shard_step", "shard_params": n,
                   "k_partials": k, "segments": len(w.shard.segments),
                   "bytes_per_param": 26 + 2 * k, "bytes_per_step": bytes_per_step,
                   "host_threads": threads, "isa": zs.zs_host_isa()},
        "params_per_s": round(n * args.steps / elapsed, 1),
        "roofline": {"bound": "host-dram", "achieved": round(value, 2),
                     "peak": round(ceiling, 1), "unit": "GB/s",
                     "frac": round(value / ceiling, 4), "traffic": None,
                     "peak_kind": "measured host copy bandwidth (threaded numpy copy, "
                                  "read + write)"},
        "cpu_baseline": cpu,
        "speedup_vs_cpu_oracle": None if not cpu else {
            "single_thread": round(value / cpu["value"], 1),
            "threaded": round(value / cpu["threaded"]["value"], 1)},
    }
    print(json.dumps(out), flush=True)


SWEEP_CFGS = [
    ("default", None),
    ("linear", dict(block_order=1, groups_per_cu=32)),
    ("linear,cap5", dict(block_order=1, groups_per_cu=5)),
    ("xcd", dict(block_order=2, groups_per_cu=32)),
    ("xcd,cap4", dict(block_order=2, groups_per_cu=4)),
    ("xcd,cap5", dict(block_order=2, groups_per_cu=5)),
    ("xcd,cap6", dict(block_order=2, groups_per_cu=6)),
    ("xcd,cap8", dict(block_order=2, groups_per_cu=8)),
]


def sweep_main(args):
    """Launch configurations of zs_shard_step_cfg (chunk order x occupancy
    cap; groups_per_cu = 32 never binds) on one set of buffers, interleaved
    over --rounds rounds in one process: per round and configuration the
    step's per-launch rate (HIP events, --steps launches) and its twin's
    (the same traffic with no arithmetic, in the same launch).  Prints one
    JSON line."""
    import torch

    import sharded_mixed_precision_shard_amd as zs
    import synth

    torch.cuda.set_device(0)
    assert zs.zs_init(0) == zs.ZS_OK
    w = synth.workload(args.config)
    n, k = w.n, w.k
    dev = torch.device("cuda:0")
    master = torch.empty(n, dtype=torch.float32, device=dev)
    m = torch.zeros(n, dtype=torch.float32, device=dev)
    v = torch.zeros(n, dtype=torch.float32, device=dev)
    param = torch.zeros(n, dtype=torch.int16, device=dev)
    grads = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(k)]
    table = torch.tensor([[s, 1 if f else 0] for s, f in w.shard.segments], dtype=torch.int64,
                         device=dev)
    st = zs.seg_table(table)
    hp = zs.hparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1.0)
    stream = torch.cuda.current_stream()
    synth.dev_master(w, master)
    synth.dev_grads(w, w.t0, grads)
    bufs = dict(master=master, m=m, v=v, param=param, grads=grads)
    runs = []
    for name, cfg in SWEEP_CFGS:
        plan = zs.zs_launch_plan(k, n, "base", cfg)
        runs.append(dict(name=name, key=launch_key(plan), plan=plan,
                         call=zs.ShardStep(master, m, v, param, grads, n, st, hp, cfg=cfg),
                         twin=Twin(torch, "base", bufs, k, n, plan), kernel=[], twin_gbps=[]))
    nbytes = zs.algorithmic_bytes("base", k, n)
    t = w.t0
    for r in range(args.rounds):
        for run in runs:
            run["call"](t, stream)
            t += 1
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                run["call"](t, stream)
                t += 1
            e1.record(stream)
            torch.cuda.synchronize()
            run["kernel"].append(nbytes / (e0.elapsed_time(e1) / args.steps * 1e-3) / 1e9)
            run["twin_gbps"].append(run["twin"].rate("step", stream, reps=max(2, args.steps // 2)))
        log("round %d: %s" % (r, ", ".join("%s %.0f" % (x["name"], x["kernel"][-1]) for x in runs)))
    out = {"metric": "launch sweep of zs_shard_step_cfg: achieved HBM GB/s per configuration",
           "unit": "GB/s", "config": {"workload": w.name, "shard_params": n, "k_partials": k,
                                      "rounds": args.rounds, "launches_per_round": args.steps},
           "sweep": {x["name"]: {"launch": x["key"],
                                 "kernel_gbps": [round(y, 1) for y in x["kernel"]],
                                 "kernel_median": round(statistics.median(x["kernel"]), 1),
                                 "twin_gbps": [round(y, 1) for y in x["twin_gbps"]],
                                 "twin_median": round(statistics.median(x["twin_gbps"]), 1)}
                     for x in runs}}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 10; 200 for the tiny and GPT-2 shards, whose "
                         "steps take microseconds)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="70b")
    ap.add_argument("--variant", default="base",
                    choices=("base", "q8ag", "q8grad", "bf16mv", "packed", "packed_q8ag",
                             "packed_q8grad", "packed_bf16mv", "bf16mv_sr", "packed_bf16mv_sr",
                             "offload"),
                    help="entry point: zs_shard_step (base), zs_shard_step_q8ag, "
                         "zs_shard_step_q8grad, zs_shard_step_bf16mv, zs_shard_step_packed "
                         "(master, m, v packed per 256-element block), zs_shard_step_packed_q8ag, "
                         "zs_shard_step_packed_q8grad, zs_shard_step_packed_bf16mv, "
                         "zs_shard_step_bf16mv_sr and zs_shard_step_packed_bf16mv_sr (bf16 "
                         "moments rounded stochastically), or the host "
                         "(ZeRO-Offload) step zs_host_shard_step, which runs on the CPU "
                         "and needs no GPU")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle time budget for the cpu_baseline leg (0 = skip)")
    ap.add_argument("--chunk-tiles", type=int, default=0, help="launch geometry override")
    ap.add_argument("--nontemporal", type=int, default=0, help="0 default, 1 on, 2 off")
    ap.add_argument("--groups-per-cu", type=int, default=0,
                    help="cap on resident workgroups per compute unit (0 = default)")
    ap.add_argument("--block-order", type=int, default=0,
                    help="0 default, 1 linear, 2 XCD-contiguous chunk order")
    ap.add_argument("--graph", action="store_true",
                    help="record the timed steps into one HIP graph and launch it once "
                         "(per-launch times are then the graph's average per step)")
    ap.add_argument("--copy-gb", type=float, default=8.0,
                    help="size of the in-run copy-ceiling measurement (0 = skip)")
    ap.add_argument("--no-twin", action="store_true",
                    help="skip the twin ceilings (the step's traffic without arithmetic)")
    ap.add_argument("--sweep", action="store_true",
                    help="measure zs_shard_step_cfg's launch configurations (chunk order x "
                         "occupancy cap) on one set of buffers instead of the timed run")
    ap.add_argument("--rounds", type=int, default=3, help="rounds of --sweep")
    ap.add_argument("--no-packed", action="store_true",
                    help="skip the same-run measurement of the packed-state form "
                         "(zs_shard_step_packed, _packed_q8ag, _packed_q8grad, _packed_bf16mv: "
                         "the same step on the state packed per 256-element block) beside "
                         "zs_shard_step, zs_shard_step_q8ag, zs_shard_step_q8grad or "
                         "zs_shard_step_bf16mv")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 200 if args.config in ("tiny", "gpt2-small") else 10

    if args.variant != "base" and (args.chunk_tiles or args.nontemporal or args.groups_per_cu
                                   or args.block_order):
        ap.error("--chunk-tiles, --nontemporal, --groups-per-cu and --block-order apply to the "
                 "base entry point (zs_shard_step_cfg) only")
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one rank's shard step on ONE GPU; the shard step has no "
              "cross-GPU work (the reduce-scatter and all-gather around it are not built). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.variant == "offload":
        offload_main(args)
        return
    if args.sweep:
        if args.variant != "base":
            ap.error("--sweep measures the base entry point")
        sweep_main(args)
        return

    import torch

    import sharded_mixed_precision_shard_amd as zs
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    rc = zs.zs_init(0)
    if rc != zs.ZS_OK:
        raise zs.ZsError(rc, "zs_init")

    w = synth.workload(args.config)
    n, k = w.n, w.k
    var = args.variant
    bytes_per_step = zs.algorithmic_bytes(var, k, n)
    bpe = bytes_per_step / n
    if var == "base":
        assert zs.zs_algorithmic_bytes(k, n) == bytes_per_step
    log("workload: %s  n=%d k=%d segments=%d bytes/step=%.3f GB" % (
        w.name, n, k, len(w.shard.segments), bytes_per_step / 1e9))
    cfg = dict(chunk_tiles=args.chunk_tiles, nontemporal=args.nontemporal,
               groups_per_cu=args.groups_per_cu, block_order=args.block_order)
    cfg = cfg if any(cfg.values()) else None
    plan = zs.zs_launch_plan(k, n, var, cfg)
    key = launch_key(plan)
    log("launch: %s" % key)

    copies = {}
    if args.copy_gb > 0:
        copies = copy_ceiling(torch, int(args.copy_gb * 1e9) // 4096 * 4096)
        log("copies of %.1f GB: streaming %.1f GB/s, torch copy_ %.1f GB/s" % (
            args.copy_gb, copies["stream"], copies["torch"]))

    dev = torch.device("cuda:0")
    nb = -(-n // zs.ZS_Q8_BLOCK)
    mv_dtype = torch.int16 if var in MV16 else torch.float32
    packed_var = var.startswith("packed")
    q8grad_var = var in ("q8grad", "packed_q8grad")
    q8ag_var = var in ("q8ag", "packed_q8ag")
    # the oracle arithmetic the variant computes (the packed forms compute their plain form's)
    arith = {"packed": "base", "packed_q8ag": "q8ag", "packed_q8grad": "q8grad",
             "packed_bf16mv": "bf16mv", "packed_bf16mv_sr": "bf16mv_sr"}.get(var, var)
    mv16 = arith in MV16
    state = master = m = v = None
    if packed_var:
        # master, m and v in one array, per 256-element block
        state = torch.empty(packed_state_floats(var, n), dtype=torch.float32, device=dev)
    else:
        master = torch.empty(n, dtype=torch.float32, device=dev)
        m = torch.zeros(n, dtype=mv_dtype, device=dev)
        v = torch.zeros(n, dtype=mv_dtype, device=dev)
    param = torch.zeros(n, dtype=torch.int16, device=dev)
    grads = qgrads = qscales = q8 = q8s = None
    if q8grad_var:
        qgrads = [torch.empty(n, dtype=torch.int8, device=dev) for _ in range(k)]
        qscales = [torch.empty(nb, dtype=torch.float32, device=dev) for _ in range(k)]
    else:
        grads = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(k)]
    if q8ag_var:
        q8 = torch.zeros(n, dtype=torch.int8, device=dev)
        q8s = torch.zeros(nb, dtype=torch.float32, device=dev)
    table = torch.tensor([[s, 1 if f else 0] for s, f in w.shard.segments], dtype=torch.int64,
                         device=dev)
    st = zs.seg_table(table)
    hp = zs.hparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1.0)
    stream = torch.cuda.current_stream()

    # Twin ceilings: the step's traffic without its arithmetic, on these very
    # buffers and in the step's launch.  Writes only first (it overwrites the
    # state, which is initialised afterwards), reads only and the whole
    # traffic (which leaves the state as it was) once the inputs are in place.
    twin = None
    ceil = {}
    if not args.no_twin:
        twin = Twin(torch, var, dict(master=state if packed_var else master, m=m, v=v,
                                     param=param, q8=q8, q8s=q8s, grads=grads, qgrads=qgrads,
                                     qscales=qscales), k, n, plan)
        if twin.ok:
            ceil["write"] = twin.rate("write", stream)
    if packed_var:
        state.zero_()
        init = torch.empty(n, dtype=torch.float32, device=dev)
        synth.dev_master(w, init)
        _fill_packed_master(state, init, n, mv16)
        del init
    else:
        synth.dev_master(w, master)
        m.zero_()
        v.zero_()

    # the call is checked and marshalled once; each step passes t and the stream
    if var == "q8grad":
        call = zs.ShardStep(master, m, v, param, qgrads, n, st, hp, variant="q8grad",
                            qscales=qscales)
    elif var == "q8ag":
        call = zs.ShardStep(master, m, v, param, grads, n, st, hp, variant="q8ag",
                            param_q8=q8, param_q8_scale=q8s)
    elif var == "bf16mv":
        call = zs.ShardStep(master, m, v, param, grads, n, st, hp, variant="bf16mv")
    elif var == "packed":
        call = zs.ShardStep(state, None, None, param, grads, n, st, hp, variant="packed")
    elif var == "packed_q8ag":
        call = zs.ShardStep(state, None, None, param, grads, n, st, hp, variant=var,
                            param_q8=q8, param_q8_scale=q8s)
    elif var == "packed_q8grad":
        call = zs.ShardStep(state, None, None, param, qgrads, n, st, hp, variant=var,
                            qscales=qscales)
    elif var == "packed_bf16mv":
        call = zs.ShardStep(state, None, None, param, grads, n, st, hp, variant=var)
    elif var == "packed_bf16mv_sr":
        call = zs.ShardStep(state, None, None, param, grads, n, st, hp, variant=var,
                            seed=sr_seed(w))
    elif var == "bf16mv_sr":
        call = zs.ShardStep(master, m, v, param, grads, n, st, hp, variant=var, seed=sr_seed(w))
    else:
        call = zs.ShardStep(master, m, v, param, grads, n, st, hp, cfg=cfg)

    def step(t, on=None):
        call(t, stream if on is None else on)

    def fill(t):
        if q8grad_var:
            synth.dev_qgrads(w, t, qgrads, qscales)
        else:
            synth.dev_grads(w, t, grads)

    # pre-warm of the moments where the workload asks for it (fresh partials per step)
    for t in range(1, w.prewarm_steps + 1):
        fill(t)
        step(t)
    # the partials of the first measured step stay resident for every timed step
    fill(w.t0)
    torch.cuda.synchronize()
    if twin is not None and twin.ok:
        ceil["read"] = twin.rate("read", stream)
        ceil["step"] = twin.rate("step", stream)
        log("twin of the step's traffic: whole %.1f GB/s, reads %.1f GB/s, writes %.1f GB/s"
            % (ceil["step"], ceil["read"], ceil["write"]))
        # the same traffic in other launch shapes (chunk order x occupancy cap):
        # the best of them is what this machine delivers for it
        best = (ceil["step"], key)
        for order, cap in TWIN_SHAPES:
            alt = dict(plan, block_order=order, groups_per_cu=cap)
            if launch_key(alt) == key:
                continue
            other = Twin(torch, var, twin.bufs, k, n, alt)
            if other.ok:
                r = other.rate("step", stream)
                if r > best[0]:
                    best = (r, launch_key(alt))
        ceil["best"], ceil["best_launch"] = best
        log("best twin over launch shapes: %.1f GB/s (%s)" % best)

    # the windows the cpu_baseline leg replays with the oracle: their inputs now
    par = None
    if args.cpu_seconds > 0:
        wins = parity_windows(w, n)
        before = snapshot_packed(state, wins, mv16) if packed_var else \
            snapshot({"master": master, "m": m, "v": v}, wins)
        if q8grad_var:
            qg = [[q[a:b].cpu().numpy().copy() for a, b in wins] for q in qgrads]
            qs = [[block_slice(s, a, b).cpu().numpy().copy() for a, b in wins] for s in qscales]
            par = dict(qgrads=qg, qscales=qs)
        else:
            par = dict(grads=[[g[a:b].cpu().numpy().copy() for a, b in wins] for g in grads])
        par.update(windows=wins, before=before)

    # the same step on the same state packed per 256-element block, timed after
    # the default step from the state as it stands now (same t, same partials)
    pstate, packed_skip = None, None
    if var in PACKED_FORM and cfg is None and not args.graph and not args.no_packed:
        torch.cuda.empty_cache()
        floats = packed_state_floats(var, n)
        need = 4 * floats + (1 << 30)
        if torch.cuda.mem_get_info()[0] >= need:
            pstate = torch.empty(floats, dtype=torch.float32, device=dev)
            pack = zs.zs_pack_state_bf16mv if mv16 else zs.zs_pack_state
            pack(master, m, v, pstate, n, stream)
        else:
            packed_skip = "needs %.1f GB more device memory" % (need / 1e9)

    t = w.t0
    for _ in range(args.warmup):
        step(t)
        t += 1
    torch.cuda.synchronize()

    if args.graph:
        # the K timed steps (each with its own t) recorded once into a HIP graph,
        # then launched as one: no host launch cost between the kernels
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            for i in range(args.steps):
                step(t + i, cap)
        t += args.steps
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_begin = time.perf_counter()
        g0.record(stream)
        graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_begin
        kernel_ms = [g0.elapsed_time(g1) / args.steps] * args.steps
        del graph
    else:
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t_begin = time.perf_counter()
        for i in range(args.steps):
            starts[i].record(stream)
            step(t)
            ends[i].record(stream)
            t += 1
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_begin
        kernel_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_ms = sum(kernel_ms) / len(kernel_ms)
    log("kernel ms per launch: avg %.4f min %.4f max %.4f" % (avg_ms, min(kernel_ms),
                                                              max(kernel_ms)))
    if par is not None:
        if packed_var:
            after = snapshot_packed(state, wins, mv16)
            after.update(snapshot({"param": param, "q8": q8}, wins))
        else:
            after = snapshot({"master": master, "m": m, "v": v, "param": param, "q8": q8}, wins)
        if q8ag_var:
            after["q8s"] = [block_slice(q8s, a, b).cpu().numpy().copy() for a, b in wins]
        par.update(after=after, ts=list(range(w.t0, t)))

    packed = None
    if pstate is not None:
        packed = packed_leg(torch, w, var, pstate,
                            dict(master=master, m=m, v=v, param=param, grads=grads, qgrads=qgrads,
                                 qscales=qscales, q8=q8, q8s=q8s),
                            st, hp, stream, args, bytes_per_step)
        log("packed state: %.1f GB/s per launch, %s of its twin, bitwise equal to the "
            "separate-array step: %s" % (packed["achieved"], packed.get("pct_of_twin"),
                                         packed["bitwise_equal_to_separate_arrays"]))
    elif packed_skip:
        packed = {"skipped": packed_skip}

    value = bytes_per_step * args.steps / elapsed / 1e9
    achieved = bytes_per_step / (avg_ms * 1e-3) / 1e9
    traffic_key = args.config if var == "base" else "%s/%s" % (args.config, var)
    traffic = measured_traffic(traffic_key, key)

    del master, m, v, param, grads, qgrads, qscales, q8, q8s, twin, pstate
    torch.cuda.empty_cache()

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, args.cpu_seconds, arith, bpe, par)
        log("cpu oracle: %.3f GB/s (%s)" % (cpu["value"], cpu["sample"]))
        log("parity of the timed run: %s" % json.dumps(cpu["parity"]))

    ceilings = None
    if ceil:
        rb, wb = twin_bytes(var, k, n)
        ceilings = {
            "twin_step_gbps": round(ceil["step"], 1),
            "twin_read_gbps": round(ceil["read"], 1),
            "twin_write_gbps": round(ceil["write"], 1),
            # reads and writes each at their own ceiling, one after the other
            "serial_read_write_gbps": round((rb + wb) / (rb / ceil["read"] +
                                                         wb / ceil["write"]), 1),
            "pct_of_twin": round(100.0 * achieved / ceil["step"], 2),
            "twin_best_gbps": round(ceil["best"], 1),
            "twin_best_launch": ceil["best_launch"],
            "pct_of_twin_best": round(100.0 * achieved / ceil["best"], 2),
            "kind": "the step's own streams, buffers and launch with no arithmetic "
                    "(libzs_ceiling.so zs_ceiling_twin): whole traffic (state written back "
                    "unchanged), reads only, writes only; twin_best: the whole traffic in the "
                    "best of the launch shapes tried (chunk order x occupancy cap); HIP events, "
                    "same run",
        }
    out = {
        "metric": "achieved HBM GB/s (% of peak) and params/s for fused ZeRO-shard AdamW step",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage": {"base": "f32 master/m/v, bf16 partials and param",
                    "q8ag": "f32 master/m/v, bf16 partials and param, int8 param copy",
                    "q8grad": "f32 master/m/v, int8 partials, bf16 param",
                    "bf16mv": "f32 master, bf16 m/v, partials and param",
                    "packed": "f32 master/m/v packed per 256-element block, bf16 partials and "
                              "param",
                    "packed_q8ag": "f32 master/m/v packed per 256-element block, bf16 partials "
                                   "and param, int8 param copy",
                    "packed_q8grad": "f32 master/m/v packed per 256-element block, int8 "
                                     "partials, bf16 param",
                    "packed_bf16mv": "f32 master and bf16 m/v packed per 256-element block, "
                                     "bf16 partials and param",
                    "bf16mv_sr": "f32 master, bf16 m/v (stochastically rounded), partials and "
                                 "param",
                    "packed_bf16mv_sr": "f32 master and bf16 m/v (stochastically rounded) "
                                        "packed per 256-element block, bf16 partials and "
                                        "param"}[var],
        "data": "synthetic (seeded SplitMix64 / Irwin-Hall draws; partials of the first "
                "measured step kept resident across timed steps)",
        "config": {
            "workload": w.name,
            "entry_point": "zs_shard_step" if var == "base" else "zs_shard_step_" + var,
            "shard_params": n,
            "k_partials": k,
            "segments": len(w.shard.segments),
            "bytes_per_param": round(bpe, 4),
            "bytes_per_step": bytes_per_step,
            "first_step_t": w.t0 + args.warmup,
            "launch": key,
        },
        "params_per_s": round(n * args.steps / elapsed, 1),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "copy_ceiling_gbps": round(copies["stream"], 1) if copies else None,
        "copy_ceiling_kind": "streaming copy with the step's access pattern "
                             "(libzs_ceiling.so) of --copy-gb bytes, read + write, same run",
        "pct_of_copy_ceiling": round(100.0 * achieved / copies["stream"], 2) if copies else None,
        "torch_copy_gbps": round(copies["torch"], 1) if copies else None,
        "ceilings": ceilings,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            # the counted bytes (rocprofv3 counters of this kernel source and
            # launch) over this run's average launch time
            "traffic_gbps": round(traffic / (avg_ms * 1e-3) / 1e9, 2) if traffic else None,
            "kernel": "shard_step_kernel<K=%d,%s>" % (k, var),
            "avg_launch_ms": round(avg_ms, 4),
            "timing": "one HIP graph of the timed steps, average per step" if args.graph
                      else "HIP events around each launch on the launch stream",
        },
        "kernel_ms": {"median": round(statistics.median(kernel_ms), 4),
                      "min": round(min(kernel_ms), 4), "max": round(max(kernel_ms), 4)},
        "parity": cpu["parity"] if cpu else None,
        "cpu_baseline": cpu,
        "speedup_vs_cpu_oracle": None if not cpu else {
            "single_thread": round(value / cpu["value"], 1),
            "threaded": round(value / cpu["threaded"]["value"], 1)},
    }
    if packed is not None:
        out["packed_state"] = packed
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
