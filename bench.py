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


def cpu_baseline(w, seconds: float, variant: str, bytes_per_elem: float):
    """Time the CPU oracle (single thread, as it stands) on a bounded window
    of the same workload: the first min(n, 2^24) elements of the shard, with
    the arithmetic of the entry point being measured.  The "threaded" entry
    times the same oracle over T contiguous ranges of that window."""
    import numpy as np

    import oracle
    import synth

    n = min(w.n, 1 << 24)
    master = synth.host_master(w, 0, n)
    mv_dtype = np.uint16 if variant == "bf16mv" else np.float32
    m = np.zeros(n, mv_dtype)
    v = np.zeros(n, mv_dtype)
    p = np.zeros(n, np.uint16)
    if variant == "q8grad":
        qgrads, qscales = synth.host_qgrads(w, w.t0, 0, n)
    else:
        grads = synth.host_grads(w, w.t0, 0, n)
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
                                segs, hp, t, variant, bytes_per_elem,
                                qgrads if variant == "q8grad" else None,
                                qscales if variant == "q8grad" else None)
    return {
        "value": round(n * steps * bytes_per_elem / elapsed / 1e9, 4),
        "unit": "GB/s",
        "params_per_s": round(n * steps / elapsed, 1),
        "cores": 1,
        "threaded": threaded,
        "kind": "oracle",
        "sample": "first %d elements of the %s shard (k=%d, %d segments in the window), "
                  "%d timed oracle steps after one untimed (%s arithmetic), single-threaded C, %.1f s" % (
                      n, w.name.split(":")[0].split(" (")[0], w.k, len(segs), steps, variant,
                      elapsed),
    }


def _threaded_oracle(master, m, v, p, grads, segs, hp, t, variant, bytes_per_elem,
                     qgrads=None, qscales=None, seconds=3.0):
    """The same oracle driven from T threads over T contiguous ranges of the
    window (the step is elementwise, so the split does not change a bit);
    T = the CPUs this process may use, at most 16."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import synth

    n = master.shape[0]
    threads = max(1, min(len(os.sched_getaffinity(0)), 16))
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
            "steps": steps}


def _ceiling_lib():
    import ctypes
    path = os.path.join(ROOT, "sharded_mixed_precision_shard_amd", "libzs_ceiling.so")
    if not os.path.exists(path):
        raise ImportError("libzs_ceiling.so is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.zs_ceiling_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_void_p]
    lib.zs_ceiling_copy.restype = ctypes.c_int
    return lib


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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 10; 200 for the tiny and GPT-2 shards, whose "
                         "steps take microseconds)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="70b")
    ap.add_argument("--variant", default="base",
                    choices=("base", "q8ag", "q8grad", "bf16mv", "offload"),
                    help="entry point: zs_shard_step (base), zs_shard_step_q8ag, "
                         "zs_shard_step_q8grad, zs_shard_step_bf16mv, or the host "
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
    bytes_per_step = zs.algorithmic_bytes(args.variant, k, n)
    bpe = bytes_per_step / n
    if args.variant == "base":
        assert zs.zs_algorithmic_bytes(k, n) == bytes_per_step
    log("workload: %s  n=%d k=%d segments=%d bytes/step=%.3f GB" % (
        w.name, n, k, len(w.shard.segments), bytes_per_step / 1e9))

    copies = {}
    if args.copy_gb > 0:
        copies = copy_ceiling(torch, int(args.copy_gb * 1e9) // 4096 * 4096)
        log("copies of %.1f GB: streaming %.1f GB/s, torch copy_ %.1f GB/s" % (
            args.copy_gb, copies["stream"], copies["torch"]))

    dev = torch.device("cuda:0")
    var = args.variant
    nb = -(-n // zs.ZS_Q8_BLOCK)
    mv_dtype = torch.int16 if var == "bf16mv" else torch.float32
    master = torch.empty(n, dtype=torch.float32, device=dev)
    m = torch.zeros(n, dtype=mv_dtype, device=dev)
    v = torch.zeros(n, dtype=mv_dtype, device=dev)
    param = torch.zeros(n, dtype=torch.int16, device=dev)
    grads = qgrads = qscales = q8 = q8s = None
    if var == "q8grad":
        qgrads = [torch.empty(n, dtype=torch.int8, device=dev) for _ in range(k)]
        qscales = [torch.empty(nb, dtype=torch.float32, device=dev) for _ in range(k)]
    else:
        grads = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(k)]
    if var == "q8ag":
        q8 = torch.zeros(n, dtype=torch.int8, device=dev)
        q8s = torch.zeros(nb, dtype=torch.float32, device=dev)
    table = torch.tensor([[s, 1 if f else 0] for s, f in w.shard.segments], dtype=torch.int64,
                         device=dev)
    st = zs.seg_table(table)
    hp = zs.hparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1.0)
    stream = torch.cuda.current_stream()
    synth.dev_master(w, master)

    # the call is checked and marshalled once; each step passes t and the stream
    if var == "q8grad":
        call = zs.ShardStep(master, m, v, param, qgrads, n, st, hp, variant="q8grad",
                            qscales=qscales)
    elif var == "q8ag":
        call = zs.ShardStep(master, m, v, param, grads, n, st, hp, variant="q8ag",
                            param_q8=q8, param_q8_scale=q8s)
    elif var == "bf16mv":
        call = zs.ShardStep(master, m, v, param, grads, n, st, hp, variant="bf16mv")
    else:
        cfg = dict(chunk_tiles=args.chunk_tiles, nontemporal=args.nontemporal,
                   groups_per_cu=args.groups_per_cu, block_order=args.block_order)
        call = zs.ShardStep(master, m, v, param, grads, n, st, hp,
                            cfg=cfg if any(cfg.values()) else None)

    def step(t, on=None):
        call(t, stream if on is None else on)

    def fill(t):
        if var == "q8grad":
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

    value = bytes_per_step * args.steps / elapsed / 1e9
    achieved = bytes_per_step / (avg_ms * 1e-3) / 1e9
    launch_key = "chunk_tiles=%d,nontemporal=%d" % (args.chunk_tiles, args.nontemporal)
    if args.groups_per_cu:
        launch_key += ",groups_per_cu=%d" % args.groups_per_cu
    if args.block_order:
        launch_key += ",block_order=%d" % args.block_order
    traffic_key = args.config if var == "base" else "%s/%s" % (args.config, var)
    traffic = measured_traffic(traffic_key, launch_key)

    del master, m, v, param, grads, qgrads, qscales, q8, q8s
    torch.cuda.empty_cache()

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, args.cpu_seconds, var, bpe)
        log("cpu oracle: %.3f GB/s (%s)" % (cpu["value"], cpu["sample"]))

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
                    "bf16mv": "f32 master, bf16 m/v, partials and param"}[var],
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
        },
        "params_per_s": round(n * args.steps / elapsed, 1),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "copy_ceiling_gbps": round(copies["stream"], 1) if copies else None,
        "copy_ceiling_kind": "streaming copy with the step's access pattern "
                             "(libzs_ceiling.so) of --copy-gb bytes, read + write, same run",
        "pct_of_copy_ceiling": round(100.0 * achieved / copies["stream"], 2) if copies else None,
        "torch_copy_gbps": round(copies["torch"], 1) if copies else None,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": "shard_step_kernel<K=%d,%s>" % (k, var),
            "avg_launch_ms": round(avg_ms, 4),
            "timing": "one HIP graph of the timed steps, average per step" if args.graph
                      else "HIP events around each launch on the launch stream",
        },
        "kernel_ms": {"median": round(statistics.median(kernel_ms), 4),
                      "min": round(min(kernel_ms), 4), "max": round(max(kernel_ms), 4)},
        "cpu_baseline": cpu,
        "speedup_vs_cpu_oracle": None if not cpu else {
            "single_thread": round(value / cpu["value"], 1),
            "threaded": round(value / cpu["threaded"]["value"], 1)},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
