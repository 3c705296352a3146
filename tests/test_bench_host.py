"""bench.py's host-side pieces (CPU only): the one-GPU refusal, the JSON
contract of a whole run of the host (ZeRO-Offload) step, the oracle timing
leg, and that the threaded oracle driver's range split changes no bit."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=timeout, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one gpu" in (r.stderr + r.stdout).lower()


def test_offload_run_prints_one_json_line():
    r = _run_bench("--variant", "offload", "--config", "tiny", "--steps", "3", "--warmup", "1",
                   "--cpu-seconds", "0.5")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    out = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in out, key
    assert out["steps"] == 3 and out["warmup"] == 1 and out["value"] > 0
    assert out["dtype"] == "f32"
    assert out["config"]["workload"].startswith("tiny")
    assert 0 < out["roofline"]["frac"] and out["roofline"]["unit"] == "GB/s"
    cpu = out["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] == 1 and cpu["value"] > 0
    assert cpu["threaded"]["cores"] >= 1
    sp = out["speedup_vs_cpu_oracle"]
    assert abs(sp["single_thread"] - out["value"] / cpu["value"]) <= 0.05 + 1e-3 * sp["single_thread"]


def test_cpu_baseline_fields():
    w = synth.workload("tiny")
    r = bench.cpu_baseline(w, 0.2, "base", 26 + 2 * w.k)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["cores"] == 1
    assert r["value"] > 0 and r["params_per_s"] > 0
    assert "first %d elements" % min(w.n, 1 << 27) in r["sample"]
    assert r["threaded"]["cores"] >= 1 and r["threaded"]["value"] > 0
    assert r["threaded"]["cores"] <= bench.HOST_THREAD_CAP
    assert r["host"]["online_cpus"] >= r["host"]["usable_cpus"] >= 1
    assert r["parity"] is None


def test_threaded_split_is_bitwise_identical():
    n = 300_000 + 77
    rng = np.random.default_rng(11)
    master = rng.normal(0, 0.02, n).astype(np.float32)
    grads = [(rng.normal(0, 1e-2, n).astype(np.float32).view(np.uint32) >> 16)
             .astype(np.uint16) for _ in range(3)]
    segs = [(0, True), (5, False), (70_000, True), (70_001, False), (250_000, True)]
    hp = oracle.hparams(1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0)
    for variant in ("base", "q8ag", "bf16mv", "q8grad"):
        mv = np.uint16 if variant == "bf16mv" else np.float32
        a = [master.copy(), np.zeros(n, mv), np.zeros(n, mv), np.zeros(n, np.uint16)]
        b = [x.copy() for x in a]
        if variant == "q8grad":
            qg = [rng.integers(-127, 128, n).astype(np.int8) for _ in range(3)]
            qs = [rng.uniform(1e-5, 1e-4, -(-n // 256)).astype(np.float32) for _ in range(3)]
            bench._threaded_oracle(*a, None, segs, hp, 4, variant, 1.0, 4, qg, qs, seconds=0.0)
            assert oracle.shard_step_q8grad(*b, qg, qs, segs, hp, 4) == 0
        else:
            bench._threaded_oracle(*a, grads, segs, hp, 4, variant, 1.0, 4, seconds=0.0)
            step = oracle.shard_step_bf16mv if variant == "bf16mv" else oracle.shard_step
            assert step(*b, grads, segs, hp, 4) == 0
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), variant


def test_kernel_hash_ignores_comments_not_code():
    src = "int f(int x) { // add one\n  return x + 1; /* done */ }\n"
    same = "// header\nint f(int x) {\n\n  return x + 1;   }\n"
    other = "int f(int x) { return x + 2; }"
    assert bench._code_only(src) == bench._code_only(same)
    assert bench._code_only(src) != bench._code_only(other)
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        entries = json.load(f)
    # a measurement is reported only for the kernel code it was taken on
    for key, e in entries.items():
        got = bench.measured_traffic(key, e["launch"])
        assert got == (e["bytes_per_launch"] if e["kernel_sha"] == h else None), key
        assert bench.measured_traffic(key, e["launch"] + ",other") is None


def test_ceiling_library_loads_and_rejects_bad_arguments():
    """Loads on the CPU; the argument checks return before any device call."""
    lib = bench._ceiling_lib()
    assert lib.zs_ceiling_copy(16, 4096, 100, None) == -1   # not a multiple of 16
    assert lib.zs_ceiling_copy(8, 4096, 64, None) == -1     # misaligned
    assert lib.zs_ceiling_copy(0, 4096, 64, None) == -1     # null source
    assert lib.zs_ceiling_copy(4096, 4112, 64, None) == -1  # overlap
    assert lib.zs_ceiling_copy(0, 0, 0, None) == 0          # nothing to do


def test_launch_key_follows_the_resolved_launch():
    """The launch key comes from zs_launch_plan, so the library's defaults
    (chunk order threshold, occupancy cap and its range) are part of it: a
    measurement keyed to one plan is not reported for another."""
    import sharded_mixed_precision_shard_amd as zs
    p70 = zs.zs_launch_plan(2, synth.workload("70b").n)
    p175 = zs.zs_launch_plan(2, synth.workload("175b").n)
    pg2 = zs.zs_launch_plan(8, synth.workload("gpt2-small").n)
    assert (p70["block_order"], p70["groups_per_cu"]) == (2, 5)    # from 2^26 on: cap 5
    assert (p175["block_order"], p175["groups_per_cu"]) == (2, 5)
    assert (pg2["block_order"], pg2["groups_per_cu"]) == (1, 0)    # below the XCD threshold
    assert zs.zs_launch_plan(2, synth.workload("175b").n, "bf16mv")["groups_per_cu"] == 0
    assert p70["window_quads"] == 1 and p175["window_quads"] == 1
    # above 2^32 elements every entry point keeps the cap; bf16 moments take the
    # wide kernel (two sub-windows per wave, 2048-element tiles) under it, for k <= 4,
    # and otherwise run uncapped as below 2^32
    n70 = synth.workload("70b").n
    q8 = zs.zs_launch_plan(2, n70, "q8ag")
    assert (q8["groups_per_cu"], q8["window_quads"], q8["chunk_elements"]) == (5, 1, 1024)
    mv = zs.zs_launch_plan(2, n70, "bf16mv")
    assert (mv["groups_per_cu"], mv["window_quads"], mv["chunk_elements"]) == (5, 2, 2048)
    assert mv["workgroups"] == -(-n70 // 2048)
    mv8 = zs.zs_launch_plan(8, n70, "bf16mv")
    assert (mv8["groups_per_cu"], mv8["window_quads"]) == (0, 1)
    assert zs.zs_launch_plan(2, (1 << 32) - 1, "bf16mv")["window_quads"] == 1
    assert zs.zs_launch_plan(2, 1 << 32, "bf16mv")["window_quads"] == 2
    assert zs.zs_launch_plan(2, n70, "q8grad")["groups_per_cu"] == 5
    assert zs.zs_launch_plan(2, n70, "packed") == p70  # the packed step launches as the step
    assert zs.zs_launch_plan(2, n70, "packed_q8ag") == q8
    assert zs.zs_launch_plan(2, n70, "packed_q8grad") == zs.zs_launch_plan(2, n70, "q8grad")
    assert zs.zs_launch_plan(2, n70, "packed_bf16mv") == mv
    assert zs.zs_launch_plan(2, n70, "bf16mv_sr") == mv
    assert zs.zs_launch_plan(2, n70, "packed_bf16mv_sr") == mv
    for nn in ((1 << 32) - 1, 1 << 32, 10 ** 8, 5000):
        for kk in (2, 8):
            for form in ("packed_bf16mv", "bf16mv_sr", "packed_bf16mv_sr"):
                assert zs.zs_launch_plan(kk, nn, form) == zs.zs_launch_plan(kk, nn, "bf16mv")
    assert zs.zs_launch_plan(2, (1 << 32) - 1, "bf16mv")["groups_per_cu"] == 0
    assert zs.zs_launch_plan(2, 1 << 32, "bf16mv")["groups_per_cu"] == 5
    assert bench.launch_key(mv).endswith(",quads=2") and "quads" not in bench.launch_key(p70)
    assert zs.zs_launch_plan(2, 10 ** 8, cfg=dict(nontemporal=2))["nontemporal"] == 0
    assert zs.zs_launch_plan(2, 0)["workgroups"] == 0
    assert zs.zs_launch_plan(2, (1 << 32) - 1)["groups_per_cu"] == 5
    assert zs.zs_launch_plan(2, (1 << 26) - 1)["groups_per_cu"] == 0
    # a default that moved (here: the cap of the 175B launch) changes the key
    moved = dict(p175, groups_per_cu=6)
    assert bench.launch_key(moved) != bench.launch_key(p175)
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        entries = json.load(f)
    for key, e in entries.items():
        if e["launch"] == bench.launch_key(p175):
            assert bench.measured_traffic(key, bench.launch_key(moved)) is None
    with __import__("pytest").raises(zs.ZsError):
        zs.zs_launch_plan(2, 100, "q8ag", cfg=dict(chunk_tiles=2))  # cfg is base-only
    with __import__("pytest").raises(zs.ZsError):
        zs.zs_launch_plan(17, 100)


def test_twin_rejects_bad_arguments_before_any_device_call():
    import ctypes
    lib = bench._ceiling_lib()
    g = (ctypes.c_void_p * 2)(4096, 8192)
    P = ctypes.c_void_p

    def call(mode=0, layout=0, k=2, n=4096, chunk=1024, order=2, cap=0, grads=g, quads=1):
        return lib.zs_ceiling_twin(mode, layout, P(4096), P(4096), P(4096), P(4096), None,
                                   None, ctypes.cast(grads, P), None, k, n, chunk, order, cap,
                                   quads, None)
    assert call(mode=3) == -1
    assert call(layout=3) == -1
    assert call(k=0) == -1 and call(k=17) == -1
    assert call(n=4097) == -1 and call(n=3072, chunk=2048) == -1
    assert call(chunk=512) == -1
    assert call(order=0) == -1 and call(cap=33) == -1
    assert call(layout=1) == -1                 # no int8 copy given
    assert call(layout=2) == -1                 # no scales given
    assert call(grads=(ctypes.c_void_p * 2)(4096, 0)) == -1
    assert call(quads=3) == -1 and call(quads=0) == -1
    assert call(quads=2) == -1                  # two sub-windows only with layout 4
    assert call(layout=4, quads=2, chunk=1024) == -1  # chunk below the wide tile
    assert call(n=0) == 0                       # nothing to do
    assert call(n=0, layout=4, quads=2, chunk=2048) == 0
    # the packed layout: m and v live in the state, so they may be null there only
    def call_mv(layout, m, v, n=0):
        return lib.zs_ceiling_twin(0, layout, P(4096), m, v, P(4096), None, None,
                                   ctypes.cast(g, P), None, 2, n, 1024, 2, 0, 1, None)
    assert call_mv(8, None, None) == 0 and call(layout=8, n=0) == 0
    assert call_mv(0, None, None) == -1 and call_mv(4, P(4096), None) == -1
    assert call(layout=8, quads=2, chunk=2048) == -1  # one sub-window per wave only
    assert call(layout=13) == -1 and call(layout=16) == -1
    # the packed bf16-moment layout (12) takes one or two sub-windows per wave
    assert call_mv(12, None, None) == 0 and call(layout=12, quads=2, chunk=2048, n=0) == 0
    assert call(layout=12, quads=2, chunk=1024) == -1


def test_parity_windows_cover_ends_and_boundaries():
    w = synth.workload("70b")
    wins = bench.parity_windows(w, w.n)
    assert wins[0][0] == 0 and wins[-1][1] == w.n
    assert len(wins) >= 8
    for a, b in wins:
        assert a % 256 == 0 and 0 < b - a <= bench.PARITY_WINDOW
    assert all(x[1] <= y[0] for x, y in zip(wins, wins[1:]))
    starts = [s for s, _ in w.shard.segments[1:]]
    assert sum(any(a < s < b for s in starts) for a, b in wins) >= 4
    t = synth.workload("tiny")
    assert bench.parity_windows(t, 1000) == [(0, 1000)]


def _fake_run(variant, steps, plant=None):
    """A run's windows whose 'GPU' results are the oracle's own, with an
    optional planted change; exercises the comparison, not the kernel."""
    w = synth.workload("tiny")
    wins = [(0, 4096), (8192, 8192 + 1000)]
    before, grads = {"master": [], "m": [], "v": []}, [[] for _ in range(w.k)]
    after = {"master": [], "m": [], "v": [], "param": []}
    hp = oracle.hparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, 1.0)
    mvt = np.uint16 if variant == "bf16mv" else np.float32
    for a, b in wins:
        mst = synth.host_master(w, a, b)
        gs = synth.host_grads(w, w.t0, a, b)
        before["master"].append(mst.copy())
        before["m"].append(np.zeros(b - a, mvt))
        before["v"].append(np.zeros(b - a, mvt))
        for j in range(w.k):
            grads[j].append(gs[j].view(np.int16))
        m, v, p = np.zeros(b - a, mvt), np.zeros(b - a, mvt), np.zeros(b - a, np.uint16)
        segs = synth.clip_segments(w.shard.segments, a, b)
        for t in range(w.t0, w.t0 + steps):
            fn = oracle.shard_step_bf16mv if variant == "bf16mv" else oracle.shard_step
            assert fn(mst, m, v, p, gs, segs, hp, t) == 0
        after["master"].append(mst)
        after["m"].append(m)
        after["v"].append(v)
        after["param"].append(p.view(np.int16))
    if plant:
        plant(after)
    return w, dict(windows=wins, before=before, after=after, grads=grads,
                   ts=list(range(w.t0, w.t0 + steps)))


def test_parity_replay_reports_equality_and_planted_differences():
    for variant in ("base", "bf16mv"):
        w, par = _fake_run(variant, 3)
        r = bench._parity_replay(w, variant, par)
        assert r["bitwise_equal"] and r["within_tolerance"], r
        assert r["max_param_bf16_ulp"] == 0 and r["steps_replayed"] == 3
    # one master element (|x| < 1, so the bound is 1e-6 absolute) off by 2e-6
    def bump(after):
        after["master"][1][7] += np.float32(2e-6)
    w, par = _fake_run("base", 2, bump)
    r = bench._parity_replay(w, "base", par)
    assert not r["bitwise_equal"] and not r["within_tolerance"]
    assert 1e-6 < r["max_rel_err"]["master"] < 1e-5
    # a parameter one bf16 ulp away: not bitwise, still within tolerance
    def ulp(after):
        after["param"][0][3] += 1
    w, par = _fake_run("base", 2, ulp)
    r = bench._parity_replay(w, "base", par)
    assert not r["bitwise_equal"] and r["within_tolerance"]
    assert r["max_param_bf16_ulp"] == 1


def test_every_entry_point_is_benchable_and_its_bytes_agree():
    """Each entry point the binding names has a bench variant, a twin layout
    and a byte count, and the bench's stream bytes add up to the binding's
    algorithmic bytes; each packed form maps back to its separate form."""
    import sharded_mixed_precision_shard_amd as zs
    help_text = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                               capture_output=True, text=True, timeout=60, cwd=ROOT).stdout
    help_text = " ".join(help_text.split())
    for var in zs.ZS_VARIANT:
        assert var in bench.Twin.LAYOUT, var
        assert var in help_text, var
        for k, n in ((1, 1), (2, 1000), (8, 10 ** 6 + 3), (16, 257)):
            r, w = bench.twin_bytes(var, k, n)
            assert r + w == zs.algorithmic_bytes(var, k, n), (var, k, n)
    for sep, packed in bench.PACKED_FORM.items():
        assert sep in zs.ZS_VARIANT and packed in zs.ZS_VARIANT
        assert zs.algorithmic_bytes(sep, 2, 999) == zs.algorithmic_bytes(packed, 2, 999)
        assert bench.Twin.LAYOUT[packed] == bench.Twin.LAYOUT[sep] | 8


def test_committed_traffic_matches_the_current_kernels():
    """profiles/traffic.json holds counted bytes for the current kernel source
    and the default launch of the headline workload (so the bench line's
    roofline.traffic is not null), within 0.1 % of the algorithmic bytes."""
    import sharded_mixed_precision_shard_amd as zs
    w = synth.workload("70b")
    key = bench.launch_key(zs.zs_launch_plan(w.k, w.n))
    traffic = bench.measured_traffic("70b", key)
    assert traffic is not None, "re-take the rocprofv3 counters for kernel %s" % (
        bench.kernel_source_hash())
    alg = zs.algorithmic_bytes("base", w.k, w.n)
    assert abs(traffic / alg - 1) < 1e-3
