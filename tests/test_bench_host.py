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
    assert "first %d elements" % min(w.n, 1 << 24) in r["sample"]
    assert r["threaded"]["cores"] >= 1 and r["threaded"]["value"] > 0


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
            bench._threaded_oracle(*a, None, segs, hp, 4, variant, 1.0, qg, qs, seconds=0.0)
            assert oracle.shard_step_q8grad(*b, qg, qs, segs, hp, 4) == 0
        else:
            bench._threaded_oracle(*a, grads, segs, hp, 4, variant, 1.0, seconds=0.0)
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
