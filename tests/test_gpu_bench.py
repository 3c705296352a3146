"""bench.py end to end on the GPU, on the tiny shard: the one JSON line and
its contract for the ordinary step, the graph-timed run and each variant."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "tiny",
                        "--steps", "5", "--warmup", "1", "--cpu-seconds", "0.2",
                        "--copy-gb", "0.5", *args],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.mark.parametrize("extra", [[], ["--graph"], ["--variant", "q8ag"],
                                   ["--variant", "q8grad"], ["--variant", "bf16mv"],
                                   ["--variant", "packed"], ["--variant", "packed_q8ag"],
                                   ["--variant", "packed_q8grad"], ["--variant", "packed_bf16mv"],
                                   ["--variant", "bf16mv_sr"], ["--variant", "packed_bf16mv_sr"],
                                   ["--block-order", "2", "--groups-per-cu", "4"]],
                         ids=["base", "graph", "q8ag", "q8grad", "bf16mv", "packed", "packed_q8ag",
                              "packed_q8grad", "packed_bf16mv", "bf16mv_sr", "packed_bf16mv_sr",
                              "cfg"])
def test_bench_line(extra):
    out = _bench(*extra)
    assert out["n_gpus"] == 1 and out["steps"] == 5 and out["warmup"] == 1
    assert out["value"] > 0 and out["ms_per_step"] > 0 and out["higher_is_better"] is True
    assert out["config"]["workload"].startswith("tiny")
    assert out["dtype"] == "f32" and "bf16" in out["storage"]
    r = out["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    if r["traffic"] is None:
        assert r["traffic_gbps"] is None
    else:
        assert abs(r["traffic_gbps"] - r["traffic"] / (r["avg_launch_ms"] * 1e-3) / 1e9) < 1
    assert out["kernel_ms"]["min"] <= out["kernel_ms"]["median"] <= out["kernel_ms"]["max"]
    cpu = out["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] == 1 and cpu["value"] > 0
    assert out["speedup_vs_cpu_oracle"]["single_thread"] > 1
    assert out["copy_ceiling_gbps"] > 0 and out["torch_copy_gbps"] > 0
    assert out["pct_of_copy_ceiling"] > 0
    variant = extra[1] if extra[:1] == ["--variant"] else "base"
    want = "zs_shard_step" if variant == "base" else "zs_shard_step_" + variant
    assert out["config"]["entry_point"] == want
    c = out["ceilings"]
    assert c["twin_step_gbps"] > 0 and c["twin_read_gbps"] > 0 and c["twin_write_gbps"] > 0
    assert c["pct_of_twin"] > 0
    assert c["twin_best_gbps"] >= c["twin_step_gbps"] and c["pct_of_twin_best"] > 0
    par = out["parity"]
    assert par == cpu["parity"] and par["windows"] >= 1
    assert par["steps_replayed"] == 6  # one warm-up step and five timed ones
    assert par["within_tolerance"] and par["bitwise_equal"], par
    pk = out.get("packed_state")
    if extra in ([], ["--variant", "q8ag"], ["--variant", "q8grad"], ["--variant", "bf16mv"],
                 ["--variant", "bf16mv_sr"]):
        # the same steps on the packed state, beside the separate-array step
        pform = {"base": "packed", "q8ag": "packed_q8ag", "q8grad": "packed_q8grad",
                 "bf16mv": "packed_bf16mv", "bf16mv_sr": "packed_bf16mv_sr"}[variant]
        assert pk["entry_point"] == "zs_shard_step_" + pform and pk["achieved"] > 0
        assert pk["separate_arrays_entry_point"] == want
        assert pk["bitwise_equal_to_separate_arrays"] is True and pk["pct_of_twin"] > 0
    else:
        assert pk is None


def test_streaming_copy_of_the_ceiling_library():
    """The copy bench.py measures as its in-run ceiling copies exactly and
    refuses bad arguments without launching."""
    import torch
    sys.path.insert(0, ROOT)
    import bench
    lib = bench._ceiling_lib()
    torch.cuda.set_device(0)
    n = (1 << 22) + 4
    src = torch.randn(n, device="cuda")
    dst = torch.zeros(n, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert lib.zs_ceiling_copy(src.data_ptr(), dst.data_ptr(), 4 * n, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    assert lib.zs_ceiling_copy(src.data_ptr(), dst.data_ptr(), 4 * n - 4, s) == -1
    assert lib.zs_ceiling_copy(src.data_ptr() + 4, dst.data_ptr(), 16, s) == -1
    assert lib.zs_ceiling_copy(src.data_ptr(), src.data_ptr() + 16, 64, s) == -1
    assert lib.zs_ceiling_copy(src.data_ptr(), dst.data_ptr(), 0, s) == 0


@pytest.mark.parametrize("variant", ["base", "q8ag", "q8grad", "bf16mv", "bf16mv-wide",
                                     "packed", "packed_q8ag", "packed_q8grad", "packed_bf16mv",
                                     "packed_bf16mv-wide"])
def test_twin_moves_the_step_traffic_without_changing_the_state(variant):
    """The twin ceiling on a step's buffers: the whole-traffic mode writes the
    state back bit for bit, the read-only mode changes nothing, the
    write-only mode overwrites the covered elements with its pattern."""
    import torch
    sys.path.insert(0, ROOT)
    import bench
    import sharded_mixed_precision_shard_amd as zs
    torch.cuda.set_device(0)
    wide = variant.endswith("-wide")
    variant = variant[:-len("-wide")] if wide else variant
    k, n = 3, 1 << 16
    nb = n // 256
    g = torch.Generator(device="cuda").manual_seed(5)
    rnd = lambda dt: torch.randint(-30000, 30000, (n,), generator=g, device="cuda",  # noqa
                                   dtype=torch.int32).to(dt)
    mvt = torch.int16 if variant == "bf16mv" else torch.float32
    packed = variant.startswith("packed")
    mv16 = variant.endswith("bf16mv")
    floats = (zs.packed_bf16mv_floats(n) if mv16 else zs.packed_floats(n)) if packed else n
    bufs = dict(master=torch.randn(floats, device="cuda", generator=g),
                m=None if packed else rnd(mvt), v=None if packed else rnd(mvt),
                param=torch.zeros(n, dtype=torch.int16, device="cuda"),
                q8=torch.zeros(n, dtype=torch.int8, device="cuda")
                if variant in ("q8ag", "packed_q8ag") else None,
                q8s=torch.zeros(nb, device="cuda") if variant in ("q8ag", "packed_q8ag") else None)
    if variant in ("q8grad", "packed_q8grad"):
        bufs["qgrads"] = [rnd(torch.int8) for _ in range(k)]
        bufs["qscales"] = [torch.rand(nb, device="cuda", generator=g) for _ in range(k)]
        bufs["grads"] = None
    else:
        bufs["grads"] = [rnd(torch.int16) for _ in range(k)]
    plan = zs.zs_launch_plan(k, n, variant)
    if wide:  # the launch shape of the largest shards, on a small buffer
        plan = dict(plan, chunk_elements=2048, workgroups=n // 2048, window_quads=2,
                    groups_per_cu=5)
    twin = bench.Twin(torch, variant, bufs, k, n, plan)
    assert twin.ok and twin.n == n
    keep = {x: bufs[x].clone() for x in ("master", "m", "v") if bufs[x] is not None}
    s = torch.cuda.current_stream()
    for mode in ("step", "read"):
        twin.launch(mode, s)
        torch.cuda.synchronize()
        for x in keep:
            assert torch.equal(bufs[x].view(torch.int16), keep[x].view(torch.int16)), (mode, x)
    assert twin.rate("step", s, reps=2) > 0
    twin.launch("write", s)
    torch.cuda.synchronize()
    pattern = torch.tensor([1.0, 2.0, 3.0, 4.0], device="cuda").repeat(bufs["master"].numel() // 4)
    if packed and mv16:
        # per 2 KB block: 256 fp32 master values, then bf16 m and v slots of 1.0 (0x3f80)
        blk = pattern.view(-1, 512).clone()
        blk[:, 256:] = torch.tensor([0x3f803f80], dtype=torch.int32, device="cuda").view(
            torch.float32)
        pattern = blk.view(-1)
    assert torch.equal(bufs["master"].view(torch.int32), pattern.view(torch.int32))


def test_launch_sweep_prints_every_configuration():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "tiny",
                        "--sweep", "--rounds", "2", "--steps", "3"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    out = json.loads(lines[0])
    sys.path.insert(0, ROOT)
    import bench
    assert list(out["sweep"]) == [name for name, _ in bench.SWEEP_CFGS]
    for name, e in out["sweep"].items():
        assert len(e["kernel_gbps"]) == 2 and len(e["twin_gbps"]) == 2, name
        assert e["kernel_median"] > 0 and e["twin_median"] > 0
    assert out["sweep"]["xcd,cap5"]["launch"].endswith("order=2,cap=5,nt=1")
    assert out["sweep"]["linear"]["launch"].endswith("order=1,cap=32,nt=1")
