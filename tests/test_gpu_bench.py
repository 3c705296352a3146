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
                                   ["--block-order", "2", "--groups-per-cu", "4"]],
                         ids=["base", "graph", "q8ag", "q8grad", "bf16mv", "cfg"])
def test_bench_line(extra):
    out = _bench(*extra)
    assert out["n_gpus"] == 1 and out["steps"] == 5 and out["warmup"] == 1
    assert out["value"] > 0 and out["ms_per_step"] > 0 and out["higher_is_better"] is True
    assert out["config"]["workload"].startswith("tiny")
    assert out["dtype"] == "f32" and "bf16" in out["storage"]
    r = out["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert out["kernel_ms"]["min"] <= out["kernel_ms"]["median"] <= out["kernel_ms"]["max"]
    cpu = out["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] == 1 and cpu["value"] > 0
    assert out["speedup_vs_cpu_oracle"]["single_thread"] > 1
    variant = extra[1] if extra[:1] == ["--variant"] else "base"
    want = "zs_shard_step" if variant == "base" else "zs_shard_step_" + variant
    assert out["config"]["entry_point"] == want
