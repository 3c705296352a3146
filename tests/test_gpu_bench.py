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
    assert out["copy_ceiling_gbps"] > 0 and out["torch_copy_gbps"] > 0
    assert out["pct_of_copy_ceiling"] > 0
    variant = extra[1] if extra[:1] == ["--variant"] else "base"
    want = "zs_shard_step" if variant == "base" else "zs_shard_step_" + variant
    assert out["config"]["entry_point"] == want


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
