"""The shard step captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

A launch of the library does no allocation, no memset and no synchronisation,
so it can be captured.  The graph keeps the arguments of the captured call,
including the step t, so every replay repeats that call.  Each replay is
compared bitwise with the same call made eagerly on twin buffers, with other
eager work and synchronisations between replays.
"""
import numpy as np
import pytest

import sharded_mixed_precision_shard_amd as zs
from tests import _gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    import torch
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    rc = zs.zs_init(0)
    assert rc == zs.ZS_OK, zs.zs_status_string(rc)
    yield torch
    torch.cuda.synchronize()


def _state(torch, w0, n, k, seed, entry):
    rng = np.random.default_rng(seed)
    f = lambda a: torch.from_numpy(a.copy()).cuda()  # noqa: E731
    st = dict(master=f(w0), m=torch.zeros(n, dtype=torch.float32, device="cuda"),
              v=torch.zeros(n, dtype=torch.float32, device="cuda"),
              param=torch.zeros(n, dtype=torch.int16, device="cuda"),
              grads=[f((rng.normal(0, 1e-2, n).astype(np.float32).view(np.uint32) >> 16)
                       .astype(np.uint16).view(np.int16)) for _ in range(k)])
    if entry in ("bf16mv", "packed_bf16mv", "bf16mv_sr"):
        st["m"] = torch.zeros(n, dtype=torch.int16, device="cuda")
        st["v"] = torch.zeros(n, dtype=torch.int16, device="cuda")
    if entry in ("packed", "packed_bf16mv"):
        z = np.zeros(n, np.uint16 if entry == "packed_bf16mv" else np.float32)
        pack = H.pack16_host if entry == "packed_bf16mv" else H.pack_host
        st["state"] = f(pack(w0, z, z))
        del st["master"], st["m"], st["v"]
    if entry == "q8ag":
        st["q8"] = torch.zeros(n, dtype=torch.int8, device="cuda")
        st["q8s"] = torch.zeros(-(-n // zs.ZS_Q8_BLOCK), dtype=torch.float32, device="cuda")
    return st


def _call(entry, st, k, n, table, hp, t, stream):
    if entry == "packed":
        zs.zs_shard_step_packed(st["state"], st["param"], st["grads"], k, n, zs.seg_table(table),
                                hp, t, stream)
    elif entry == "packed_bf16mv":
        zs.zs_shard_step_packed_bf16mv(st["state"], st["param"], st["grads"], k, n,
                                       zs.seg_table(table), hp, t, stream)
    elif entry == "bf16mv_sr":
        zs.zs_shard_step_bf16mv_sr(st["master"], st["m"], st["v"], st["param"], st["grads"], k,
                                   n, zs.seg_table(table), hp, t, 0xC0FFEE, stream)
    elif entry == "bf16mv":
        zs.zs_shard_step_bf16mv(st["master"], st["m"], st["v"], st["param"], st["grads"], k, n,
                                zs.seg_table(table), hp, t, stream)
    elif entry == "q8ag":
        zs.zs_shard_step_q8ag(st["master"], st["m"], st["v"], st["param"], st["q8"], st["q8s"],
                              st["grads"], k, n, zs.seg_table(table), hp, t, stream)
    else:
        zs.zs_shard_step(st["master"], st["m"], st["v"], st["param"], st["grads"], k, n,
                         zs.seg_table(table), hp, t, stream)


def _same(torch, a, b):
    for key in a:
        xs = a[key] if isinstance(a[key], list) else [a[key]]
        ys = b[key] if isinstance(b[key], list) else [b[key]]
        for x, y in zip(xs, ys):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), key


@pytest.mark.parametrize("entry", ["base", "q8ag", "bf16mv", "packed", "packed_bf16mv",
                                   "bf16mv_sr"],
                         ids=["zs_shard_step", "zs_shard_step_q8ag", "zs_shard_step_bf16mv",
                              "zs_shard_step_packed", "zs_shard_step_packed_bf16mv",
                              "zs_shard_step_bf16mv_sr"])
@pytest.mark.parametrize("t", [7, 10000])
def test_graph_replays_match_eager_calls(gpu, entry, t):
    torch = gpu
    n, k = 100_003, 3
    rng = np.random.default_rng(21)
    w0 = rng.normal(0, 0.02, n).astype(np.float32)
    segs, a = [], 0
    while a < n:
        segs.append((a, bool(rng.random() < 0.5)))
        a += int(rng.integers(1, 5000))
    table = H.segment_tensor(segs, "cuda")
    hp = zs.hparams(1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0)
    eager = _state(torch, w0, n, k, 5, entry)
    graphed = _state(torch, w0, n, k, 5, entry)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(entry, graphed, k, n, table, hp, t, torch.cuda.current_stream())
    torch.cuda.synchronize()
    _same(torch, graphed, _state(torch, w0, n, k, 5, entry))  # capture ran nothing

    for rep in range(4):
        g.replay()
        _call(entry, eager, k, n, table, hp, t, torch.cuda.current_stream())
        torch.cuda.synchronize()
        x = torch.randn(4096, device="cuda")
        assert torch.isfinite((x * x).sum())  # unrelated eager work between replays
        torch.cuda.synchronize()
        _same(torch, graphed, eager)
    if entry in ("packed", "packed_bf16mv"):
        block = 512 if entry == "packed_bf16mv" else 768
        moved = graphed["state"].view(-1, block)[:, :256].reshape(-1)[:n]
    else:
        moved = graphed["master"]
    assert not torch.equal(moved, torch.from_numpy(w0).cuda())
