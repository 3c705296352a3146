"""The C-ABI library loads and exports every symbol include/zs.h declares;
struct layouts of the binding match the header (CPU only: no compute call)."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import sharded_mixed_precision_shard_amd as zs
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "zs.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(zs_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_entry_points():
    assert _declared_functions() == sorted(zs.EXPORTS)


def test_library_loads_and_exports_every_declared_symbol():
    lib = zs.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", zs.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (zs_\w+)", out))
    assert set(_declared_functions()) <= exported


def test_host_only_calls():
    assert zs.zs_status_string(zs.ZS_OK) == "ok"
    assert zs.zs_status_string(99) == "unknown status"
    assert zs.zs_algorithmic_bytes(2, 1000) == 30 * 1000
    assert zs.zs_algorithmic_bytes(8, 10) == 42 * 10
    assert zs.zs_algorithmic_bytes(0, 10) == 0


def test_step_before_init_is_rejected_without_touching_a_device():
    rc = zs.load_library().zs_shard_step(None, None, None, None, None, 1, 1, None, None, 1, None)
    assert rc == zs.ZS_ERR_NOT_INITIALIZED


def test_constants_match_header():
    text = open(HEADER).read()
    for name in ("ZS_MAX_K", "ZS_MAX_SEGMENTS", "ZS_Q8_BLOCK", "ZS_MAX_GROUPS_PER_CU"):
        m = re.search(r"#define %s (\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(zs, name), name


def test_struct_layout_matches_header():
    src = r'''
    #include <stddef.h>
    #include <stdio.h>
    #include "zs.h"
    int main(void) {
      printf("%zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(zs_hparams), sizeof(zs_segment),
             sizeof(zs_seg_table), sizeof(zs_launch_cfg), offsetof(zs_segment, wd_on),
             offsetof(zs_seg_table, count), offsetof(zs_hparams, grad_scale),
             offsetof(zs_launch_cfg, groups_per_cu));
      return 0; }
    '''
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "probe.c")
        exe = os.path.join(d, "probe")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), "-o", exe, c],
                       check=True)
        got = [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                              check=True).stdout.split()]
    want = [ctypes.sizeof(zs.ZsHparams), ctypes.sizeof(zs.ZsSegment),
            ctypes.sizeof(zs.ZsSegTable), ctypes.sizeof(zs.ZsLaunchCfg),
            zs.ZsSegment.wd_on.offset, zs.ZsSegTable.count.offset,
            zs.ZsHparams.grad_scale.offset, zs.ZsLaunchCfg.groups_per_cu.offset]
    assert got == want
    import oracle
    assert ctypes.sizeof(oracle.Segment) == ctypes.sizeof(zs.ZsSegment)
    assert ctypes.sizeof(oracle.Hparams) == ctypes.sizeof(zs.ZsHparams)


def test_product_has_no_oracle_dependency():
    """The product library and binding never reference the oracle."""
    out = subprocess.run(["nm", "-D", zs.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    assert "oracle" not in out
    pkg = os.path.dirname(zs.__file__)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "zs_oracle" not in text, f


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(zs, "_lib", None)
    monkeypatch.setattr(zs, "LIB_PATH", "/nonexistent/libzs.so")
    with pytest.raises(ImportError):
        zs.load_library()


def test_launch_geometry_keeps_the_grid_describable():
    """The grid a step launches (host-only query, no device): one 1024-element
    tile per workgroup by default, chunks doubled once workgroups * 256 would
    reach 2^32, every element covered exactly once."""
    tile = 1024
    assert zs.zs_launch_geometry(2, 0) == (0, 0)
    assert zs.zs_launch_geometry(2, 1) == (1, tile)
    assert zs.zs_launch_geometry(8, 8_053_473_280) == (7_864_720, tile)
    assert zs.zs_launch_geometry(2, 5 * tile + 1, chunk_tiles=3) == (2, 3 * tile)
    limit = (2 ** 32 - 1) // 256
    for n in (limit * tile, limit * tile + 1, 17_500_000_000, 18 * 10 ** 9, 2 ** 40 + 3):
        wg, chunk = zs.zs_launch_geometry(1, n)
        assert wg * 256 < 2 ** 32, n
        assert chunk % tile == 0 and (chunk // tile) & (chunk // tile - 1) == 0, n
        assert (wg - 1) * chunk < n <= wg * chunk, n
    assert zs.zs_launch_geometry(1, limit * tile)[1] == tile
    assert zs.zs_launch_geometry(1, limit * tile + 1)[1] == 2 * tile
    lib = zs.load_library()
    out = ctypes.c_int64(0)
    assert lib.zs_launch_geometry(0, 10, None, ctypes.byref(out), ctypes.byref(out)) == \
        zs.ZS_ERR_INVALID_ARGUMENT
    assert lib.zs_launch_geometry(1, -1, None, ctypes.byref(out), ctypes.byref(out)) == \
        zs.ZS_ERR_INVALID_ARGUMENT
    assert lib.zs_launch_geometry(1, 10, None, None, ctypes.byref(out)) == \
        zs.ZS_ERR_INVALID_ARGUMENT
    with pytest.raises(zs.ZsError):
        zs.zs_launch_geometry(1, 10, chunk_tiles=4097)
