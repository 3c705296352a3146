"""Seeded synthetic inputs for the shard step: one definition, two twins.

``gen_host.c`` (host, gcc) and ``gen_device.hip`` (gfx950) implement the same
counter-based generator (SplitMix64 + Irwin-Hall, defined at the top of
``gen_host.c``) and produce bit-identical values, so any window of a shard
that was filled on the GPU can be regenerated on the host for the oracle.
This package holds none of the optimizer's arithmetic.

Roles of the streams: MASTER (fp32 master weights), GRAD (partial j of step
t), HEAVY (heavy-tail selector of partial j of step t).  m and v start at 0.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import numpy as np

from .layouts import (WORKLOADS, Shard, Workload, clip_segments, decay_mask_full,  # noqa
                      shard_of, workload)

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libzs_synth_host.so")
DEV_LIB = os.path.join(_HERE, "libzs_synth.so")

ROLE_MASTER = 1
ROLE_GRAD = 2
ROLE_HEAVY = 3
ROLE_QGRAD = 4    # int8 partial j of step t
ROLE_QSCALE = 5   # block scales of int8 partial j of step t

Q8_BLOCK = 256
Q8_SD = 42.0      # standard deviation of the drawn int8 codes (Irwin-Hall / 1560)


def build_host() -> str:
    tmp = HOST_LIB + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared", "-o",
                    tmp, os.path.join(_HERE, "gen_host.c")], check=True)
    os.replace(tmp, HOST_LIB)
    return HOST_LIB


def build_device() -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    tmp = DEV_LIB + ".tmp%d" % os.getpid()
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
                    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "-o", tmp, os.path.join(_HERE, "gen_device.hip")],
                   check=True)
    os.replace(tmp, DEV_LIB)
    return DEV_LIB


def build() -> None:
    build_host()
    build_device()


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            build_host()
        lib = ctypes.CDLL(HOST_LIB)
        U64, I64, P = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        lib.synth_stream_key.argtypes = [U64, ctypes.c_uint32, ctypes.c_uint32, U64]
        lib.synth_stream_key.restype = U64
        lib.synth_output.argtypes = [U64, U64]
        lib.synth_output.restype = U64
        for fn in (lib.synth_normal_f32, lib.synth_normal_bf16):
            fn.argtypes = [P, I64, U64, U64, I64, I64, ctypes.c_float, ctypes.c_uint32,
                           ctypes.c_float]
            fn.restype = None
        lib.synth_q8.argtypes = [P, I64, U64, I64, I64]
        lib.synth_q8.restype = None
        lib.synth_q8_scales.argtypes = [P, I64, U64, I64, ctypes.c_float]
        lib.synth_q8_scales.restype = None
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise ImportError("libzs_synth.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEV_LIB)
        U64, I64, P = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        for fn in (lib.synth_dev_normal_f32, lib.synth_dev_normal_bf16):
            fn.argtypes = [P, I64, U64, U64, I64, I64, ctypes.c_float, ctypes.c_uint32,
                           ctypes.c_float, P]
            fn.restype = ctypes.c_int
        lib.synth_dev_q8.argtypes = [P, I64, U64, I64, I64, P]
        lib.synth_dev_q8.restype = ctypes.c_int
        lib.synth_dev_q8_scales.argtypes = [P, I64, U64, I64, ctypes.c_float, P]
        lib.synth_dev_q8_scales.restype = ctypes.c_int
        _dev = lib
    return _dev


def stream_key(seed: int, role: int, j: int, t: int) -> int:
    return int(_host_lib().synth_stream_key(seed, role, j, t))


def splitmix_output(key: int, i: int) -> int:
    return int(_host_lib().synth_output(key, i))


def scale_of(sigma: float) -> np.float32:
    """sigma * 2^-16 in binary32 (exact power-of-two scaling of fp32(sigma))."""
    return np.float32(np.float32(sigma) * np.float32(2.0 ** -16))


def heavy_threshold(p: float) -> int:
    return int(round(p * 2.0 ** 32)) if p > 0 else 0


# ---------------------------------------------------------------- host side

def host_normal_f32(n, key, index0, valid_end, sigma, hkey=0, heavy_p=0.0, heavy_sigma=0.0):
    out = np.empty(int(n), dtype=np.float32)
    _host_lib().synth_normal_f32(out.ctypes.data, int(n), key, hkey, int(index0),
                                 int(valid_end), scale_of(sigma), heavy_threshold(heavy_p),
                                 scale_of(heavy_sigma))
    return out


def host_normal_bf16(n, key, index0, valid_end, sigma, hkey=0, heavy_p=0.0, heavy_sigma=0.0):
    out = np.empty(int(n), dtype=np.uint16)
    _host_lib().synth_normal_bf16(out.ctypes.data, int(n), key, hkey, int(index0),
                                  int(valid_end), scale_of(sigma), heavy_threshold(heavy_p),
                                  scale_of(heavy_sigma))
    return out


def _fill_parallel(out, fn, index0, threads):
    """Fill out[:] with fn(sub_out, n, index0 + offset) in `threads` slices
    (the C generators release the GIL, so the slices run concurrently)."""
    n = out.shape[0]
    if threads <= 1 or n < (1 << 20):
        fn(out, n, index0)
        return out
    from concurrent.futures import ThreadPoolExecutor
    step = -(-n // threads)
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda a: fn(out[a:a + step], min(step, n - a), index0 + a),
                    range(0, n, step)))
    return out


def host_master(w: Workload, lo: int = 0, hi: int = None, threads: int = 1):
    """fp32 master weights of shard elements [lo, hi)."""
    hi = w.n if hi is None else hi
    key = stream_key(w.seed, ROLE_MASTER, 0, 0)
    sc = scale_of(w.master_sigma)
    lib = _host_lib()
    out = np.empty(hi - lo, dtype=np.float32)
    return _fill_parallel(out, lambda o, n, i0: lib.synth_normal_f32(
        o.ctypes.data, n, key, 0, i0, w.shard.valid_end, sc, 0, np.float32(0)),
        w.shard.index0 + lo, threads)


def host_grads(w: Workload, t: int, lo: int = 0, hi: int = None, threads: int = 1):
    """The k bf16 partials of step t for shard elements [lo, hi)."""
    hi = w.n if hi is None else hi
    lib = _host_lib()
    out = []
    for j in range(w.k):
        key = stream_key(w.seed, ROLE_GRAD, j, t)
        hkey = stream_key(w.seed, ROLE_HEAVY, j, t)
        sc, hth, hsc = scale_of(w.grad_sigma), heavy_threshold(w.heavy_p), \
            scale_of(w.heavy_sigma)
        o = np.empty(hi - lo, dtype=np.uint16)
        out.append(_fill_parallel(o, lambda oo, n, i0: lib.synth_normal_bf16(
            oo.ctypes.data, n, key, hkey, i0, w.shard.valid_end, sc, hth, hsc),
            w.shard.index0 + lo, threads))
    return out


def q8_base_scale(sigma: float) -> np.float32:
    """Block scale base so that q * scale has about the partials' sigma."""
    return np.float32(sigma / Q8_SD)


def host_q8(n, key, index0, valid_end):
    out = np.empty(int(n), dtype=np.int8)
    _host_lib().synth_q8(out.ctypes.data, int(n), key, int(index0), int(valid_end))
    return out


def host_q8_scales(nblocks, skey, block0, base):
    out = np.empty(int(nblocks), dtype=np.float32)
    _host_lib().synth_q8_scales(out.ctypes.data, int(nblocks), skey, int(block0),
                                np.float32(base))
    return out


def host_qgrads(w: Workload, t: int, lo: int = 0, hi: int = None):
    """Int8 partials of step t for shard elements [lo, hi) (lo a multiple of
    the block) and the scales of the blocks they cover."""
    hi = w.n if hi is None else hi
    if lo % Q8_BLOCK:
        raise ValueError("window must start on a quantization block")
    nb = -(-(hi - lo) // Q8_BLOCK)
    qs, ss = [], []
    for j in range(w.k):
        qs.append(host_q8(hi - lo, stream_key(w.seed, ROLE_QGRAD, j, t), w.shard.index0 + lo,
                          w.shard.valid_end))
        ss.append(host_q8_scales(nb, stream_key(w.seed, ROLE_QSCALE, j, t), lo // Q8_BLOCK,
                                 q8_base_scale(w.grad_sigma)))
    return qs, ss


# -------------------------------------------------------------- device side

def _check_dev(out, dtype_name, n):
    import torch
    want = {"f32": torch.float32, "bf16bits": (torch.uint16, torch.int16, torch.bfloat16)}
    if not out.is_cuda or not out.is_contiguous() or out.numel() < n:
        raise ValueError("output must be a contiguous device tensor with >= %d elements" % n)
    ok = want[dtype_name]
    if (out.dtype not in ok) if isinstance(ok, tuple) else (out.dtype != ok):
        raise ValueError("wrong dtype %s for %s" % (out.dtype, dtype_name))


def _stream():
    import torch
    return ctypes.c_void_p(int(torch.cuda.current_stream().cuda_stream))


def dev_normal_f32(out, n, key, index0, valid_end, sigma, hkey=0, heavy_p=0.0, heavy_sigma=0.0):
    _check_dev(out, "f32", n)
    rc = _dev_lib().synth_dev_normal_f32(out.data_ptr(), int(n), key, hkey, int(index0),
                                         int(valid_end), scale_of(sigma),
                                         heavy_threshold(heavy_p), scale_of(heavy_sigma),
                                         _stream())
    if rc != 0:
        raise RuntimeError("synth_dev_normal_f32 failed with hip error %d" % rc)


def dev_normal_bf16(out, n, key, index0, valid_end, sigma, hkey=0, heavy_p=0.0,
                    heavy_sigma=0.0):
    _check_dev(out, "bf16bits", n)
    rc = _dev_lib().synth_dev_normal_bf16(out.data_ptr(), int(n), key, hkey, int(index0),
                                          int(valid_end), scale_of(sigma),
                                          heavy_threshold(heavy_p), scale_of(heavy_sigma),
                                          _stream())
    if rc != 0:
        raise RuntimeError("synth_dev_normal_bf16 failed with hip error %d" % rc)


def dev_master(w: Workload, out):
    dev_normal_f32(out, w.n, stream_key(w.seed, ROLE_MASTER, 0, 0), w.shard.index0,
                   w.shard.valid_end, w.master_sigma)


def dev_grads(w: Workload, t: int, outs):
    for j in range(w.k):
        dev_normal_bf16(outs[j], w.n, stream_key(w.seed, ROLE_GRAD, j, t), w.shard.index0,
                        w.shard.valid_end, w.grad_sigma, stream_key(w.seed, ROLE_HEAVY, j, t),
                        w.heavy_p, w.heavy_sigma)


def dev_q8(out, n, key, index0, valid_end):
    import torch
    if out.dtype != torch.int8 or not out.is_cuda or out.numel() < n:
        raise ValueError("out must be a device int8 tensor with >= %d elements" % n)
    rc = _dev_lib().synth_dev_q8(out.data_ptr(), int(n), key, int(index0), int(valid_end),
                                 _stream())
    if rc != 0:
        raise RuntimeError("synth_dev_q8 failed with hip error %d" % rc)


def dev_q8_scales(out, nblocks, skey, block0, base):
    _check_dev(out, "f32", nblocks)
    rc = _dev_lib().synth_dev_q8_scales(out.data_ptr(), int(nblocks), skey, int(block0),
                                        np.float32(base), _stream())
    if rc != 0:
        raise RuntimeError("synth_dev_q8_scales failed with hip error %d" % rc)


def dev_qgrads(w: Workload, t: int, qouts, souts):
    nb = -(-w.n // Q8_BLOCK)
    for j in range(w.k):
        dev_q8(qouts[j], w.n, stream_key(w.seed, ROLE_QGRAD, j, t), w.shard.index0,
               w.shard.valid_end)
        dev_q8_scales(souts[j], nb, stream_key(w.seed, ROLE_QSCALE, j, t), 0,
                      q8_base_scale(w.grad_sigma))
