"""CPU oracle for one rank's share of the sharded mixed-precision AdamW step.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does.

This module is a ctypes wrapper around ``libzs_oracle.so`` (built from
``zs_oracle.c`` by :func:`build`) plus numpy conveniences.  All arithmetic
lives in the C file; the wrapper only marshals arrays.  Sources and readings
are listed at the top of ``zs_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "zs_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libzs_oracle.so")

# gcc, one operation at a time: no contraction, no fast-math, denormals kept.
CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
          "-fno-unsafe-math-optimizations", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libzs_oracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class Segment(ctypes.Structure):
    _fields_ = [("start", ctypes.c_int64), ("wd_on", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class Hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float),
                ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("grad_scale", ctypes.c_float)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = load_library(_LIB_PATH)
    return _lib


def load_library(path: str):
    """Load an oracle shared library from `path` with its C signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.zs_oracle_shard_step.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int64,
                                         P, ctypes.c_int32, P, ctypes.c_int64]
    lib.zs_oracle_shard_step.restype = ctypes.c_int
    lib.zs_oracle_adamw_unsharded.argtypes = [P, P, P, P, P, P, ctypes.c_int64, P,
                                              ctypes.c_int64]
    lib.zs_oracle_adamw_unsharded.restype = ctypes.c_int
    lib.zs_oracle_bf16_rne.argtypes = [ctypes.c_float]
    lib.zs_oracle_bf16_rne.restype = ctypes.c_uint16
    lib.zs_oracle_bf16_rne_array.argtypes = [P, P, ctypes.c_int64]
    lib.zs_oracle_bf16_rne_array.restype = None
    lib.zs_oracle_scalars.argtypes = [P, ctypes.c_int64, P]
    lib.zs_oracle_scalars.restype = None
    lib.zs_oracle_q8_blocks.argtypes = [P, ctypes.c_int64, ctypes.c_int32, P, P]
    lib.zs_oracle_q8_blocks.restype = ctypes.c_int
    lib.zs_oracle_q8_dequant.argtypes = [P, P, ctypes.c_int64, ctypes.c_int32, P]
    lib.zs_oracle_q8_dequant.restype = None
    lib.zs_oracle_shard_step_q8grad.argtypes = [P, P, P, P, P, P, ctypes.c_int,
                                                ctypes.c_int64, ctypes.c_int32, P,
                                                ctypes.c_int32, P, ctypes.c_int64]
    lib.zs_oracle_shard_step_q8grad.restype = ctypes.c_int
    lib.zs_oracle_shard_step_bf16mv.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int64,
                                                P, ctypes.c_int32, P, ctypes.c_int64]
    lib.zs_oracle_shard_step_bf16mv.restype = ctypes.c_int
    lib.zs_oracle_splitmix64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    lib.zs_oracle_splitmix64.restype = ctypes.c_uint64
    lib.zs_oracle_bf16_sr_array.argtypes = [P, P, P, ctypes.c_int64]
    lib.zs_oracle_bf16_sr_array.restype = None
    lib.zs_oracle_sr_bits.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_int64]
    lib.zs_oracle_sr_bits.restype = ctypes.c_uint32
    lib.zs_oracle_shard_step_bf16mv_sr.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int64,
                                                   P, ctypes.c_int32, P, ctypes.c_int64,
                                                   ctypes.c_uint64, ctypes.c_int64]
    lib.zs_oracle_shard_step_bf16mv_sr.restype = ctypes.c_int
    return lib


def hparams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=1.0):
    return Hparams(lr, beta1, beta2, eps, weight_decay, grad_scale)


def segments_array(segs):
    """[(start, wd_on), ...] -> ctypes array of Segment."""
    arr = (Segment * len(segs))()
    for i, (s, f) in enumerate(segs):
        arr[i].start = int(s)
        arr[i].wd_on = 1 if f else 0
        arr[i].reserved = 0
    return arr


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _check(a, dtype, n, name):
    if not isinstance(a, np.ndarray) or a.dtype != dtype or a.ndim != 1 or a.shape[0] != n \
            or not a.flags["C_CONTIGUOUS"]:
        raise ValueError("%s must be a contiguous 1-D %s array of length %d" % (name, dtype, n))


def shard_step(master, m, v, param_bf16, grads, segs, hp: Hparams, step: int) -> int:
    """In-place oracle shard step on numpy arrays.

    master, m, v: float32[n]; param_bf16: uint16[n]; grads: list of uint16[n]
    (bf16 bit patterns); segs: list of (start, wd_on) or a Segment array.
    Returns the C status code (0 = ok, 2 = invalid argument).
    """
    n = master.shape[0]
    _check(master, np.float32, n, "master")
    _check(m, np.float32, n, "m")
    _check(v, np.float32, n, "v")
    _check(param_bf16, np.uint16, n, "param_bf16")
    for g in grads:
        _check(g, np.uint16, n, "grad")
    k = len(grads)
    gp = (ctypes.c_void_p * max(k, 1))(*[g.ctypes.data for g in grads])
    seg_arr = segs if isinstance(segs, ctypes.Array) else segments_array(segs)
    return _load().zs_oracle_shard_step(_ptr(master), _ptr(m), _ptr(v), _ptr(param_bf16),
                                        ctypes.cast(gp, ctypes.c_void_p), k, n,
                                        ctypes.cast(seg_arr, ctypes.c_void_p), len(seg_arr),
                                        ctypes.byref(hp), int(step))


def adamw_unsharded(w, m, v, param_bf16, g, decay_mask, hp: Hparams, step: int) -> int:
    """In-place unsharded AdamW: g float32[n] (reduced), decay_mask uint8[n]."""
    n = w.shape[0]
    _check(w, np.float32, n, "w")
    _check(m, np.float32, n, "m")
    _check(v, np.float32, n, "v")
    _check(param_bf16, np.uint16, n, "param_bf16")
    _check(g, np.float32, n, "g")
    _check(decay_mask, np.uint8, n, "decay_mask")
    return _load().zs_oracle_adamw_unsharded(_ptr(w), _ptr(m), _ptr(v), _ptr(param_bf16),
                                             _ptr(g), _ptr(decay_mask), n, ctypes.byref(hp),
                                             int(step))


def bf16_rne(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(x.shape[0], dtype=np.uint16)
    _load().zs_oracle_bf16_rne_array(_ptr(x), _ptr(out), x.shape[0])
    return out


def scalars(hp: Hparams, step: int):
    """(c1, c2, bc1, bc2, df) as float32, the per-call constants of the step."""
    out = np.zeros(5, dtype=np.float32)
    _load().zs_oracle_scalars(ctypes.byref(hp), int(step), _ptr(out))
    return tuple(np.float32(x) for x in out)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact: the 16 low bits are zero)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def q8_blocks(x_bf16: np.ndarray, block: int = 256):
    """Block-wise int8 quantization of bf16 bit patterns -> (q int8[n], scale float32[nb])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    n = x.shape[0]
    q = np.zeros(n, dtype=np.int8)
    sc = np.zeros(max(0, -(-n // block)), dtype=np.float32)
    rc = _load().zs_oracle_q8_blocks(_ptr(x), n, block, _ptr(q), _ptr(sc) if sc.size else None)
    if rc != 0:
        raise ValueError("zs_oracle_q8_blocks: invalid argument")
    return q, sc


def q8_dequant(q: np.ndarray, scale: np.ndarray, block: int = 256) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    scale = np.ascontiguousarray(scale, dtype=np.float32)
    out = np.empty(q.shape[0], dtype=np.float32)
    _load().zs_oracle_q8_dequant(_ptr(q), _ptr(scale), q.shape[0], block, _ptr(out))
    return out


def shard_step_q8grad(master, m, v, param_bf16, qgrads, qscales, segs, hp: Hparams, step: int,
                      block: int = 256) -> int:
    """Oracle step on int8 partials qgrads[j] (int8[n]) with block scales
    qscales[j] (float32[ceil(n/block)])."""
    n = master.shape[0]
    _check(master, np.float32, n, "master")
    _check(m, np.float32, n, "m")
    _check(v, np.float32, n, "v")
    _check(param_bf16, np.uint16, n, "param_bf16")
    nb = -(-n // block)
    for q, s in zip(qgrads, qscales):
        _check(q, np.int8, n, "qgrad")
        _check(s, np.float32, nb, "qscale")
    k = len(qgrads)
    qp = (ctypes.c_void_p * max(k, 1))(*[q.ctypes.data for q in qgrads])
    sp = (ctypes.c_void_p * max(k, 1))(*[s.ctypes.data for s in qscales])
    seg_arr = segs if isinstance(segs, ctypes.Array) else segments_array(segs)
    return _load().zs_oracle_shard_step_q8grad(
        _ptr(master), _ptr(m), _ptr(v), _ptr(param_bf16), ctypes.cast(qp, ctypes.c_void_p),
        ctypes.cast(sp, ctypes.c_void_p), k, n, block, ctypes.cast(seg_arr, ctypes.c_void_p),
        len(seg_arr), ctypes.byref(hp), int(step))


def shard_step_bf16mv(master, m_bf16, v_bf16, param_bf16, grads, segs, hp: Hparams,
                      step: int) -> int:
    """Oracle step with bf16 moments (uint16 bit patterns, updated in place)."""
    n = master.shape[0]
    _check(master, np.float32, n, "master")
    _check(m_bf16, np.uint16, n, "m")
    _check(v_bf16, np.uint16, n, "v")
    _check(param_bf16, np.uint16, n, "param_bf16")
    for g in grads:
        _check(g, np.uint16, n, "grad")
    k = len(grads)
    gp = (ctypes.c_void_p * max(k, 1))(*[g.ctypes.data for g in grads])
    seg_arr = segs if isinstance(segs, ctypes.Array) else segments_array(segs)
    return _load().zs_oracle_shard_step_bf16mv(
        _ptr(master), _ptr(m_bf16), _ptr(v_bf16), _ptr(param_bf16),
        ctypes.cast(gp, ctypes.c_void_p), k, n, ctypes.cast(seg_arr, ctypes.c_void_p),
        len(seg_arr), ctypes.byref(hp), int(step))


def splitmix64(key: int, i: int) -> int:
    """Output i of the SplitMix64 stream with key `key` (counter-style)."""
    return int(_load().zs_oracle_splitmix64(key & (2 ** 64 - 1), i & (2 ** 64 - 1)))


def bf16_sr(x: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Stochastic fp32 -> bf16 of each x with its 16 random bits r (low 16
    bits of uint32); uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    r = np.ascontiguousarray(r, dtype=np.uint32)
    if x.shape != r.shape:
        raise ValueError("x and r differ in shape")
    out = np.empty(x.shape, np.uint16)
    _load().zs_oracle_bf16_sr_array(_ptr(x), _ptr(r), _ptr(out), x.size)
    return out


def sr_bits(seed: int, step: int, which: int, i: int) -> int:
    """The 16 random bits the stochastic step uses for element i's m
    (which = 0) or v (which = 1) at step t."""
    return int(_load().zs_oracle_sr_bits(seed & (2 ** 64 - 1), int(step), int(which), int(i)))


def shard_step_bf16mv_sr(master, m_bf16, v_bf16, param_bf16, grads, segs, hp: Hparams,
                         step: int, seed: int, index0: int = 0) -> int:
    """Oracle step with bf16 moments rounded stochastically (uint16 bit
    patterns, updated in place); `seed` selects the random streams and the
    arrays hold shard elements index0 .. index0 + n - 1."""
    n = master.shape[0]
    _check(master, np.float32, n, "master")
    _check(m_bf16, np.uint16, n, "m")
    _check(v_bf16, np.uint16, n, "v")
    _check(param_bf16, np.uint16, n, "param_bf16")
    for g in grads:
        _check(g, np.uint16, n, "grad")
    k = len(grads)
    gp = (ctypes.c_void_p * max(k, 1))(*[g.ctypes.data for g in grads])
    seg_arr = segs if isinstance(segs, ctypes.Array) else segments_array(segs)
    return _load().zs_oracle_shard_step_bf16mv_sr(
        _ptr(master), _ptr(m_bf16), _ptr(v_bf16), _ptr(param_bf16),
        ctypes.cast(gp, ctypes.c_void_p), k, n, ctypes.cast(seg_arr, ctypes.c_void_p),
        len(seg_arr), ctypes.byref(hp), int(step), seed & (2 ** 64 - 1), int(index0))
