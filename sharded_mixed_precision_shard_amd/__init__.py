"""Python binding of libzs (include/zs.h): one rank's fused ZeRO-shard AdamW step.

Argument marshalling only: every step of the path runs in the HIP library.
Device buffers may be given as torch tensors (their ``data_ptr()`` is used)
or as plain integer device addresses.  There is no CPU fallback: if
``libzs.so`` has not been built, importing the library raises.

Entry points keep the C names: :func:`zs_init`, :func:`zs_shard_step`,
:func:`zs_shard_step_cfg`, :func:`zs_shard_step_q8ag`, :func:`zs_shard_step_q8grad`,
:func:`zs_shard_step_bf16mv`, :func:`zs_shard_step_packed`,
:func:`zs_shard_step_packed_q8ag`, :func:`zs_shard_step_packed_q8grad`,
:func:`zs_shard_step_packed_bf16mv`, :func:`zs_shard_step_bf16mv_sr`,
:func:`zs_shard_step_packed_bf16mv_sr`, :func:`zs_pack_state`, :func:`zs_unpack_state`,
:func:`zs_pack_state_bf16mv`, :func:`zs_unpack_state_bf16mv`, :func:`zs_fini`,
:func:`zs_status_string`, :func:`zs_last_device_error`, :func:`zs_algorithmic_bytes`,
:func:`zs_launch_geometry`, :func:`zs_launch_plan`.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libzs.so")
HOST_LIB_PATH = os.path.join(PKG_DIR, "libzs_host.so")

ZS_MAX_K = 16
ZS_MAX_SEGMENTS = 65536
ZS_Q8_BLOCK = 256
ZS_MAX_GROUPS_PER_CU = 32

ZS_OK = 0
ZS_ERR_NOT_INITIALIZED = 1
ZS_ERR_INVALID_ARGUMENT = 2
ZS_ERR_MISALIGNED = 3
ZS_ERR_TOO_MANY_SEGMENTS = 4
ZS_ERR_DEVICE = 5
ZS_ERR_ALIASING = 6

ZS_VARIANT = {"base": 0, "q8ag": 1, "q8grad": 2, "bf16mv": 4, "packed": 16, "packed_q8ag": 17,
              "packed_q8grad": 18, "packed_bf16mv": 20, "bf16mv_sr": 36, "packed_bf16mv_sr": 52}

# Symbols declared in include/zs.h.
EXPORTS = ("zs_init", "zs_shard_step", "zs_shard_step_cfg", "zs_shard_step_q8ag",
           "zs_shard_step_q8grad", "zs_shard_step_bf16mv", "zs_shard_step_packed",
           "zs_shard_step_packed_q8ag", "zs_shard_step_packed_q8grad",
           "zs_shard_step_packed_bf16mv", "zs_shard_step_bf16mv_sr",
           "zs_shard_step_packed_bf16mv_sr", "zs_pack_state", "zs_unpack_state",
           "zs_pack_state_bf16mv", "zs_unpack_state_bf16mv", "zs_fini", "zs_status_string",
           "zs_last_device_error", "zs_algorithmic_bytes", "zs_launch_geometry",
           "zs_launch_plan")


def packed_floats(n: int) -> int:
    """Floats of the packed optimizer state for n elements (ZS_PACKED_FLOATS)."""
    return 768 * ((int(n) + 255) // 256)


def packed_bf16mv_floats(n: int) -> int:
    """Floats' room of the packed bf16-moment state for n elements
    (ZS_PACKED_BF16MV_FLOATS)."""
    return 512 * ((int(n) + 255) // 256)


class ZsHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("grad_scale", ctypes.c_float)]


class ZsSegment(ctypes.Structure):
    _fields_ = [("start", ctypes.c_int64), ("wd_on", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class ZsSegTable(ctypes.Structure):
    _fields_ = [("segs", ctypes.c_void_p), ("count", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class ZsLaunchCfg(ctypes.Structure):
    _fields_ = [("chunk_tiles", ctypes.c_int32), ("nontemporal", ctypes.c_int32),
                ("groups_per_cu", ctypes.c_int32), ("block_order", ctypes.c_int32)]


class ZsLaunchInfo(ctypes.Structure):
    _fields_ = [("workgroups", ctypes.c_int64), ("chunk_elements", ctypes.c_int64),
                ("block_order", ctypes.c_int32), ("groups_per_cu", ctypes.c_int32),
                ("nontemporal", ctypes.c_int32), ("window_quads", ctypes.c_int32)]


class ZsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (status %d, hip error %d)" % (
            where, zs_status_string(status), status, zs_last_device_error()))


_lib = None


def load_library():
    """Load libzs.so; raise if it is missing (no fallback of any kind)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libzs.so is not built (expected at %s); run "
                          "__graft_entry__.build() first" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    lib.zs_init.argtypes = [ctypes.c_int]
    lib.zs_init.restype = ctypes.c_int
    step_args = [P, P, P, P, P, ctypes.c_int, ctypes.c_int64, P, P, ctypes.c_int64, P]
    lib.zs_shard_step.argtypes = step_args
    lib.zs_shard_step.restype = ctypes.c_int
    lib.zs_shard_step_cfg.argtypes = step_args + [P]
    lib.zs_shard_step_cfg.restype = ctypes.c_int
    lib.zs_shard_step_q8ag.argtypes = [P, P, P, P, P, P, P, ctypes.c_int, ctypes.c_int64, P, P,
                                       ctypes.c_int64, P]
    lib.zs_shard_step_q8ag.restype = ctypes.c_int
    lib.zs_shard_step_q8grad.argtypes = [P, P, P, P, P, P, ctypes.c_int, ctypes.c_int64, P, P,
                                         ctypes.c_int64, P]
    lib.zs_shard_step_q8grad.restype = ctypes.c_int
    lib.zs_shard_step_bf16mv.argtypes = step_args
    lib.zs_shard_step_bf16mv.restype = ctypes.c_int
    lib.zs_shard_step_packed.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int64, P, P,
                                         ctypes.c_int64, P]
    lib.zs_shard_step_packed.restype = ctypes.c_int
    lib.zs_shard_step_packed_q8ag.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int64, P, P,
                                              ctypes.c_int64, P]
    lib.zs_shard_step_packed_q8ag.restype = ctypes.c_int
    lib.zs_shard_step_packed_q8grad.argtypes = [P, P, P, P, ctypes.c_int, ctypes.c_int64, P, P,
                                                ctypes.c_int64, P]
    lib.zs_shard_step_packed_q8grad.restype = ctypes.c_int
    lib.zs_shard_step_packed_bf16mv.argtypes = lib.zs_shard_step_packed.argtypes
    lib.zs_shard_step_packed_bf16mv.restype = ctypes.c_int
    lib.zs_shard_step_bf16mv_sr.argtypes = step_args[:-1] + [ctypes.c_uint64, P]
    lib.zs_shard_step_bf16mv_sr.restype = ctypes.c_int
    lib.zs_shard_step_packed_bf16mv_sr.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int64, P, P,
                                                   ctypes.c_int64, ctypes.c_uint64, P]
    lib.zs_shard_step_packed_bf16mv_sr.restype = ctypes.c_int
    lib.zs_pack_state_bf16mv.argtypes = [P, P, P, P, ctypes.c_int64, P]
    lib.zs_pack_state_bf16mv.restype = ctypes.c_int
    lib.zs_unpack_state_bf16mv.argtypes = [P, P, P, P, ctypes.c_int64, P]
    lib.zs_unpack_state_bf16mv.restype = ctypes.c_int
    lib.zs_pack_state.argtypes = [P, P, P, P, ctypes.c_int64, P]
    lib.zs_pack_state.restype = ctypes.c_int
    lib.zs_unpack_state.argtypes = [P, P, P, P, ctypes.c_int64, P]
    lib.zs_unpack_state.restype = ctypes.c_int
    lib.zs_fini.argtypes = []
    lib.zs_fini.restype = ctypes.c_int
    lib.zs_status_string.argtypes = [ctypes.c_int]
    lib.zs_status_string.restype = ctypes.c_char_p
    lib.zs_last_device_error.argtypes = []
    lib.zs_last_device_error.restype = ctypes.c_int
    lib.zs_algorithmic_bytes.argtypes = [ctypes.c_int, ctypes.c_int64]
    lib.zs_algorithmic_bytes.restype = ctypes.c_int64
    lib.zs_launch_geometry.argtypes = [ctypes.c_int, ctypes.c_int64, P, P, P]
    lib.zs_launch_geometry.restype = ctypes.c_int
    lib.zs_launch_plan.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, P, P]
    lib.zs_launch_plan.restype = ctypes.c_int
    _lib = lib
    return lib


def _host(x, nbytes: int, name: str) -> int:
    """Address of a buffer for the host step: a contiguous numpy array or CPU
    tensor holding at least ``nbytes``, or an integer host address."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if hasattr(x, "ctypes") and hasattr(x, "dtype"):  # numpy array
        if not x.flags["C_CONTIGUOUS"]:
            raise ValueError("%s must be contiguous" % name)
        have = x.nbytes
        addr = int(x.ctypes.data)
    elif hasattr(x, "data_ptr"):
        if getattr(x, "is_cuda", False):
            raise ValueError("%s: a GPU tensor cannot be passed to the host step" % name)
        if not x.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        have = x.numel() * x.element_size()
        addr = int(x.data_ptr())
    else:
        raise TypeError("%s: expected a host array or an integer address, got %r" % (name,
                                                                                   type(x)))
    if have < nbytes:
        raise ValueError("%s holds %d bytes; the call needs %d" % (name, have, nbytes))
    return addr


def _dev(x, nbytes: int, name: str) -> int:
    """Address of a buffer for a GPU entry point.  A torch tensor must live on
    a GPU, be contiguous and hold at least ``nbytes``; a host (numpy) array is
    refused, since its address would reach the kernel.  An integer is taken
    as a device address on the caller's word; None is the null pointer."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if hasattr(x, "ctypes") and hasattr(x, "dtype"):
        raise TypeError("%s: a host (numpy) array cannot be passed to a GPU entry point" % name)
    if hasattr(x, "data_ptr"):
        if not getattr(x, "is_cuda", False):
            raise ValueError("%s must be a GPU tensor (got device %s)" % (name, x.device))
        if not x.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        have = x.numel() * x.element_size()
        if have < nbytes:
            raise ValueError("%s holds %d bytes; the call needs %d" % (name, have, nbytes))
        return int(x.data_ptr())
    raise TypeError("%s: expected a GPU tensor or an integer address, got %r" % (name, type(x)))


def _stream_handle(stream) -> int:
    if stream is None:
        return 0
    if isinstance(stream, int):
        return stream
    if hasattr(stream, "cuda_stream"):
        return int(stream.cuda_stream)
    raise TypeError("stream must be None, an int hipStream_t or a torch stream")


def hparams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, grad_scale=1.0):
    return ZsHparams(lr, beta1, beta2, eps, weight_decay, grad_scale)


def seg_table(segs, count=None) -> ZsSegTable:
    """Describe a device-resident table.  ``segs`` is a device tensor of int64
    pairs [count, 2] = (start, wd_on | reserved << 32) or an address.  A count
    beyond the tensor's rows is refused here unless the library itself would
    refuse it (more than ZS_MAX_SEGMENTS entries: nothing is read)."""
    if count is None:
        count = int(segs.shape[0])
    count = int(count)
    need = 16 * count if 0 < count <= ZS_MAX_SEGMENTS else 0
    return ZsSegTable(_dev(segs, need, "segment table"), count, 0)


def zs_init(device_ordinal: int = 0) -> int:
    return load_library().zs_init(int(device_ordinal))


def zs_fini() -> int:
    return load_library().zs_fini()


def zs_status_string(status: int) -> str:
    return load_library().zs_status_string(int(status)).decode()


def zs_last_device_error() -> int:
    return load_library().zs_last_device_error()


def zs_algorithmic_bytes(k: int, n: int) -> int:
    return load_library().zs_algorithmic_bytes(int(k), int(n))


def zs_launch_geometry(k: int, n: int, chunk_tiles: int = 0):
    """(workgroups, elements per workgroup) of the grid a step would launch."""
    cfg = ZsLaunchCfg(int(chunk_tiles), 0, 0, 0)
    wg, ch = ctypes.c_int64(0), ctypes.c_int64(0)
    rc = load_library().zs_launch_geometry(int(k), int(n), ctypes.byref(cfg), ctypes.byref(wg),
                                           ctypes.byref(ch))
    if rc != ZS_OK:
        raise ZsError(rc, "zs_launch_geometry")
    return wg.value, ch.value


def _check_k(k, arrays, name):
    """The partial count the C call receives: len(arrays), or an explicit k
    that must equal it (the library reads k pointers from the array, so a
    larger k would read past its end)."""
    if k is None:
        return len(arrays)
    if int(k) != len(arrays):
        raise ValueError("k=%d but %d %s were given" % (int(k), len(arrays), name))
    return int(k)


def zs_launch_plan(k: int, n: int, variant: str = "base", cfg=None) -> dict:
    """The launch a call of entry point ``variant`` (a key of ZS_VARIANT:
    "base", "q8ag", "q8grad", "bf16mv" or a packed form) would make: grid,
    chunk, chunk order, occupancy cap, cache policy and sub-windows per
    wavefront, as a dict of the zs_launch_info fields.  ``cfg`` (base only)
    is a dict of ZsLaunchCfg fields or None."""
    c = None
    if cfg:
        c = ZsLaunchCfg(**{f: int(cfg.get(f, 0)) for f, _ in ZsLaunchCfg._fields_})
    out = ZsLaunchInfo()
    rc = load_library().zs_launch_plan(int(k), int(n), ZS_VARIANT[variant],
                                       ctypes.byref(c) if c is not None else None,
                                       ctypes.byref(out))
    if rc != ZS_OK:
        raise ZsError(rc, "zs_launch_plan")
    return {f: getattr(out, f) for f, _ in ZsLaunchInfo._fields_}


def _marshal(master, m, v, param_bf16, grads, k, n, seg_table_, hparams_, mv_size=4):
    """Pointers of one step call; every tensor checked against n elements."""
    k = _check_k(k, grads, "grads")
    nn = max(int(n), 0)
    gp = _ptr_array(grads, 2 * nn, "grads")
    st = seg_table_ if isinstance(seg_table_, ZsSegTable) else seg_table(seg_table_)
    return (ctypes.c_void_p(_dev(master, 4 * nn, "master")),
            ctypes.c_void_p(_dev(m, mv_size * nn, "m")),
            ctypes.c_void_p(_dev(v, mv_size * nn, "v")),
            ctypes.c_void_p(_dev(param_bf16, 2 * nn, "param_bf16")),
            ctypes.cast(gp, ctypes.c_void_p), int(k), st, hparams_, gp)


def _ptr_array(xs, nbytes, name):
    return (ctypes.c_void_p * max(len(xs), 1))(
        *[_dev(x, nbytes, "%s[%d]" % (name, j)) for j, x in enumerate(xs)])


def zs_shard_step(master, m, v, param_bf16, grads, k, n, seg_table_, hparams_, step,
                  stream=None, check=True) -> int:
    """Enqueue one shard step (see include/zs.h).  Raises ZsError on a
    non-zero status when ``check`` is true; returns the status otherwise."""
    pm, pmm, pv, pp, pg, kk, st, hp, keep = _marshal(master, m, v, param_bf16, grads, k, n,
                                                     seg_table_, hparams_)
    rc = load_library().zs_shard_step(pm, pmm, pv, pp, pg, kk, int(n), ctypes.byref(st),
                                      ctypes.byref(hp), int(step),
                                      ctypes.c_void_p(_stream_handle(stream)))
    del keep
    if check and rc != ZS_OK:
        raise ZsError(rc, "zs_shard_step")
    return rc


def zs_shard_step_cfg(master, m, v, param_bf16, grads, k, n, seg_table_, hparams_, step,
                      stream=None, chunk_tiles=0, nontemporal=0, groups_per_cu=0,
                      block_order=0, check=True) -> int:
    """zs_shard_step with an explicit launch geometry (results never change)."""
    pm, pmm, pv, pp, pg, kk, st, hp, keep = _marshal(master, m, v, param_bf16, grads, k, n,
                                                     seg_table_, hparams_)
    cfg = ZsLaunchCfg(int(chunk_tiles), int(nontemporal), int(groups_per_cu), int(block_order))
    rc = load_library().zs_shard_step_cfg(pm, pmm, pv, pp, pg, kk, int(n), ctypes.byref(st),
                                          ctypes.byref(hp), int(step),
                                          ctypes.c_void_p(_stream_handle(stream)),
                                          ctypes.byref(cfg))
    del keep
    if check and rc != ZS_OK:
        raise ZsError(rc, "zs_shard_step_cfg")
    return rc


def zs_shard_step_q8ag(master, m, v, param_bf16, param_q8, param_q8_scale, grads, k, n,
                       seg_table_, hparams_, step, stream=None, check=True) -> int:
    """zs_shard_step that also writes the int8 block-quantized parameter copy
    (param_q8: int8[n]) and its block scales (float32[ceil(n/256)])."""
    pm, pmm, pv, pp, pg, kk, st, hp, keep = _marshal(master, m, v, param_bf16, grads, k, n,
                                                     seg_table_, hparams_)
    nn = max(int(n), 0)
    nb = -(-nn // ZS_Q8_BLOCK)
    rc = load_library().zs_shard_step_q8ag(
        pm, pmm, pv, pp, ctypes.c_void_p(_dev(param_q8, nn, "param_q8")),
        ctypes.c_void_p(_dev(param_q8_scale, 4 * nb, "param_q8_scale")), pg, kk, int(n),
        ctypes.byref(st), ctypes.byref(hp), int(step), ctypes.c_void_p(_stream_handle(stream)))
    del keep
    if check and rc != ZS_OK:
        raise ZsError(rc, "zs_shard_step_q8ag")
    return rc


def zs_shard_step_q8grad(master, m, v, param_bf16, qgrads, qscales, k, n, seg_table_, hparams_,
                         step, stream=None, check=True) -> int:
    """zs_shard_step on int8 partials qgrads[j] (int8[n]) with block scales
    qscales[j] (float32[ceil(n/256)])."""
    nn = max(int(n), 0)
    nb = -(-nn // ZS_Q8_BLOCK)
    k = _check_k(k, qgrads, "qgrads")
    if len(qscales) != len(qgrads):
        raise ValueError("%d qscales for %d qgrads: one scale array per int8 partial"
                         % (len(qscales), len(qgrads)))
    pm, pmm, pv, pp, _, _, st, hp, _ = _marshal(master, m, v, param_bf16, [], 0, n, seg_table_,
                                                hparams_)
    qp = _ptr_array(qgrads, nn, "qgrads")
    sp = _ptr_array(qscales, 4 * nb, "qscales")
    rc = load_library().zs_shard_step_q8grad(
        pm, pmm, pv, pp, ctypes.cast(qp, ctypes.c_void_p), ctypes.cast(sp, ctypes.c_void_p),
        k, int(n), ctypes.byref(st), ctypes.byref(hp),
        int(step), ctypes.c_void_p(_stream_handle(stream)))
    if check and rc != ZS_OK:
        raise ZsError(rc, "zs_shard_step_q8grad")
    return rc


def zs_shard_step_bf16mv(master, m_bf16, v_bf16, param_bf16, grads, k, n, seg_table_, hparams_,
                         step, stream=None, check=True) -> int:
    """zs_shard_step with bf16 moments m_bf16, v_bf16 (bf16[n], in place)."""
    pm, pmm, pv, pp, pg, kk, st, hp, keep = _marshal(master, m_bf16, v_bf16, param_bf16, grads,
                                                     k, n, seg_table_, hparams_, mv_size=2)
    rc = load_library().zs_shard_step_bf16mv(pm, pmm, pv, pp, pg, kk, int(n), ctypes.byref(st),
                                             ctypes.byref(hp), int(step),
                                             ctypes.c_void_p(_stream_handle(stream)))
    del keep
    if check and rc != ZS_OK:
        raise ZsError(rc, "zs_shard_step_bf16mv")
    return rc


def zs_shard_step_bf16mv_sr(master, m_bf16, v_bf16, param_bf16, grads, k, n, seg_table_,
                            hparams_, step, seed, stream=None, check=True) -> int:
    """zs_shard_step_bf16mv with m and v rounded stochastically; `seed`
    (uint64) selects the random streams."""
    pm, pmm, pv, pp, pg, kk, st, hp, keep = _marshal(master, m_bf16, v_bf16, param_bf16, grads,
                                                     k, n, seg_table_, hparams_, mv_size=2)
    rc = load_library().zs_shard_step_bf16mv_sr(pm, pmm, pv, pp, pg, kk, int(n), ctypes.byref(st),
                                                ctypes.byref(hp), int(step), _seed(seed),
                                                ctypes.c_void_p(_stream_handle(stream)))
    del keep
    if check and rc != ZS_OK:
        raise ZsError(rc, "zs_shard_step_bf16mv_sr")
    return rc


def _seed(seed) -> int:
    s = int(seed)
    if not 0 <= s < 2 ** 64:
        raise ValueError("seed must be an unsigned 64-bit integer, got %d" % s)
    return s


def zs_shard_step_packed(state, param_bf16, grads, k, n, seg_table_, hparams_, step,
                         stream=None, check=True) -> int:
    """zs_shard_step on the packed optimizer state (fp32 [packed_floats(n)]:
    per 256-element block its master values, then m, then v)."""
    k = _check_k(k, grads, "grads")
    nn = max(int(n), 0)
    gp = _ptr_array(grads, 2 * nn, "grads")
    st = seg_table_ if isinstance(seg_table_, ZsSegTable) else seg_table(seg_table_)
    rc = load_library().zs_shard_step_packed(
        ctypes.c_void_p(_dev(state, 4 * packed_floats(nn), "state")),
        ctypes.c_void_p(_dev(param_bf16, 2 * nn, "param_bf16")), ctypes.cast(gp, ctypes.c_void_p),
        int(k), int(n), ctypes.byref(st), ctypes.byref(hparams_), int(step),
        ctypes.c_void_p(_stream_handle(stream)))
    if check and rc != ZS_OK:
        raise ZsError(rc, "zs_shard_step_packed")
    return rc


def zs_shard_step_packed_q8ag(state, param_bf16, param_q8, param_q8_scale, grads, k, n,
                              seg_table_, hparams_, step, stream=None, check=True) -> int:
    """zs_shard_step_q8ag on the packed state."""
    k = _check_k(k, grads, "grads")
    nn = max(int(n), 0)
    nb = -(-nn // ZS_Q8_BLOCK)
    gp = _ptr_array(grads, 2 * nn, "grads")
    st = seg_table_ if isinstance(seg_table_, ZsSegTable) else seg_table(seg_table_)
    rc = load_library().zs_shard_step_packed_q8ag(
        ctypes.c_void_p(_dev(state, 4 * packed_floats(nn), "state")),
        ctypes.c_void_p(_dev(param_bf16, 2 * nn, "param_bf16")),
        ctypes.c_void_p(_dev(param_q8, nn, "param_q8")),
        ctypes.c_void_p(_dev(param_q8_scale, 4 * nb, "param_q8_scale")),
        ctypes.cast(gp, ctypes.c_void_p), int(k), int(n), ctypes.byref(st),
        ctypes.byref(hparams_), int(step), ctypes.c_void_p(_stream_handle(stream)))
    if check and rc != ZS_OK:
        raise ZsError(rc, "zs_shard_step_packed_q8ag")
    return rc


def zs_shard_step_packed_q8grad(state, param_bf16, qgrads, qscales, k, n, seg_table_, hparams_,
                                step, stream=None, check=True) -> int:
    """zs_shard_step_q8grad on the packed state."""
    nn = max(int(n), 0)
    nb = -(-nn // ZS_Q8_BLOCK)
    k = _check_k(k, qgrads, "qgrads")
    if len(qscales) != len(qgrads):
        raise ValueError("%d qscales for %d qgrads: one scale array per int8 partial"
                         % (len(qscales), len(qgrads)))
    qp = _ptr_array(qgrads, nn, "qgrads")
    sp = _ptr_array(qscales, 4 * nb, "qscales")
    st = seg_table_ if isinstance(seg_table_, ZsSegTable) else seg_table(seg_table_)
    rc = load_library().zs_shard_step_packed_q8grad(
        ctypes.c_void_p(_dev(state, 4 * packed_floats(nn), "state")),
        ctypes.c_void_p(_dev(param_bf16, 2 * nn, "param_bf16")),
        ctypes.cast(qp, ctypes.c_void_p), ctypes.cast(sp, ctypes.c_void_p), int(k), int(n),
        ctypes.byref(st), ctypes.byref(hparams_), int(step),
        ctypes.c_void_p(_stream_handle(stream)))
    if check and rc != ZS_OK:
        raise ZsError(rc, "zs_shard_step_packed_q8grad")
    return rc


def zs_shard_step_packed_bf16mv(state, param_bf16, grads, k, n, seg_table_, hparams_, step,
                                stream=None, check=True) -> int:
    """zs_shard_step_bf16mv on the packed state (packed_bf16mv_floats(n)
    floats: per 256-element block its fp32 master values, then bf16 m and v)."""
    k = _check_k(k, grads, "grads")
    nn = max(int(n), 0)
    gp = _ptr_array(grads, 2 * nn, "grads")
    st = seg_table_ if isinstance(seg_table_, ZsSegTable) else seg_table(seg_table_)
    rc = load_library().zs_shard_step_packed_bf16mv(
        ctypes.c_void_p(_dev(state, 4 * packed_bf16mv_floats(nn), "state")),
        ctypes.c_void_p(_dev(param_bf16, 2 * nn, "param_bf16")), ctypes.cast(gp, ctypes.c_void_p),
        int(k), int(n), ctypes.byref(st), ctypes.byref(hparams_), int(step),
        ctypes.c_void_p(_stream_handle(stream)))
    if check and rc != ZS_OK:
        raise ZsError(rc, "zs_shard_step_packed_bf16mv")
    return rc


def zs_pack_state(master, m, v, state, n, stream=None, check=True) -> int:
    """Separate fp32 master, m, v [n] -> packed state [packed_floats(n)] (padding +0)."""
    nn = max(int(n), 0)
    rc = load_library().zs_pack_state(
        ctypes.c_void_p(_dev(master, 4 * nn, "master")), ctypes.c_void_p(_dev(m, 4 * nn, "m")),
        ctypes.c_void_p(_dev(v, 4 * nn, "v")),
        ctypes.c_void_p(_dev(state, 4 * packed_floats(nn), "state")), int(n),
        ctypes.c_void_p(_stream_handle(stream)))
    if check and rc != ZS_OK:
        raise ZsError(rc, "zs_pack_state")
    return rc


def zs_unpack_state(state, master, m, v, n, stream=None, check=True) -> int:
    """Packed state [packed_floats(n)] -> separate fp32 master, m, v [n]."""
    nn = max(int(n), 0)
    rc = load_library().zs_unpack_state(
        ctypes.c_void_p(_dev(state, 4 * packed_floats(nn), "state")),
        ctypes.c_void_p(_dev(master, 4 * nn, "master")), ctypes.c_void_p(_dev(m, 4 * nn, "m")),
        ctypes.c_void_p(_dev(v, 4 * nn, "v")), int(n), ctypes.c_void_p(_stream_handle(stream)))
    if check and rc != ZS_OK:
        raise ZsError(rc, "zs_unpack_state")
    return rc


def zs_shard_step_packed_bf16mv_sr(state, param_bf16, grads, k, n, seg_table_, hparams_, step,
                                   seed, stream=None, check=True) -> int:
    """zs_shard_step_packed_bf16mv with m and v rounded stochastically."""
    k = _check_k(k, grads, "grads")
    nn = max(int(n), 0)
    gp = _ptr_array(grads, 2 * nn, "grads")
    st = seg_table_ if isinstance(seg_table_, ZsSegTable) else seg_table(seg_table_)
    rc = load_library().zs_shard_step_packed_bf16mv_sr(
        ctypes.c_void_p(_dev(state, 4 * packed_bf16mv_floats(nn), "state")),
        ctypes.c_void_p(_dev(param_bf16, 2 * nn, "param_bf16")), ctypes.cast(gp, ctypes.c_void_p),
        int(k), int(n), ctypes.byref(st), ctypes.byref(hparams_), int(step), _seed(seed),
        ctypes.c_void_p(_stream_handle(stream)))
    if check and rc != ZS_OK:
        raise ZsError(rc, "zs_shard_step_packed_bf16mv_sr")
    return rc


def zs_pack_state_bf16mv(master, m_bf16, v_bf16, state, n, stream=None, check=True) -> int:
    """fp32 master, bf16 m, v [n] -> packed bf16-moment state (padding zero)."""
    nn = max(int(n), 0)
    rc = load_library().zs_pack_state_bf16mv(
        ctypes.c_void_p(_dev(master, 4 * nn, "master")),
        ctypes.c_void_p(_dev(m_bf16, 2 * nn, "m_bf16")),
        ctypes.c_void_p(_dev(v_bf16, 2 * nn, "v_bf16")),
        ctypes.c_void_p(_dev(state, 4 * packed_bf16mv_floats(nn), "state")), int(n),
        ctypes.c_void_p(_stream_handle(stream)))
    if check and rc != ZS_OK:
        raise ZsError(rc, "zs_pack_state_bf16mv")
    return rc


def zs_unpack_state_bf16mv(state, master, m_bf16, v_bf16, n, stream=None, check=True) -> int:
    """Packed bf16-moment state -> fp32 master, bf16 m, v [n]."""
    nn = max(int(n), 0)
    rc = load_library().zs_unpack_state_bf16mv(
        ctypes.c_void_p(_dev(state, 4 * packed_bf16mv_floats(nn), "state")),
        ctypes.c_void_p(_dev(master, 4 * nn, "master")),
        ctypes.c_void_p(_dev(m_bf16, 2 * nn, "m_bf16")),
        ctypes.c_void_p(_dev(v_bf16, 2 * nn, "v_bf16")), int(n),
        ctypes.c_void_p(_stream_handle(stream)))
    if check and rc != ZS_OK:
        raise ZsError(rc, "zs_unpack_state_bf16mv")
    return rc


class ShardStep:
    """One rank's step with its buffers fixed: the arguments are checked and
    marshalled once, and each call passes only the step t and the stream to
    the C ABI (include/zs.h) -- for loops that call the step many times on
    the same state.  ``variant`` is "base" (zs_shard_step, or
    zs_shard_step_cfg when ``cfg`` is given as a dict of ZsLaunchCfg fields),
    "q8ag" (needs ``param_q8`` and ``param_q8_scale``), "q8grad" (``grads``
    are the int8 partials, ``qscales`` their block scales) or "bf16mv" (m and
    v are bf16) or "packed" (``master`` is the packed state, m and v are None),
    and "packed_q8ag" / "packed_q8grad" / "packed_bf16mv" (those forms on
    their packed state); "bf16mv_sr" and "packed_bf16mv_sr" round the bf16
    moments stochastically with the random streams of ``seed``.
    The tensors are referenced for the object's lifetime."""

    def __init__(self, master, m, v, param_bf16, grads, n, seg_table_, hparams_,
                 variant="base", param_q8=None, param_q8_scale=None, qscales=None, cfg=None,
                 seed=None):
        lib = load_library()
        # the stochastic forms take the seed between the step and the stream
        self._mid = []
        if variant.endswith("_sr"):
            if seed is None:
                raise ValueError("%s needs a seed" % variant)
            self._mid = [_seed(seed)]
        elif seed is not None:
            raise ValueError("a seed applies to the stochastic-rounding forms only")
        self._keep = [master, m, v, param_bf16, list(grads), seg_table_, param_q8,
                      param_q8_scale, qscales]
        self.n = int(n)
        nn = max(self.n, 0)
        nb = -(-nn // ZS_Q8_BLOCK)
        k = len(grads)
        if variant == "q8grad":
            pm, pmm, pv, pp, _, _, st, hp, _ = _marshal(master, m, v, param_bf16, [], 0, n,
                                                        seg_table_, hparams_)
            qp = _ptr_array(grads, nn, "qgrads")
            sp = _ptr_array(qscales or [], 4 * nb, "qscales")
            if len(qscales or []) != k:
                raise ValueError("q8grad needs one scale array per int8 partial")
            self._c = (qp, sp)
            head = [pm, pmm, pv, pp, ctypes.cast(qp, ctypes.c_void_p),
                    ctypes.cast(sp, ctypes.c_void_p)]
            fn = lib.zs_shard_step_q8grad
        elif variant in ("packed", "packed_q8ag", "packed_q8grad", "packed_bf16mv",
                         "packed_bf16mv_sr"):
            if m is not None or v is not None:
                raise ValueError("the packed step takes its m and v inside the state")
            st = seg_table_ if isinstance(seg_table_, ZsSegTable) else seg_table(seg_table_)
            hp = hparams_
            floats = packed_bf16mv_floats(nn) if variant.startswith("packed_bf16mv") \
                else packed_floats(nn)
            head = [ctypes.c_void_p(_dev(master, 4 * floats, "state")),
                    ctypes.c_void_p(_dev(param_bf16, 2 * nn, "param_bf16"))]
            if variant == "packed_q8grad":
                if len(qscales or []) != k:
                    raise ValueError("q8grad needs one scale array per int8 partial")
                qp = _ptr_array(grads, nn, "qgrads")
                sp = _ptr_array(qscales, 4 * nb, "qscales")
                self._c = (qp, sp)
                head += [ctypes.cast(qp, ctypes.c_void_p), ctypes.cast(sp, ctypes.c_void_p)]
                fn = lib.zs_shard_step_packed_q8grad
            else:
                gp = _ptr_array(grads, 2 * nn, "grads")
                self._c = (gp,)
                if variant == "packed_q8ag":
                    head += [ctypes.c_void_p(_dev(param_q8, nn, "param_q8")),
                             ctypes.c_void_p(_dev(param_q8_scale, 4 * nb, "param_q8_scale"))]
                    fn = lib.zs_shard_step_packed_q8ag
                elif variant == "packed_bf16mv":
                    fn = lib.zs_shard_step_packed_bf16mv
                elif variant == "packed_bf16mv_sr":
                    fn = lib.zs_shard_step_packed_bf16mv_sr
                else:
                    fn = lib.zs_shard_step_packed
                head.append(ctypes.cast(gp, ctypes.c_void_p))
        else:
            mv = 2 if variant in ("bf16mv", "bf16mv_sr") else 4
            pm, pmm, pv, pp, pg, _, st, hp, gp = _marshal(master, m, v, param_bf16, grads, k, n,
                                                          seg_table_, hparams_, mv_size=mv)
            self._c = (gp,)
            if variant == "q8ag":
                head = [pm, pmm, pv, pp, ctypes.c_void_p(_dev(param_q8, nn, "param_q8")),
                        ctypes.c_void_p(_dev(param_q8_scale, 4 * nb, "param_q8_scale")), pg]
                fn = lib.zs_shard_step_q8ag
            elif variant == "bf16mv":
                head, fn = [pm, pmm, pv, pp, pg], lib.zs_shard_step_bf16mv
            elif variant == "bf16mv_sr":
                head, fn = [pm, pmm, pv, pp, pg], lib.zs_shard_step_bf16mv_sr
            elif variant == "base":
                head = [pm, pmm, pv, pp, pg]
                fn = lib.zs_shard_step_cfg if cfg else lib.zs_shard_step
            else:
                raise ValueError("unknown variant %r" % (variant,))
        self._st, self._hp = st, hp
        self._head = head + [int(k), self.n, ctypes.byref(st), ctypes.byref(hp)]
        self._tail = []
        if cfg and variant == "base":
            self._cfg = ZsLaunchCfg(**{f: int(cfg.get(f, 0)) for f, _ in ZsLaunchCfg._fields_})
            self._tail = [ctypes.byref(self._cfg)]
        elif cfg:
            raise ValueError("a launch cfg applies to the base entry point only")
        self._fn = fn
        self.variant = variant

    def __call__(self, step, stream=None, check=True) -> int:
        rc = self._fn(*self._head, int(step), *self._mid,
                      ctypes.c_void_p(_stream_handle(stream)), *self._tail)
        if check and rc != ZS_OK:
            raise ZsError(rc, "ShardStep(%s)" % self.variant)
        return rc


def algorithmic_bytes(variant: str, k: int, n: int) -> int:
    """HBM bytes one call moves by the algorithm, per entry point."""
    nb = -(-n // ZS_Q8_BLOCK)
    if variant in ("base", "packed"):
        return (26 + 2 * k) * n
    if variant in ("q8ag", "packed_q8ag"):
        return (26 + 2 * k) * n + n + 4 * nb
    if variant in ("q8grad", "packed_q8grad"):
        return (12 + k + 14) * n + 4 * k * nb
    if variant in ("bf16mv", "packed_bf16mv", "bf16mv_sr", "packed_bf16mv_sr"):
        return (18 + 2 * k) * n
    raise ValueError(variant)


# ------------------------------------------------ host (ZeRO-Offload) step

HOST_EXPORTS = ("zs_host_shard_step", "zs_host_max_threads", "zs_host_isa")
_host_lib = None


def load_host_library():
    """Load libzs_host.so (include/zs_host.h); raise if it is missing."""
    global _host_lib
    if _host_lib is not None:
        return _host_lib
    if not os.path.exists(HOST_LIB_PATH):
        raise ImportError("libzs_host.so is not built (expected at %s)" % HOST_LIB_PATH)
    lib = ctypes.CDLL(HOST_LIB_PATH)
    P = ctypes.c_void_p
    lib.zs_host_shard_step.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int64, P,
                                       ctypes.c_int32, P, ctypes.c_int64, ctypes.c_int]
    lib.zs_host_shard_step.restype = ctypes.c_int
    lib.zs_host_max_threads.argtypes = []
    lib.zs_host_max_threads.restype = ctypes.c_int
    lib.zs_host_isa.argtypes = []
    lib.zs_host_isa.restype = ctypes.c_char_p
    _host_lib = lib
    return lib


def host_segments(segs):
    """[(start, wd_on), ...] -> ctypes array of ZsSegment (host table)."""
    arr = (ZsSegment * len(segs))()
    for i, (st, f) in enumerate(segs):
        arr[i].start = int(st)
        arr[i].wd_on = 1 if f else 0
        arr[i].reserved = 0
    return arr


def zs_host_shard_step(master, m, v, param_bf16, grads, k, n, segs, hparams_, step,
                       nthreads=0, check=True) -> int:
    """Host shard step on host buffers (numpy arrays, CPU tensors or addresses).
    ``segs`` is a list of (start, wd_on) or a ZsSegment array."""
    nn = max(int(n), 0)
    k = _check_k(k, grads, "grads")
    gp = (ctypes.c_void_p * max(len(grads), 1))(
        *[_host(g, 2 * nn, "grads[%d]" % j) for j, g in enumerate(grads)])
    arr = segs if isinstance(segs, ctypes.Array) else host_segments(segs)
    rc = load_host_library().zs_host_shard_step(
        ctypes.c_void_p(_host(master, 4 * nn, "master")), ctypes.c_void_p(_host(m, 4 * nn, "m")),
        ctypes.c_void_p(_host(v, 4 * nn, "v")),
        ctypes.c_void_p(_host(param_bf16, 2 * nn, "param_bf16")), ctypes.cast(gp, ctypes.c_void_p),
        k, int(n), ctypes.cast(arr, ctypes.c_void_p), len(arr),
        ctypes.byref(hparams_), int(step), int(nthreads))
    if check and rc != ZS_OK:
        raise RuntimeError("zs_host_shard_step failed: %s (status %d)" % (
            zs_status_string(rc) if os.path.exists(LIB_PATH) else "", rc))
    return rc


def zs_host_max_threads() -> int:
    return load_host_library().zs_host_max_threads()


def zs_host_isa() -> str:
    return load_host_library().zs_host_isa().decode()
