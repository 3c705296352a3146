"""The Python binding refuses buffers that would send a host address to the
GPU kernel (or a device address to the host step), and buffers too small for
n, before anything reaches the C library (CPU only: no call gets that far)."""
import numpy as np
import pytest

import sharded_mixed_precision_shard_amd as zs


class FakeGpuTensor:
    """Stands in for a device tensor: the binding only asks these questions.
    Its address is null, so even a check that wrongly let it through would
    meet the library's null-pointer error, never a kernel launch."""

    def __init__(self, nbytes, contiguous=True, addr=0):
        self._n, self._c, self._a = nbytes, contiguous, addr
        self.is_cuda = True
        self.device = "cuda:0"

    def data_ptr(self):
        return self._a

    def is_contiguous(self):
        return self._c

    def numel(self):
        return self._n

    def element_size(self):
        return 1


N = 1000
HP = zs.hparams()


def _dev_args(**over):
    a = dict(master=FakeGpuTensor(4 * N), m=FakeGpuTensor(4 * N), v=FakeGpuTensor(4 * N),
             param=FakeGpuTensor(2 * N), grads=[FakeGpuTensor(2 * N), FakeGpuTensor(2 * N)],
             table=FakeGpuTensor(16))
    a.update(over)
    return a


def _call(**over):
    a = _dev_args(**over)
    return zs.zs_shard_step(a["master"], a["m"], a["v"], a["param"], a["grads"], 2, N,
                            zs.seg_table(a["table"], 1), HP, 1)


def test_host_arrays_are_refused_by_the_gpu_entry_points():
    with pytest.raises(TypeError, match="host"):
        _call(master=np.zeros(N, np.float32))
    with pytest.raises(TypeError, match="host"):
        _call(grads=[FakeGpuTensor(2 * N), np.zeros(N, np.uint16)])
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError, match="GPU tensor"):
        _call(v=torch.zeros(N))
    with pytest.raises(ValueError, match="GPU tensor"):
        zs.seg_table(torch.zeros(1, 2, dtype=torch.int64))


def test_short_or_strided_device_buffers_are_refused():
    with pytest.raises(ValueError, match="master holds"):
        _call(master=FakeGpuTensor(4 * N - 4))
    with pytest.raises(ValueError, match=r"grads\[1\] holds"):
        _call(grads=[FakeGpuTensor(2 * N), FakeGpuTensor(2 * N - 2)])
    with pytest.raises(ValueError, match="contiguous"):
        _call(m=FakeGpuTensor(4 * N, contiguous=False))
    with pytest.raises(ValueError, match="segment table"):
        zs.seg_table(FakeGpuTensor(16), 2)
    # a count the library refuses by itself is passed through (nothing is read)
    assert zs.seg_table(FakeGpuTensor(16), zs.ZS_MAX_SEGMENTS + 1).count == \
        zs.ZS_MAX_SEGMENTS + 1


def test_variant_buffers_are_sized_by_their_own_types():
    a = _dev_args()
    nb = -(-N // zs.ZS_Q8_BLOCK)
    with pytest.raises(ValueError, match="param_q8 holds"):
        zs.zs_shard_step_q8ag(a["master"], a["m"], a["v"], a["param"], FakeGpuTensor(N - 1),
                              FakeGpuTensor(4 * nb), a["grads"], 2, N,
                              zs.seg_table(a["table"], 1), HP, 1)
    with pytest.raises(ValueError, match="param_q8_scale holds"):
        zs.zs_shard_step_q8ag(a["master"], a["m"], a["v"], a["param"], FakeGpuTensor(N),
                              FakeGpuTensor(4 * nb - 4), a["grads"], 2, N,
                              zs.seg_table(a["table"], 1), HP, 1)
    with pytest.raises(ValueError, match=r"qscales\[0\] holds"):
        zs.zs_shard_step_q8grad(a["master"], a["m"], a["v"], a["param"], [FakeGpuTensor(N)],
                                [FakeGpuTensor(4 * nb - 1)], 1, N,
                                zs.seg_table(a["table"], 1), HP, 1)
    # bf16 moments need 2 bytes per element, not 4
    with pytest.raises(ValueError, match="v holds"):
        zs.zs_shard_step_bf16mv(a["master"], FakeGpuTensor(2 * N), FakeGpuTensor(2 * N - 1),
                                a["param"], a["grads"], 2, N, zs.seg_table(a["table"], 1), HP, 1)


def test_host_step_refuses_device_and_short_buffers():
    w, m, v = (np.zeros(N, np.float32) for _ in range(3))
    p = np.zeros(N, np.uint16)
    g = [np.zeros(N, np.uint16)]
    with pytest.raises(ValueError, match="GPU tensor"):
        zs.zs_host_shard_step(FakeGpuTensor(4 * N), m, v, p, g, 1, N, [(0, True)], HP, 1)
    with pytest.raises(ValueError, match="m holds"):
        zs.zs_host_shard_step(w, np.zeros(N - 1, np.float32), v, p, g, 1, N, [(0, True)], HP, 1)
    with pytest.raises(ValueError, match="contiguous"):
        zs.zs_host_shard_step(w, m, np.zeros(2 * N, np.float32)[::2], p, g, 1, N, [(0, True)],
                              HP, 1)
    assert zs.zs_host_shard_step(w, m, v, p, g, 1, N, [(0, True)], HP, 1) == zs.ZS_OK


def test_prepared_call_checks_once_at_construction():
    a = _dev_args()
    with pytest.raises(TypeError, match="host"):
        zs.ShardStep(np.zeros(N, np.float32), a["m"], a["v"], a["param"], a["grads"], N,
                     zs.seg_table(a["table"], 1), HP)
    with pytest.raises(ValueError, match="m holds"):
        zs.ShardStep(a["master"], FakeGpuTensor(2 * N), a["v"], a["param"], a["grads"], N,
                     zs.seg_table(a["table"], 1), HP)
    # bf16 moments take 2 bytes per element
    zs.ShardStep(a["master"], FakeGpuTensor(2 * N), FakeGpuTensor(2 * N), a["param"],
                 a["grads"], N, zs.seg_table(a["table"], 1), HP, variant="bf16mv")
    with pytest.raises(ValueError, match="one scale array"):
        zs.ShardStep(a["master"], a["m"], a["v"], a["param"], [FakeGpuTensor(N)] * 2, N,
                     zs.seg_table(a["table"], 1), HP, variant="q8grad",
                     qscales=[FakeGpuTensor(16)])
    with pytest.raises(ValueError, match="unknown variant"):
        zs.ShardStep(a["master"], a["m"], a["v"], a["param"], a["grads"], N,
                     zs.seg_table(a["table"], 1), HP, variant="fp8")
    with pytest.raises(ValueError, match="base entry point only"):
        zs.ShardStep(a["master"], FakeGpuTensor(2 * N), FakeGpuTensor(2 * N), a["param"],
                     a["grads"], N, zs.seg_table(a["table"], 1), HP, variant="bf16mv",
                     cfg=dict(chunk_tiles=2))


def test_k_must_match_the_number_of_partials():
    """An explicit k that differs from the number of partial pointers is
    refused in Python: the library would read k pointers from the array."""
    a = _dev_args()
    st = zs.seg_table(a["table"], 1)
    f = (a["master"], a["m"], a["v"], a["param"])
    for k in (1, 3, 16):
        with pytest.raises(ValueError, match="k=%d but 2 grads" % k):
            zs.zs_shard_step(*f, a["grads"], k, N, st, HP, 1)
        with pytest.raises(ValueError, match="k=%d but 2 grads" % k):
            zs.zs_shard_step_cfg(*f, a["grads"], k, N, st, HP, 1, chunk_tiles=2)
        with pytest.raises(ValueError, match="k=%d but 2 grads" % k):
            zs.zs_shard_step_q8ag(*f, FakeGpuTensor(N), FakeGpuTensor(16), a["grads"], k, N,
                                  st, HP, 1)
        with pytest.raises(ValueError, match="k=%d but 2 grads" % k):
            zs.zs_shard_step_bf16mv(a["master"], FakeGpuTensor(2 * N), FakeGpuTensor(2 * N),
                                    a["param"], a["grads"], k, N, st, HP, 1)
    q = [FakeGpuTensor(N), FakeGpuTensor(N)]
    s = [FakeGpuTensor(16), FakeGpuTensor(16)]
    with pytest.raises(ValueError, match="k=3 but 2 qgrads"):
        zs.zs_shard_step_q8grad(*f, q, s, 3, N, st, HP, 1)
    with pytest.raises(ValueError, match="1 qscales for 2 qgrads"):
        zs.zs_shard_step_q8grad(*f, q, s[:1], 2, N, st, HP, 1)
    with pytest.raises(ValueError, match="3 qscales for 2 qgrads"):
        zs.zs_shard_step_q8grad(*f, q, s + s[:1], None, N, st, HP, 1)
    # the host step: plain integer host addresses, never dereferenced here
    with pytest.raises(ValueError, match="k=2 but 1 grads"):
        zs.zs_host_shard_step(4096, 4096, 4096, 4096, [4096], 2, 16, [(0, True)], HP, 1)
    # k=None takes the list's length; k=0 with no partials reaches the
    # library, which refuses k=0 itself
    w, m, v = (np.zeros(N, np.float32) for _ in range(3))
    p = np.zeros(N, np.uint16)
    assert zs.zs_host_shard_step(w, m, v, p, [], 0, N, [(0, True)], HP, 1, check=False) == \
        zs.ZS_ERR_INVALID_ARGUMENT
    assert zs.zs_host_shard_step(w, m, v, p, [np.zeros(N, np.uint16)], None, N, [(0, True)],
                                 HP, 1) == zs.ZS_OK


def test_packed_entry_points_check_their_buffers():
    """zs_shard_step_packed sizes the state as ZS_PACKED_FLOATS(n) floats and
    refuses host buffers; the conversions check all four buffers; the packed
    ShardStep takes no separate m or v."""
    nf = zs.packed_floats(N)
    assert nf == 768 * 4  # 1000 elements: four 256-element blocks
    st = zs.seg_table(FakeGpuTensor(16), 1)
    g = [FakeGpuTensor(2 * N), FakeGpuTensor(2 * N)]
    with pytest.raises(ValueError, match="state holds"):
        zs.zs_shard_step_packed(FakeGpuTensor(4 * 3 * N), FakeGpuTensor(2 * N), g, 2, N, st,
                                HP, 1)
    with pytest.raises(TypeError, match="host"):
        zs.zs_shard_step_packed(np.zeros(nf, np.float32), FakeGpuTensor(2 * N), g, 2, N, st,
                                HP, 1)
    with pytest.raises(ValueError, match="k=3 but 2 grads"):
        zs.zs_shard_step_packed(FakeGpuTensor(4 * nf), FakeGpuTensor(2 * N), g, 3, N, st, HP, 1)
    with pytest.raises(ValueError, match="state holds"):
        zs.zs_pack_state(FakeGpuTensor(4 * N), FakeGpuTensor(4 * N), FakeGpuTensor(4 * N),
                         FakeGpuTensor(4 * nf - 4), N)
    with pytest.raises(ValueError, match="m holds"):
        zs.zs_unpack_state(FakeGpuTensor(4 * nf), FakeGpuTensor(4 * N), FakeGpuTensor(4 * N - 4),
                           FakeGpuTensor(4 * N), N)
    with pytest.raises(TypeError, match="host"):
        zs.zs_pack_state(np.zeros(N, np.float32), FakeGpuTensor(4 * N), FakeGpuTensor(4 * N),
                         FakeGpuTensor(4 * nf), N)
    with pytest.raises(ValueError, match="inside the state"):
        zs.ShardStep(FakeGpuTensor(4 * nf), FakeGpuTensor(4 * N), None, FakeGpuTensor(2 * N),
                     g, N, st, HP, variant="packed")
    assert zs.algorithmic_bytes("packed", 2, N) == zs.algorithmic_bytes("base", 2, N)
    assert zs.algorithmic_bytes("packed_q8ag", 2, N) == zs.algorithmic_bytes("q8ag", 2, N)
    assert zs.algorithmic_bytes("packed_q8grad", 2, N) == zs.algorithmic_bytes("q8grad", 2, N)
    q = [FakeGpuTensor(N), FakeGpuTensor(N)]
    with pytest.raises(ValueError, match="2 qscales for 2 qgrads|1 qscales for 2 qgrads"):
        zs.zs_shard_step_packed_q8grad(FakeGpuTensor(4 * nf), FakeGpuTensor(2 * N), q,
                                       [FakeGpuTensor(16)], 2, N, st, HP, 1)
    with pytest.raises(ValueError, match="state holds"):
        zs.zs_shard_step_packed_q8ag(FakeGpuTensor(4 * N), FakeGpuTensor(2 * N),
                                     FakeGpuTensor(N), FakeGpuTensor(16), g, 2, N, st, HP, 1)
    assert zs.ZS_VARIANT["packed"] == 16
    # the bf16-moment state: 2 KB per 256-element block
    nf16 = zs.packed_bf16mv_floats(N)
    assert nf16 == 512 * 4 and zs.ZS_VARIANT["packed_bf16mv"] == 20
    assert zs.algorithmic_bytes("packed_bf16mv", 2, N) == zs.algorithmic_bytes("bf16mv", 2, N)
    with pytest.raises(ValueError, match="state holds"):
        zs.zs_shard_step_packed_bf16mv(FakeGpuTensor(4 * nf16 - 16), FakeGpuTensor(2 * N), g, 2,
                                       N, st, HP, 1)
    with pytest.raises(ValueError, match="m_bf16 holds"):
        zs.zs_pack_state_bf16mv(FakeGpuTensor(4 * N), FakeGpuTensor(2 * N - 2),
                                FakeGpuTensor(2 * N), FakeGpuTensor(4 * nf16), N)
    with pytest.raises(ValueError, match="state holds"):
        zs.zs_unpack_state_bf16mv(FakeGpuTensor(4 * nf16 - 4), FakeGpuTensor(4 * N),
                                  FakeGpuTensor(2 * N), FakeGpuTensor(2 * N), N)
    with pytest.raises(ValueError, match="inside the state"):
        zs.ShardStep(FakeGpuTensor(4 * nf16), None, FakeGpuTensor(2 * N), FakeGpuTensor(2 * N),
                     g, N, st, HP, variant="packed_bf16mv")
    with pytest.raises(ValueError, match="state holds"):
        zs.ShardStep(FakeGpuTensor(4 * nf16 - 4), None, None, FakeGpuTensor(2 * N), g, N, st,
                     HP, variant="packed_bf16mv")
    # stochastic rounding: the same buffers, plus an unsigned 64-bit seed
    assert zs.ZS_VARIANT["bf16mv_sr"] == 36 and zs.ZS_VARIANT["packed_bf16mv_sr"] == 52
    assert zs.algorithmic_bytes("bf16mv_sr", 2, N) == zs.algorithmic_bytes("bf16mv", 2, N)
    assert zs.algorithmic_bytes("packed_bf16mv_sr", 2, N) == zs.algorithmic_bytes("bf16mv", 2, N)
    with pytest.raises(ValueError, match="unsigned 64-bit"):
        zs.zs_shard_step_packed_bf16mv_sr(FakeGpuTensor(4 * nf16), FakeGpuTensor(2 * N), g, 2, N,
                                          st, HP, 1, -5)
    with pytest.raises(ValueError, match="m holds"):
        zs.zs_shard_step_bf16mv_sr(FakeGpuTensor(4 * N), FakeGpuTensor(2 * N - 2),
                                   FakeGpuTensor(2 * N), FakeGpuTensor(2 * N), g, 2, N, st, HP, 1,
                                   7)
    with pytest.raises(ValueError, match="needs a seed"):
        zs.ShardStep(FakeGpuTensor(4 * nf16), None, None, FakeGpuTensor(2 * N), g, N, st, HP,
                     variant="packed_bf16mv_sr")
