"""Pins of the oracle's block int8 quantizer (quantized all-gather payload).

"Chapter 9: Distributed Training and Data Parallelism", section 9.4.3 (ZeRO++):
16-bit weights become INT8 before the all-gather, roughly halving its volume,
and are dequantized after it; quantization is block-wise.  Pins: exact ties
and special blocks worked by hand, the rounding error bound, the extreme
element landing on +-127, the volume claim, and a torch cross-check.
"""
import numpy as np
import pytest

import oracle

F32 = np.float32


def _bf16(vals):
    f = np.asarray(vals, F32)
    h = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_to_f32(h), f)
    return h


def test_hand_worked_block_with_ties():
    """a = 127 -> scale = 1 exactly; halves round to even."""
    x = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, 126.5, -127.0, 0.0]
    q, s = oracle.q8_blocks(_bf16(x), block=16)
    assert s.tolist() == [1.0]
    assert q.tolist() == [127, 2, 4, -2, -4, 0, 2, 126, -127, 0]


def test_zero_block_and_single_element():
    q, s = oracle.q8_blocks(_bf16([0.0] * 8 + [0.0] * 7 + [-3.0]), block=8)
    assert s[0] == 0.0 and not q[:8].any()
    assert s[1] == F32(3.0) / F32(127.0) and q[15] == -127 and not q[8:15].any()


def test_nonfinite_blocks_only_poison_themselves():
    x = np.zeros(12, F32)
    x[:4] = [1.0, np.nan, 2.0, 3.0]
    x[4:8] = [1.0, np.inf, 2.0, -1.0]
    x[8:12] = [1.0, -2.0, 0.5, 4.0]
    q, s = oracle.q8_blocks((x.view(np.uint32) >> 16).astype(np.uint16), block=4)
    assert np.isnan(s[0]) and not q[:4].any()
    assert np.isinf(s[1]) and not q[4:8].any()
    assert s[2] == F32(4.0) / F32(127.0)
    assert q[8:12].tolist() == [32, -64, 16, 127]  # 1/(4/127) = 31.75 -> 32, etc.


@pytest.mark.parametrize("block", [1, 7, 64, 256])
def test_error_bound_and_extremes(block):
    """|x - q*s| <= s/2 (plus the binary32 rounding of x/s and of q*s), the
    block maximum maps to +-127, signs agree, ragged last block."""
    rng = np.random.default_rng(block)
    n = 10_000 + 37
    x = (rng.standard_normal(n) * rng.choice([1e-6, 1e-2, 3.0], n)).astype(F32)
    h = (x.view(np.uint32) >> 16).astype(np.uint16)
    xf = oracle.bf16_to_f32(h).astype(np.float64)
    q, s = oracle.q8_blocks(h, block=block)
    assert s.shape[0] == -(-n // block)
    xh = oracle.q8_dequant(q, s, block).astype(np.float64)
    sb = np.repeat(s.astype(np.float64), block)[:n]
    assert np.all(np.abs(xf - xh) <= sb * (0.5 + 1e-6) + np.abs(xf) * 2e-7)
    assert np.all((np.sign(q) == np.sign(xf)) | (q == 0))
    for b in range(s.shape[0]):
        blk = xf[b * block:(b + 1) * block]
        qb = q[b * block:(b + 1) * block]
        if np.abs(blk).max() > 0:
            assert np.abs(qb).max() == 127
            assert qb[np.argmax(np.abs(blk))] == 127 * np.sign(blk[np.argmax(np.abs(blk))])
            assert s[b] == F32(F32(np.abs(blk).max()) / F32(127.0))


def test_payload_is_about_half_of_bf16():
    """The page: INT8 halves the 16-bit all-gather volume.  With one fp32
    scale per 256 elements the payload is (1 + 4/256) / 2 of the bf16 one."""
    n, block = 1 << 20, 256
    q, s = oracle.q8_blocks(np.zeros(n, np.uint16), block)
    ratio = (q.nbytes + s.nbytes) / (2 * n)
    assert abs(ratio - 0.5078125) < 1e-12


def test_matches_torch_elementwise_formula():
    """Library cross-check of the rounding: torch.round (half to even) of
    x / scale in float32, clamped, on blocks of 256."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    n = 256 * 40 + 100
    x = (rng.standard_normal(n) * 0.02).astype(F32)
    h = (x.view(np.uint32) >> 16).astype(np.uint16)
    q, s = oracle.q8_blocks(h, 256)
    xt = torch.from_numpy(oracle.bf16_to_f32(h).copy())
    nb = s.shape[0]
    pad = torch.zeros(nb * 256 - n)
    blocks = torch.cat([xt, pad]).view(nb, 256)
    st = blocks.abs().amax(dim=1) / 127.0
    qt = torch.clamp(torch.round(blocks / st[:, None]), -127, 127).to(torch.int8).view(-1)[:n]
    assert np.array_equal(st.numpy(), s)
    assert np.array_equal(qt.numpy(), q)
