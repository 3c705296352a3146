"""Byte accounting for mixed-precision AdamW under ZeRO sharding.

TEST INFRASTRUCTURE ONLY (part of the oracle package).

Sources:
  * "Chapter 9: Distributed Training and Data Parallelism", section 9.1.1
    (parameter count N ~ n_layers * (12 d^2 + 5 d)), section 9.2.1 (static
    memory of a 175B model), section 9.4.2 (per-GPU memory of ZeRO-1/2/3:
    4 Psi + 12 Psi/Nd, 2 Psi + 14 Psi/Nd, 16 Psi/Nd).
  * "Lecture 7: Parallelism I -- collectives, data parallelism and ZeRO"
    (CS336 notes), section 7 (five copies, 16 bytes per parameter) and
    exercise 6 (100B parameters on 64 GPUs).
"""
from __future__ import annotations

# bytes per parameter of each copy under mixed-precision AdamW
BF16_PARAM = 2
BF16_GRAD = 2
FP32_MASTER = 4
FP32_M = 4
FP32_V = 4


def bytes_per_param() -> int:
    """Total state bytes per parameter: bf16 weight + bf16 grad + fp32 master, m, v."""
    return BF16_PARAM + BF16_GRAD + FP32_MASTER + FP32_M + FP32_V


def optimizer_state_bytes_per_param() -> int:
    return FP32_MASTER + FP32_M + FP32_V


def transformer_params(n_layers: int, d_model: int) -> int:
    """N ~ n_layers * (12 d^2 + 5 d): 4 d^2 attention, 8 d^2 + 5 d MLP (d_ff = 4 d)."""
    return n_layers * (12 * d_model * d_model + 5 * d_model)


def ddp_bytes_per_gpu(psi: float) -> float:
    return bytes_per_param() * psi


def zero1_bytes_per_gpu(psi: float, nd: int) -> float:
    return (BF16_PARAM + BF16_GRAD) * psi + optimizer_state_bytes_per_param() * psi / nd


def zero2_bytes_per_gpu(psi: float, nd: int) -> float:
    return BF16_PARAM * psi + (BF16_GRAD + optimizer_state_bytes_per_param()) * psi / nd


def zero3_bytes_per_gpu(psi: float, nd: int) -> float:
    return bytes_per_param() * psi / nd


def shard_step_hbm_bytes_per_param(k: int) -> int:
    """Bytes one fused shard step moves per parameter with k bf16 partials.

    Reads the three fp32 state words (12 B) and k bf16 partials (2k B);
    writes the three fp32 state words (12 B) and the bf16 parameter (2 B).
    """
    return 3 * 4 + 2 * k + 3 * 4 + 2


def shard_resident_bytes_per_param(k: int) -> int:
    """Device-resident bytes per shard parameter: 12 B state, 2 B param, 2k B partials."""
    return 3 * 4 + 2 + 2 * k
