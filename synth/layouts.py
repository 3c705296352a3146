"""Model-shaped flat buffers, their even split across ranks, and the seeded
workloads used by the tests and the benchmark.

Holds none of the optimizer's arithmetic.  Shapes follow the pages:
  * "Chapter 9: Distributed Training and Data Parallelism", section 9.1.1:
    per layer W_Q, W_K, W_V (d x d_head per head), W_O, and an MLP with
    d_ff = 4d and biases of size 4d and d, which gives 12 d^2 + 5 d per layer;
    GPT-3 175B has 96 layers with d = 12288.
  * "Lecture 7: Parallelism I", section 8.1 (FlatZeRO1: one flat vector split
    evenly into p parts) and exercise 1(e) (pad with zeros until the length
    divides by p).
Weight decay is on for weight matrices and embeddings and off for biases,
LayerNorm parameters and the zero padding.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

Tensor = Tuple[str, int, bool]  # (name, numel, weight decay on)


def transformer_12d2_layer(prefix: str, d: int, n_heads: int = 0) -> List[Tensor]:
    """One layer of 12 d^2 + 5 d parameters.  With n_heads > 0 the Q, K and V
    projections are split into one d x d_head piece per head."""
    out: List[Tensor] = []
    if n_heads > 0:
        dh = d // n_heads
        for proj in ("q", "k", "v"):
            for h in range(n_heads):
                out.append(("%s.w_%s.h%d" % (prefix, proj, h), d * dh, True))
    else:
        out += [(prefix + ".w_q", d * d, True), (prefix + ".w_k", d * d, True),
                (prefix + ".w_v", d * d, True)]
    out += [(prefix + ".w_o", d * d, True),
            (prefix + ".w_fc1", 4 * d * d, True), (prefix + ".b_fc1", 4 * d, False),
            (prefix + ".w_fc2", 4 * d * d, True), (prefix + ".b_fc2", d, False)]
    return out


def transformer_12d2(n_layers: int, d: int, n_heads: int = 0) -> List[Tensor]:
    out: List[Tensor] = []
    for layer in range(n_layers):
        out += transformer_12d2_layer("l%d" % layer, d, n_heads)
    return out


def gpt2_small(n_layers=12, d=768, vocab=50257, n_ctx=1024) -> List[Tensor]:
    """GPT-2-small parameter list, flattened blocks first (then ln_f, wpe, wte),
    so that rank 0 of 8 spans several tensors rather than the embedding only."""
    out: List[Tensor] = []
    for b in range(n_layers):
        p = "h%d" % b
        out += [(p + ".ln1.g", d, False), (p + ".ln1.b", d, False),
                (p + ".attn.w_qkv", 3 * d * d, True), (p + ".attn.b_qkv", 3 * d, False),
                (p + ".attn.w_o", d * d, True), (p + ".attn.b_o", d, False),
                (p + ".ln2.g", d, False), (p + ".ln2.b", d, False),
                (p + ".mlp.w_fc", 4 * d * d, True), (p + ".mlp.b_fc", 4 * d, False),
                (p + ".mlp.w_proj", 4 * d * d, True), (p + ".mlp.b_proj", d, False)]
    out += [("ln_f.g", d, False), ("ln_f.b", d, False),
            ("wpe", n_ctx * d, True), ("wte", vocab * d, True)]
    return out


@dataclass
class Shard:
    """Rank r's slice [index0, index0 + n) of the zero-padded flat buffer."""
    n: int               # elements in the shard
    index0: int          # flat index of the shard's first element
    valid_end: int       # flat index where the model ends and padding begins
    segments: List[Tuple[int, bool]]  # (start inside the shard, wd on), sorted
    total: int           # unpadded model size
    padded: int          # p * n


def shard_of(tensors: List[Tensor], p: int, rank: int) -> Shard:
    total = sum(t[1] for t in tensors)
    n = -(-total // p)
    padded = n * p
    lo, hi = rank * n, (rank + 1) * n
    segs: List[Tuple[int, bool]] = []
    a = 0
    for _, numel, wd in tensors:
        b = a + numel
        if b > lo and a < hi and numel > 0:
            segs.append((max(a, lo) - lo, wd))
        a = b
    if padded > total and hi > total:  # zero padding: one decay-free segment
        segs.append((max(total, lo) - lo, False))
    return Shard(n=n, index0=lo, valid_end=total, segments=segs, total=total, padded=padded)


def clip_segments(segments, lo, hi):
    """The shard's table restricted to window [lo, hi), rebased to lo."""
    out = []
    for i, (s, f) in enumerate(segments):
        e = segments[i + 1][0] if i + 1 < len(segments) else None
        if (e is None or e > lo) and s < hi:
            out.append((max(s, lo) - lo, f))
    # collapse entries that all start at 0 to the last one (same lookup result)
    while len(out) > 1 and out[1][0] == 0:
        out.pop(0)
    return out


def decay_mask_full(tensors: List[Tensor], padded: int):
    """Per-element decay flag of the whole padded flat buffer (numpy uint8)."""
    import numpy as np
    mask = np.zeros(padded, dtype=np.uint8)
    a = 0
    for _, numel, wd in tensors:
        if wd:
            mask[a:a + numel] = 1
        a += numel
    return mask


@dataclass
class Workload:
    """A seeded synthetic shard-step workload."""
    name: str
    tensors: List[Tensor]
    p: int
    rank: int
    k: int
    grad_sigma: float
    master_sigma: float
    lr: float
    beta1: float
    beta2: float
    eps: float
    weight_decay: float
    steps: int
    t0: int = 1               # optimizer step of the first measured step
    prewarm_steps: int = 0    # steps at t = 1 .. prewarm_steps run beforehand
    heavy_p: float = 0.0      # probability that a partial element draws sigma = heavy_sigma
    heavy_sigma: float = 0.0
    seed: int = 0
    note: str = ""
    shard: Shard = field(init=False)

    def __post_init__(self):
        self.shard = shard_of(self.tensors, self.p, self.rank)

    def with_rank(self, rank: int) -> "Workload":
        import dataclasses
        return dataclasses.replace(self, rank=rank)

    @property
    def n(self) -> int:
        return self.shard.n

    def step_ts(self):
        return list(range(self.t0, self.t0 + self.steps))


SEED_BASE = 0x5A5A0000

_HP_SMALL = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
_HP_LARGE = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def workload(name: str) -> Workload:
    """The five shard workloads: tiny, gpt2-small, 7b, 175b, 70b."""
    if name == "tiny":
        return Workload("tiny: n=2^20 flat shard, 1 segment, k=4", [("flat", 1 << 20, True)],
                        p=1, rank=0, k=4, grad_sigma=0.01, master_sigma=0.02, steps=10,
                        seed=SEED_BASE + 0, **_HP_SMALL)
    if name == "gpt2-small":
        return Workload("GPT-2-small (12 layers, d=768) rank 0 of 8, k=8", gpt2_small(), p=8,
                        rank=0, k=8, grad_sigma=1e-3, master_sigma=0.02, steps=10,
                        seed=SEED_BASE + 1, **_HP_SMALL)
    if name == "7b":
        return Workload("7B-shaped (32 layers, d=4096) rank 0 of 8, k=8, 1% heavy tail, "
                        "m/v pre-warmed 100 steps", transformer_12d2(32, 4096), p=8, rank=0,
                        k=8, grad_sigma=1e-3, master_sigma=0.02, steps=10, t0=101,
                        prewarm_steps=100, heavy_p=0.01, heavy_sigma=1.0,
                        seed=SEED_BASE + 2, **_HP_LARGE)
    if name == "175b":
        return Workload("GPT-3-175B-shaped (96 layers, d=12288) rank 0 of 64, k=2",
                        transformer_12d2(96, 12288), p=64, rank=0, k=2, grad_sigma=1e-3,
                        master_sigma=0.02, steps=5, seed=SEED_BASE + 3, **_HP_LARGE)
    if name == "70b":
        return Workload("70B-shaped (80 layers, d=8192, 64 heads, per-head Q/K/V segments) "
                        "rank 0 of 8, k=2, t=10000", transformer_12d2(80, 8192, n_heads=64),
                        p=8, rank=0, k=2, grad_sigma=1e-3, master_sigma=0.02, steps=3,
                        t0=10000, seed=SEED_BASE + 4, **_HP_LARGE)
    raise KeyError("unknown workload %r" % name)


WORKLOADS = ("tiny", "gpt2-small", "7b", "175b", "70b")
