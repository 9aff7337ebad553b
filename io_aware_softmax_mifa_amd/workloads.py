"""Seeded synthetic attention inputs shared by the kernel tests, the bench and the oracle checks.

This module only draws numbers.  It holds no attention arithmetic, so both the HIP path
and the CPU oracle can consume its tensors without sharing any of the method's code.

The workloads are synthetic stand-ins for the attention shapes the pages talk about
(long-context causal self-attention and the softmax over a triangular score matrix,
"Show HN: Flash Attention in ~100 lines of CUDA" and the FlashAttention-3 discussion on
Hacker News).  The pages print no dataset, so every tensor is i.i.d. noise with the stated
distribution, drawn in float32 from a seeded CPU generator and rounded to bfloat16 with
round-to-nearest-even.  Draw order is always Q, then K, then V from one generator.
"""
from __future__ import annotations

import dataclasses
import math

import torch

__all__ = ["Workload", "CONFIGS", "SHARD_CONFIGS", "by_name", "fp32_scale", "make_inputs", "sample_rows", "DecodeWorkload",
           "DECODE_CONFIGS", "decode_by_name", "make_rect_inputs", "SoftmaxWorkload",
           "SOFTMAX_CONFIGS", "softmax_by_name", "make_softmax_input", "sample_softmax_rows"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    seed: int
    # "normal": Q, K, V ~ N(0, 1).
    # "stress": Q, K ~ N(0, 2^2) (large logits), V ~ U(-1, 1).
    dist: str = "normal"
    # None: compare every output row with the oracle.  An int: compare that many seeded
    # sampled (b, h, i) rows.
    oracle_rows: int | None = None

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)


# The five seeded configurations; C1 and C2 run both with and without the causal mask.
CONFIGS = [
    Workload("C1-nc", 1, 1, 128, 64, False, 101),
    Workload("C1-c", 1, 1, 128, 64, True, 101),
    Workload("C2-nc", 4, 8, 1024, 64, False, 102),
    Workload("C2-c", 4, 8, 1024, 64, True, 102),
    Workload("C3", 2, 16, 4096, 128, True, 103),
    Workload("C4", 1, 32, 16384, 128, True, 104, oracle_rows=256),
    Workload("C5", 8, 16, 2048, 128, True, 105, dist="stress"),
]


# One GPU's share of C4 when its 32 heads are split over 8 GPUs with no communication (4 heads
# per GPU): what a single GPU shows of the head-sharded path.
SHARD_CONFIGS = [
    Workload("C4-shard", 1, 4, 16384, 128, True, 104, oracle_rows=128),
]


def by_name(name: str) -> Workload:
    for w in CONFIGS + SHARD_CONFIGS:
        if w.name == name:
            return w
    raise KeyError(name)


def fp32_scale(d: int) -> float:
    """1/sqrt(d) rounded to float32, returned as a Python float.

    The library takes the softmax scale as a float32, so this is the exact value both the
    kernel and the oracle use."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())


def make_inputs(B: int, H: int, N: int, d: int, seed: int, dist: str = "normal"):
    """Return bf16 CPU tensors q, k, v of shape [B, H, N, d], contiguous, d fastest."""
    g = torch.Generator().manual_seed(seed)
    shape = (B, H, N, d)
    if dist == "normal":
        q = torch.randn(shape, generator=g)
        k = torch.randn(shape, generator=g)
        v = torch.randn(shape, generator=g)
    elif dist == "stress":
        q = 2.0 * torch.randn(shape, generator=g)
        k = 2.0 * torch.randn(shape, generator=g)
        v = 2.0 * torch.rand(shape, generator=g) - 1.0
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return (q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16))


def make_workload_inputs(w: Workload):
    return make_inputs(w.B, w.H, w.N, w.d, w.seed, w.dist)


def sample_rows(B: int, H: int, N: int, count: int, seed: int) -> torch.Tensor:
    """Distinct seeded (b, h, i) query rows, as an int64 tensor of shape [count, 3].

    The edge rows i in {0, 1, 127, 128, N-1} of one seeded head are always included (those
    that exist); the rest are drawn uniformly without replacement from all B*H*N rows."""
    g = torch.Generator().manual_seed(seed + 1000)
    total = B * H * N
    count = min(count, total)
    head = int(torch.randint(0, B * H, (1,), generator=g).item())
    edge = sorted({i for i in (0, 1, 127, 128, N - 1) if 0 <= i < N})
    chosen = [head * N + i for i in edge][:count]
    taken = set(chosen)
    perm = torch.randperm(total, generator=g)
    for flat in perm.tolist():
        if len(chosen) >= count:
            break
        if flat not in taken:
            taken.add(flat)
            chosen.append(flat)
    flat = torch.tensor(chosen, dtype=torch.int64)
    bh, i = flat // N, flat % N
    return torch.stack([bh // H, bh % H, i], dim=1)


# ---- row-softmax workloads -------------------------------------------------------------------
# Stand-ins for the score rows the online-softmax trick normalises: a row is one query's
# scores over the keys, i.i.d. normal with the stated standard deviation (1 for unit-scale
# logits, 4 for the large-logit case), drawn in float32 from a seeded CPU generator and, for
# bf16, rounded to nearest even.

@dataclasses.dataclass(frozen=True)
class SoftmaxWorkload:
    name: str
    rows: int
    cols: int
    dtype: str     # "bf16" or "f32"
    std: float
    seed: int
    scale: float = 1.0

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def element_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


SOFTMAX_CONFIGS = [
    # the score matrix of the B=8 H=16 N=2048 attention (rows = B*H*N queries, cols = N keys)
    SoftmaxWorkload("SM1", 8 * 16 * 2048, 2048, "bf16", 1.0, 201),
    # the longest rows kept in registers, large logits
    SoftmaxWorkload("SM2", 4096, 32768, "bf16", 4.0, 202),
    # long rows, fp32
    SoftmaxWorkload("SM3", 4096, 16384, "f32", 2.0, 203),
    # short rows whose length is no multiple of 16 bytes (element loads), fp32
    SoftmaxWorkload("SM4", 65536, 1001, "f32", 1.0, 204),
    # rows longer than LDS holds (streamed: read twice)
    SoftmaxWorkload("SM5", 1024, 131072, "bf16", 1.0, 205),
]


def softmax_by_name(name: str) -> SoftmaxWorkload:
    for w in SOFTMAX_CONFIGS:
        if w.name == name:
            return w
    raise KeyError(name)


def make_softmax_input(rows: int, cols: int, dtype: str, std: float, seed: int) -> torch.Tensor:
    """A [rows, cols] CPU tensor of i.i.d. N(0, std^2) values in bf16 or fp32."""
    g = torch.Generator().manual_seed(seed)
    x = std * torch.randn((rows, cols), generator=g)
    return x.to(torch.bfloat16 if dtype == "bf16" else torch.float32)


def sample_softmax_rows(rows: int, count: int, seed: int) -> torch.Tensor:
    """Distinct seeded row indices (always including the first and last row), int64."""
    g = torch.Generator().manual_seed(seed + 2000)
    count = min(count, rows)
    chosen = sorted({0, rows - 1})[:count]
    taken = set(chosen)
    for r in torch.randperm(rows, generator=g).tolist():
        if len(chosen) >= count:
            break
        if r not in taken:
            taken.add(r)
            chosen.append(r)
    return torch.tensor(chosen, dtype=torch.int64)


# ---- few queries against many keys (decoding with a key/value cache) ---------------------------
# The pages give no decoding workload; these stand in for it: the newest Nq positions of a
# sequence of Nk cached keys, i.i.d. N(0, 1) like the square configurations.

@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    seed: int
    dist: str = "normal"


DECODE_CONFIGS = [
    # one new token per sequence, 16 sequences of 8 heads with 32K cached keys
    DecodeWorkload("D1", 16, 8, 1, 32768, 128, True, 301),
    # a 16-token chunk (speculative / chunked decoding) against 16K keys, 32 heads
    DecodeWorkload("D2", 1, 32, 16, 16384, 128, True, 302),
]


def decode_by_name(name: str) -> DecodeWorkload:
    for w in DECODE_CONFIGS:
        if w.name == name:
            return w
    raise KeyError(name)


def make_rect_inputs(B: int, H: int, Nq: int, Nk: int, d: int, seed: int, dist: str = "normal"):
    """bf16 CPU tensors q [B, H, Nq, d], k and v [B, H, Nk, d]; drawn like make_inputs."""
    g = torch.Generator().manual_seed(seed)
    sq, skv = (B, H, Nq, d), (B, H, Nk, d)
    if dist == "normal":
        q = torch.randn(sq, generator=g)
        k = torch.randn(skv, generator=g)
        v = torch.randn(skv, generator=g)
    elif dist == "stress":
        q = 2.0 * torch.randn(sq, generator=g)
        k = 2.0 * torch.randn(skv, generator=g)
        v = 2.0 * torch.rand(skv, generator=g) - 1.0
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return (q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16))


def make_grad_output(B: int, H: int, Nq: int, d: int, seed: int) -> torch.Tensor:
    """bf16 CPU tensor dO [B, H, Nq, d] ~ N(0, 1): the upstream gradient of a backward pass."""
    g = torch.Generator().manual_seed(seed + 7919)
    return torch.randn((B, H, Nq, d), generator=g).to(torch.bfloat16)


def sample_rows_in_heads(B: int, H: int, N: int, heads: int, per_head: int, seed: int) -> torch.Tensor:
    """Seeded (b, h, i) rows confined to `heads` distinct (b, h) pairs, `per_head` rows each,
    always including i in {0, 1, 127, 128, N-1} (those that exist).  For checks whose cost
    grows with the number of distinct heads (key-side gradients need a whole head)."""
    g = torch.Generator().manual_seed(seed + 2000)
    pairs = torch.randperm(B * H, generator=g)[:heads].tolist()
    out = []
    for ph in pairs:
        b, h = divmod(ph, H)
        edges = [i for i in (0, 1, 127, 128, N - 1) if i < N]
        rest = [i for i in torch.randperm(N, generator=g).tolist() if i not in edges]
        chosen = sorted(set(edges + rest[: max(0, per_head - len(edges))]))
        out.extend((b, h, i) for i in chosen)
    return torch.tensor(out, dtype=torch.int64)
