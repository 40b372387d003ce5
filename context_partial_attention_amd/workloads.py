"""Seeded synthetic workloads: shapes and random draws only.

This module holds no step of the method: it defines the five workload shapes
and draws their random inputs (sequence lengths, Q/K/V values, the shuffled
order of physical cache blocks). Both the HIP path and the CPU oracle consume
the tensors it returns; neither is imported here.

Recipe (every workload):
  * Lengths are drawn first from a CPU torch.Generator seeded with `seed`
    (integers uniform on the inclusive range, via randint(lo, hi + 1)).
  * Sequence b draws from its own generator seeded with seed * 1_000_003 + b,
    on the device the caller names: K [L, hkv, d], then V [L, hkv, d], then Q
    for the query positions of the workload, each fp32 N(0, 1) and then cast
    to the workload dtype (bf16 casts round to nearest even). Values therefore
    depend on the device they were drawn on; callers pass the same tensors to
    both sides.
  * The physical order of a rank's cache blocks is a permutation drawn from a
    CPU generator seeded with seed * 1_000_003 + 500_000 + rank.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "pass_kv" | "pass_q" | "decode"
    seed: int
    hq: int
    hkv: int
    d: int
    dtype: torch.dtype
    cp: int
    rank: int
    batch: int
    lengths: tuple = ()  # fixed lengths, or empty when drawn from len_range
    len_range: tuple = ()  # inclusive (lo, hi)
    cached: int = 0  # pass_q: cached tokens per sequence
    new: int = 0  # pass_q: new (query) tokens per sequence
    interleave: int = 0  # round-robin group size (pass_q, decode)
    block_size: int = 16
    description: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)


WORKLOADS = {
    w.name: w
    for w in [
        Workload(
            "tiny_prefill_cp2", "pass_kv", seed=0, hq=8, hkv=2, d=64, dtype=torch.float32, cp=2, rank=0, batch=1,
            lengths=(256,),
            description="1 sequence of 256 tokens, zigzag into 4 chunks of 64, rank 0 (chunks 0 and 3), "
                        "2 pass-KV steps, fp32, 8/2 heads, d=64",
        ),
        Workload(
            "qwen2.5_3b_cp2_rank0", "pass_kv", seed=1, hq=16, hkv=2, d=128, dtype=torch.bfloat16, cp=2, rank=0,
            batch=4, len_range=(2048, 8192),
            description="4 sequences, lengths uniform in [2048, 8192], zigzag into 4 chunks, rank 0, "
                        "2 pass-KV steps + 2-way merge, bf16, 16/2 heads, d=128",
        ),
        Workload(
            "llama3_8b_128k_cp4_rank1", "pass_kv", seed=2, hq=32, hkv=8, d=128, dtype=torch.bfloat16, cp=4, rank=1,
            batch=1, lengths=(131072,),
            description="1 sequence of 131072 tokens, zigzag into 8 chunks of 16384, rank 1 (chunks 1 and 6), "
                        "4 pass-KV steps + 4-way merge, bf16, 32/8 heads, d=128",
        ),
        Workload(
            "chunked_prefill_passq_cp4", "pass_q", seed=3, hq=16, hkv=2, d=128, dtype=torch.bfloat16, cp=4, rank=0,
            batch=2, cached=65536, new=4096, interleave=8,
            description="2 sequences of 65536 cached + 4096 new tokens, KV round-robin over 4 ranks "
                        "(interleave 8, 16-token blocks, shuffled block table), 8192 queries against each "
                        "rank's paged shard + 4-way merge, bf16, 16/2 heads, d=128",
        ),
        Workload(
            "allgather_decode_cp2", "decode", seed=4, hq=32, hkv=8, d=128, dtype=torch.bfloat16, cp=2, rank=0,
            batch=256, len_range=(8192, 32768), interleave=8,
            description="256 sequences, 1 query each, context uniform in [8192, 32768], KV round-robin over 2 "
                        "ranks (interleave 8, 16-token blocks, shuffled block table), local partial + 2-way "
                        "merge, bf16, 32/8 heads, d=128",
        ),
    ]
}


def seq_lengths(w: Workload) -> list[int]:
    """Total (KV) length of every sequence of the workload."""
    if w.kind == "pass_q":
        return [w.cached + w.new] * w.batch
    if w.lengths:
        return list(w.lengths)
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    lo, hi = w.len_range
    return [int(x) for x in torch.randint(lo, hi + 1, (w.batch,), generator=g)]


def _gen(device, seed: int) -> torch.Generator:
    return torch.Generator(device=torch.device(device)).manual_seed(seed)


def draw_sequence(w: Workload, b: int, L: int, q_rows: int, device="cpu"):
    """Draws (q, k, v) for sequence b: k, v [L, hkv, d] and q [q_rows, hq, d] for
    the workload's query positions (the last q_rows positions of the sequence)."""
    g = _gen(device, w.seed * 1_000_003 + b)
    k = torch.randn((L, w.hkv, w.d), generator=g, device=device, dtype=torch.float32).to(w.dtype)
    v = torch.randn((L, w.hkv, w.d), generator=g, device=device, dtype=torch.float32).to(w.dtype)
    q = torch.randn((q_rows, w.hq, w.d), generator=g, device=device, dtype=torch.float32).to(w.dtype)
    return q, k, v


def query_rows(w: Workload, L: int) -> int:
    """How many trailing positions of a length-L sequence carry queries."""
    if w.kind == "pass_kv":
        return L
    if w.kind == "pass_q":
        return w.new
    return 1


def block_permutation(w: Workload, n_blocks: int, rank: int) -> torch.Tensor:
    """Physical block order of `rank`'s cache pool (int64 permutation on the CPU)."""
    g = _gen("cpu", w.seed * 1_000_003 + 500_000 + rank)
    return torch.randperm(n_blocks, generator=g)


def scaled(w: Workload, **changes) -> Workload:
    """A copy of `w` with some fields changed (for smaller test variants)."""
    d = {f: getattr(w, f) for f in w.__dataclass_fields__}
    d.update(changes)
    return Workload(**d)
