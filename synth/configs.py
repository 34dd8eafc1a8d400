"""The workloads the measurements and parity checks run on.

Shapes follow the pages' workloads (long causal sequences, head dim 128, 16-32
heads, 8-way sequence sharding); the values are synthetic (see ``synth``).
Assignment names: ``contiguous`` (rank r holds one run of L/N tokens),
``striped`` (token t on rank t mod N), ``zigzag`` (2N chunks, rank r holds
chunks r and 2N-1-r), ``ulysses`` (sequence-sharded input permuted to
head-sharded, then one full-sequence causal attention). ``usp_u4r2`` is one device of a USP
mesh (Ulysses degree u = 4 inside a group, zigzag ring of r = 2 groups, 128K tokens, as in the
pages' 8-GPU u=4, r=2 run): ``world`` and ``rank`` are the ring degree and ring rank,
``ulysses`` and ``ulysses_rank`` the Ulysses degree and the device's head group.
``gqa_zigzag_rank3`` is grouped-query attention with the head counts of the pages' GQA example
(64 query heads sharing 8 KV heads), on a 64K-token zigzag ring of 8. ``contig_rank7_256k`` and
``striped_rank7_256k`` are the heaviest ranks of the contiguous and striped assignments of the
headline's sequence (256K tokens over 8 ranks, 16 heads): the shares the pages' Striped Attention
comparison sets against each other.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    number: int            # seeds are 1000*number + {0,1,2}
    batch: int
    heads: int
    head_dim: int
    global_len: int
    world: int             # ring size N (or Ulysses degree P)
    rank: int              # the rank whose share is computed (-1: every rank)
    assign: str            # contiguous | striped | zigzag | ulysses
    causal: bool
    dtype: str             # "bf16" or "f32" (input and accumulation-state precision)
    qk_std: float = 1.0
    sampled_rows: int = 0  # 0: full oracle; else 512-row sampled check
    ulysses: int = 1       # USP: Ulysses degree u (the ring degree is `world`)
    ulysses_rank: int = 0  # USP: the device's Ulysses rank (its head group)
    kv_heads: int = 0      # K/V heads for grouped-query attention (0: as many as query heads)

    @property
    def heads_kv(self) -> int:
        return self.kv_heads or self.heads

    @property
    def share_len(self) -> int:
        return self.global_len // self.world


CONFIGS = {
    "tiny_exact": Workload("tiny_exact", 1, 1, 1, 64, 256, 4, -1, "contiguous", False, "f32"),
    "contig_rank7": Workload("contig_rank7", 2, 1, 32, 128, 8192, 8, 7, "contiguous", True, "bf16"),
    "striped_rank0": Workload("striped_rank0", 3, 1, 32, 128, 32768, 8, 0, "striped", True, "bf16"),
    "striped_rank0_std4": Workload("striped_rank0_std4", 3, 1, 32, 128, 32768, 8, 0, "striped", True,
                                   "bf16", qk_std=4.0),
    "ulysses_local": Workload("ulysses_local", 4, 1, 32, 128, 65536, 8, 0, "ulysses", True, "bf16",
                              sampled_rows=512),
    "zigzag_rank3": Workload("zigzag_rank3", 5, 1, 16, 128, 262144, 8, 3, "zigzag", True, "bf16",
                             sampled_rows=512),
    "usp_u4r2": Workload("usp_u4r2", 6, 1, 32, 128, 131072, 2, 1, "zigzag", True, "bf16",
                         sampled_rows=512, ulysses=4, ulysses_rank=2),
    "gqa_zigzag_rank3": Workload("gqa_zigzag_rank3", 7, 1, 64, 128, 65536, 8, 3, "zigzag", True, "bf16",
                                 sampled_rows=512, kv_heads=8),
    "contig_rank7_256k": Workload("contig_rank7_256k", 8, 1, 16, 128, 262144, 8, 7, "contiguous", True, "bf16",
                                  sampled_rows=512),
    "striped_rank7_256k": Workload("striped_rank7_256k", 9, 1, 16, 128, 262144, 8, 7, "striped", True, "bf16",
                                   sampled_rows=512),
}


def get(name: str) -> Workload:
    return CONFIGS[name]
