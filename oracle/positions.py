"""Token -> rank assignments: the global position of each local row of a share.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Each function returns, for ``rank``'s share of a global sequence of
``global_len`` tokens split over ``world`` ranks, the global token position of
local row 0, 1, 2, ... in that order. Local order is ascending global position
(the pages list every share in ascending order).
"""
from __future__ import annotations

import numpy as np

CONTIGUOUS, STRIPED, ZIGZAG = 0, 1, 2
NAMES = {"contiguous": CONTIGUOUS, "striped": STRIPED, "zigzag": ZIGZAG}


def _check(world: int, rank: int, global_len: int, parts: int) -> None:
    if world < 1 or not (0 <= rank < world):
        raise ValueError(f"bad world/rank {world}/{rank}")
    if global_len < 0 or global_len % parts:
        raise ValueError(f"global_len {global_len} not divisible into {parts} equal parts")


def contiguous(world: int, rank: int, global_len: int) -> np.ndarray:
    """Sequential split: rank r holds tokens [r*L/N, (r+1)*L/N).

    [Digest] §3.4 (contiguous split, the source of the causal imbalance) and the
    "original Ring Attention (contiguous)" listing in §4: GPU0 tokens 0-3,
    GPU1 4-7, ... for 16 tokens on 4 GPUs.
    """
    _check(world, rank, global_len, world)
    s = global_len // world
    return np.arange(rank * s, (rank + 1) * s, dtype=np.int64)


def striped(world: int, rank: int, global_len: int) -> np.ndarray:
    """Striped split: token t goes to rank t mod N ([Digest] §4, striped listing:
    GPU0 holds 0, 4, 8, 12 of 16 tokens on 4 GPUs)."""
    _check(world, rank, global_len, world)
    # the tokens t with t mod N == r, in ascending order: r, r + N, r + 2N, ...
    return np.arange(rank, global_len, world, dtype=np.int64)


def zigzag(world: int, rank: int, global_len: int) -> np.ndarray:
    """Zigzag split ([Digest] §6 item 1): the sequence is cut into 2*cp equal
    blocks and rank k holds block k and block 2*cp-1-k.

    Reading: the page's cp=4 example says "16 tokens, one block per token" but
    lists 8 blocks; the blocks are taken as 2*cp equal chunks of L/(2*cp)
    tokens (2 tokens each in that example), held in ascending order.
    """
    _check(world, rank, global_len, 2 * world)
    c = global_len // (2 * world)
    blocks = [rank, 2 * world - 1 - rank]
    return np.concatenate([np.arange(b * c, (b + 1) * c, dtype=np.int64) for b in blocks])


def positions(assign, world: int, rank: int, global_len: int) -> np.ndarray:
    """Dispatch on ``assign`` (0/1/2 or "contiguous"/"striped"/"zigzag")."""
    a = NAMES.get(assign, assign)
    if a == CONTIGUOUS:
        return contiguous(world, rank, global_len)
    if a == STRIPED:
        return striped(world, rank, global_len)
    if a == ZIGZAG:
        return zigzag(world, rank, global_len)
    raise ValueError(f"unknown assignment {assign!r}")
