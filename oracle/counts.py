"""Counts of visible (query, key) pairs and of tile classes.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

The causal work of a share is the number of (query, key) pairs with key
position <= query position ([Digest] §3.4: the lower-triangular causal matrix
is why contiguous shards are unbalanced). FLOP accounting uses 4*D per visible
pair per head (2*D for q.k, 2*D for p*v).
"""
from __future__ import annotations

import numpy as np


def visible_pairs(qpos, kpos, causal: bool = True) -> int:
    """Number of (i, j) with kpos[j] <= qpos[i] (all pairs if not causal)."""
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    if not causal:
        return int(qpos.size) * int(kpos.size)
    ks = np.sort(kpos)
    return int(np.searchsorted(ks, qpos, side="right").sum())


def visible_pairs_brute(qpos, kpos) -> int:
    """Same count by an explicit double loop (tiny inputs only)."""
    return sum(1 for qp in qpos for kp in kpos if kp <= qp)


def tile_classes(qpos, kpos, bm: int, bn: int, causal: bool = True):
    """(full, partial, skip) counts over the bm x bn tiles of the [Sq, Sk] mask.

    A tile is *skip* when none of its pairs is visible, *full* when all are and
    *partial* otherwise; decided from the tile's own positions (its largest
    query position against its smallest key position, and vice versa), which
    is exact for any order of positions within the tile.
    """
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    full = partial = skip = 0
    for i0 in range(0, qpos.size, bm):
        qt = qpos[i0:i0 + bm]
        qmin, qmax = qt.min(), qt.max()
        for j0 in range(0, kpos.size, bn):
            kt = kpos[j0:j0 + bn]
            if not causal or qmin >= kt.max():
                full += 1
            elif qmax < kt.min():
                skip += 1
            else:
                partial += 1
    return full, partial, skip


def tiled_walk(qpos, kpos_steps, bm: int, bn: int, wr: int, causal: bool = True):
    """The tiles a blocked kernel must touch, per query tile and per block of ``wr`` query rows.

    Query rows are cut into tiles of ``bm`` (each made of ``bm // wr`` row blocks of ``wr``),
    every step's keys into tiles of ``bn``. A (query tile, key tile) pair must be visited unless
    none of its pairs is visible (the skipped upper triangle of the causal matrix, [Digest]
    §3.4). A row block has to apply the mask on a visited key tile when the tile is shorter than
    ``bn`` (the ragged end of a share) or when some (row, key) pair of the block and the tile is
    invisible. Row blocks lying past the last query row are not counted.

    Whether a set of pairs has a visible one, or only visible ones, is decided from the sets'
    extreme positions (some pair visible iff the smallest key position <= the largest query
    position; all visible iff the largest key position <= the smallest query position), which
    is exact for any order of positions; ``tiled_walk_brute`` decides the same from explicit
    masks. Returns (visited [n_qt], masked [n_qt, bm // wr]) summed over the steps;
    ``kpos_steps`` is the list of every step's key positions.
    """
    qpos = np.asarray(qpos, dtype=np.int64)
    sq = qpos.size
    n_qt = (sq + bm - 1) // bm
    nw = bm // wr
    pad = np.full(n_qt * bm, -1, dtype=np.int64)
    pad[:sq] = qpos
    tiles = pad.reshape(n_qt, bm)
    qmax = tiles.max(axis=1)
    blocks = np.where(tiles >= 0, tiles, np.iinfo(np.int64).max).reshape(n_qt, nw, wr)
    wmin = blocks.min(axis=2)                                   # [n_qt, nw]
    live = (np.arange(n_qt)[:, None] * bm + np.arange(nw)[None, :] * wr) < sq
    visited = np.zeros(n_qt, dtype=np.int64)
    masked = np.zeros((n_qt, nw), dtype=np.int64)
    for kpos in kpos_steps:
        kpos = np.asarray(kpos, dtype=np.int64)
        n_kt = (kpos.size + bn - 1) // bn
        if n_kt == 0:
            continue
        kmin = np.array([kpos[j * bn:(j + 1) * bn].min() for j in range(n_kt)])
        kmax = np.array([kpos[j * bn:(j + 1) * bn].max() for j in range(n_kt)])
        ragged = np.array([kpos[j * bn:(j + 1) * bn].size < bn for j in range(n_kt)])
        if causal:
            vis = kmin[None, :] <= qmax[:, None]                # [n_qt, n_kt]
            part = kmax[None, None, :] > wmin[:, :, None]       # [n_qt, nw, n_kt]
        else:
            vis = np.ones((n_qt, n_kt), dtype=bool)
            part = np.zeros((n_qt, nw, n_kt), dtype=bool)
        visited += vis.sum(axis=1)
        masked += (vis[:, None, :] & (part | ragged[None, None, :])).sum(axis=2) * live
    return visited, masked


def tiled_walk_brute(qpos, kpos_steps, bm: int, bn: int, wr: int, causal: bool = True):
    """``tiled_walk`` from explicit (row, key) masks, tile by tile (tiny inputs only)."""
    qpos = np.asarray(qpos, dtype=np.int64)
    sq = qpos.size
    n_qt = (sq + bm - 1) // bm
    nw = bm // wr
    visited = np.zeros(n_qt, dtype=np.int64)
    masked = np.zeros((n_qt, nw), dtype=np.int64)
    for kpos in kpos_steps:
        kpos = np.asarray(kpos, dtype=np.int64)
        for t in range(n_qt):
            rows = qpos[t * bm:(t + 1) * bm]
            for j0 in range(0, kpos.size, bn):
                keys = kpos[j0:j0 + bn]
                vis = keys[None, :] <= rows[:, None] if causal else np.ones((rows.size, keys.size), bool)
                if not vis.any():
                    continue
                visited[t] += 1
                for w in range(nw):
                    blk = vis[w * wr:(w + 1) * wr]
                    if blk.size and (keys.size < bn or not blk.all()):
                        masked[t, w] += 1
    return visited, masked
