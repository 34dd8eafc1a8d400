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
