"""Ulysses sequence-sharded <-> head-sharded layout change, by index formula.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

[Digest] §5.1: before the all-to-all, rank src holds Q/K/V of shape
[bs, L/P, H, d_head] (its contiguous run of the sequence, every head); after
it, rank p holds [bs, L, H/P, d_head]: the whole sequence for heads
p*H/P .. (p+1)*H/P - 1. The full sequence of rank p is ordered by source rank
(rank src's rows come at src*L/P ..). On one device the P source shares are
stacked as x [P, B, S_loc, H, D] and the layout change for rank p is

    out[b, src*S_loc + s, h', :] = x[src, b, s, p*H/P + h', :]

The head-count constraint of [Digest] §5.3 (P must divide H) raises ValueError.
"""
from __future__ import annotations

import numpy as np


def seq2head(x, dst_rank):
    """x [P, B, S, H, D] -> [B, P*S, H/P, D] for ``dst_rank``, or the stack of all
    ranks' results [P, B, P*S, H/P, D] when ``dst_rank`` is None or -1."""
    x = np.asarray(x)
    p_, b_, s_, h_, d_ = x.shape
    if h_ % p_:
        raise ValueError(f"P={p_} does not divide H={h_}")
    hp = h_ // p_
    if dst_rank is None or dst_rank == -1:
        return np.stack([seq2head(x, p) for p in range(p_)])
    out = np.empty((b_, p_ * s_, hp, d_), dtype=x.dtype)
    for src in range(p_):
        for s in range(s_):
            out[:, src * s_ + s, :, :] = x[src, :, s, dst_rank * hp:(dst_rank + 1) * hp, :]
    return out


def head2seq(y, dst_rank, x_out):
    """Inverse of ``seq2head`` for one rank: write y [B, P*S, H/P, D] (rank
    ``dst_rank``'s head slice) back into x_out [P, B, S, H, D] in place; the other
    heads of x_out are left untouched. With ``dst_rank`` None/-1, y is the stack
    [P, B, P*S, H/P, D] and every head slice is written."""
    x_out = np.asarray(x_out)
    p_, b_, s_, h_, d_ = x_out.shape
    if h_ % p_:
        raise ValueError(f"P={p_} does not divide H={h_}")
    hp = h_ // p_
    if dst_rank is None or dst_rank == -1:
        for p in range(p_):
            head2seq(y[p], p, x_out)
        return x_out
    for src in range(p_):
        for s in range(s_):
            x_out[src, :, s, dst_rank * hp:(dst_rank + 1) * hp, :] = y[:, src * s_ + s, :, :]
    return x_out
