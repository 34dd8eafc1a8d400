"""Online-softmax recurrence, LSE merge and the ring loop, in fp64.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

These forms are used only for the oracle's own invariants (the ring equals
one-shot attention, the result does not depend on block order or count) and
as the reference for the standalone merge call; the parity reference for O
and LSE is always ``attention.attention`` (the plain definition).
"""
from __future__ import annotations

import math

import numpy as np

from .attention import attention, visible


def online_softmax(q, k_blocks, v_blocks, masks, scale=None):
    """[Digest] §3.2: fold KV blocks one by one into the running (m, l, O).

    q [Sq, D]; k_blocks/v_blocks lists of [n_j, D]; masks list of bool [Sq, n_j].
    With s = q . k / sqrt(d) for the keys k of block j+1:
        m_{j+1} = max(m_j, max_k s)
        l_{j+1} = l_j e^{m_j - m_{j+1}} + sum_k e^{s - m_{j+1}}
        O_{j+1} = (O_j l_j e^{m_j - m_{j+1}} + sum_k e^{s - m_{j+1}} v_k) / l_{j+1}
    Masked keys contribute nothing. A row that has seen no key keeps
    m = -inf, l = 0, O = 0. Returns (O, LSE = m + ln l).
    """
    q = np.asarray(q, dtype=np.float64)
    sq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    m = np.full(sq, -np.inf)
    l = np.zeros(sq)
    o = np.zeros((sq, d))
    for kb, vb, mk in zip(k_blocks, v_blocks, masks):
        kb = np.asarray(kb, dtype=np.float64)
        vb = np.asarray(vb, dtype=np.float64)
        s = np.where(mk, (q @ kb.T) * scale, -np.inf)
        bmax = s.max(axis=1) if s.shape[1] else np.full(sq, -np.inf)
        m_new = np.maximum(m, bmax)
        live = np.isfinite(m_new)
        base = np.where(live, m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(np.where(np.isfinite(m), m, 0.0) - base), 0.0)
        p = np.exp(s - base[:, None])
        l_new = l * alpha + p.sum(axis=1)
        num = o * (l * alpha)[:, None] + p @ vb
        o = np.where(live[:, None], num / np.where(live, l_new, 1.0)[:, None], 0.0)
        m, l = m_new, l_new
    lse = np.where(np.isfinite(m), np.where(np.isfinite(m), m, 0.0) + np.log(np.where(l > 0, l, 1.0)),
                   -np.inf)
    return o, lse


def lse_merge(o_a, lse_a, o_b, lse_b):
    """[Digest] §6 item 3: merge two normalised partial results.

        lse = max(lse_a, lse_b) + log(1 + e^{-|lse_a - lse_b|})
        O   = O_a e^{lse_a - lse} + O_b e^{lse_b - lse}

    Reading of the garbled printed O formula: the weights are e^{lse_X - lse_new}
    on *normalised* O's, with nothing further divided. Reading for empty rows
    (the page is silent): a side with lse = -inf contributes nothing, and two
    empty sides give O = 0, lse = -inf, without evaluating (-inf) - (-inf).

    o_* [..., D] with lse_* of shape [...]. Returns (O, lse) in fp64.
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    a = np.asarray(lse_a, dtype=np.float64)
    b = np.asarray(lse_b, dtype=np.float64)
    fa, fb = np.isfinite(a), np.isfinite(b)
    both = fa & fb
    a0 = np.where(fa, a, 0.0)
    b0 = np.where(fb, b, 0.0)
    hi = np.maximum(a0, b0)
    lse = np.where(both, hi + np.log1p(np.exp(-np.abs(a0 - b0))),
                   np.where(fa, a, np.where(fb, b, -np.inf)))
    l0 = np.where(np.isfinite(lse), lse, 0.0)
    wa = np.where(fa, np.exp(a0 - l0), 0.0)
    wb = np.where(fb, np.exp(b0 - l0), 0.0)
    o = o_a * wa[..., None] + o_b * wb[..., None]
    return o, lse


def ring_attention(q_share, k_shares, v_shares, rank, q_pos, kv_pos, causal, scale=None,
                   steps=None):
    """[Digest] §3.1/§3.3: one rank's ring loop, run as a plain loop.

    Round ``step`` uses the KV share of rank ``(rank - step) mod N`` (round 0 is
    local; KV is sent to rank+1 and received from rank-1). Each round computes
    the block result (O, LSE) of the local Q against that share with
    ``attention.attention`` and merges it into the accumulator with
    ``lse_merge``. q_share [B, S, H, D]; k_shares/v_shares lists of N arrays
    [B, S_k, H, D]; kv_pos list of N position arrays. ``steps`` optionally
    overrides the visiting order (for the order-independence invariant).
    Returns (O [B, S, H, D], LSE [B, H, S]).
    """
    n = len(k_shares)
    b_, s, h_, d = np.shape(q_share)
    acc_o = np.zeros((b_, s, h_, d))
    acc_lse = np.full((b_, h_, s), -np.inf)
    order = [(rank - st) % n for st in range(n)] if steps is None else list(steps)
    for src in order:
        o_blk, lse_blk = attention(q_share, k_shares[src], v_shares[src], q_pos, kv_pos[src], causal,
                                   scale)
        # LSE is [B, H, S]; O is [B, S, H, D]: merge per (b, s, h) row.
        lse_a = np.transpose(acc_lse, (0, 2, 1))
        lse_b = np.transpose(lse_blk, (0, 2, 1))
        acc_o, lse_m = lse_merge(acc_o, lse_a, o_blk, lse_b)
        acc_lse = np.transpose(lse_m, (0, 2, 1))
    return acc_o, acc_lse


__all__ = ["online_softmax", "lse_merge", "ring_attention", "visible"]
