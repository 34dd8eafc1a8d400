"""Gradients of attention by the chain rule, in fp64.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

The pages train with ring attention but give no backward formulas, so this is the
derivative of the definition in ``attention.py`` (softmax of the scaled, masked logits
times V; [Digest] §2 with the causal visibility of §3.4), written out for one (batch,
head):

    s_ij    = scale * (q_i . k_j)                     visible pairs only
    P_ij    = exp(s_ij - LSE_i)                       0 for invisible pairs
    dV_j    = sum_i P_ij dO_i
    dP_ij   = dO_i . v_j
    Delta_i = sum_j P_ij dP_ij                        (= dO_i . O_i)
    dS_ij   = P_ij (dP_ij - Delta_i)
    dQ_i    = scale * sum_j dS_ij k_j
    dK_j    = scale * sum_i dS_ij q_i

With grouped KV heads (query head h reads KV head h // (H / H_kv)), dK and dV of a KV
head sum the contributions of its query heads. A query row with no visible key has P = 0
and contributes nothing.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import visible


def attention_bwd(q, k, v, do, qpos=None, kpos=None, causal: bool = False, scale=None,
                  row_chunk: int = 256):
    """dQ [B, Sq, H, D], dK and dV [B, Sk, H_kv, D] (float64) of O = attention(q, k, v)
    for the upstream gradient ``do`` [B, Sq, H, D]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    b_, sq, h_, d = q.shape
    sk, h_kv = k.shape[1], k.shape[2]
    if h_kv < 1 or h_ % h_kv or v.shape != k.shape or do.shape != q.shape:
        raise ValueError("shapes: q/do [B,Sq,H,D], k/v [B,Sk,H_kv,D] with H_kv dividing H")
    group = h_ // h_kv
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    if causal:
        qpos = np.asarray(qpos, dtype=np.int64)
        kpos = np.asarray(kpos, dtype=np.int64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(b_):
        for h in range(h_):
            kk, vv = k[b, :, h // group], v[b, :, h // group]
            for r0 in range(0, sq, row_chunk):
                r1 = min(sq, r0 + row_chunk)
                mask = visible(qpos[r0:r1], kpos, True) if causal else np.ones((r1 - r0, sk), dtype=bool)
                s = np.where(mask, (q[b, r0:r1, h] @ kk.T) * scale, -np.inf)
                m = s.max(axis=1) if sk else np.full(r1 - r0, -np.inf)
                has = np.isfinite(m)
                p = np.exp(s - np.where(has, m, 0.0)[:, None])
                p /= np.where(has, p.sum(axis=1), 1.0)[:, None]      # softmax; 0 on masked keys
                g = do[b, r0:r1, h]
                dv[b, :, h // group] += p.T @ g
                dp = g @ vv.T
                delta = (p * dp).sum(axis=1)
                ds = p * (dp - delta[:, None])
                dq[b, r0:r1, h] = scale * (ds @ kk)
                dk[b, :, h // group] += scale * (ds.T @ q[b, r0:r1, h])
    return dq, dk, dv


def delta_rows(o, do):
    """Delta [B, H, Sq] = sum over d of dO * O (the row term of dS)."""
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    return np.einsum("bshd,bshd->bhs", o, do)


def attention_bwd_magnitudes(q, k, v, do, qpos=None, kpos=None, causal: bool = False, scale=None,
                             delta_err=None, row_chunk: int = 256):
    """Entry-wise magnitudes of the sums that make up each gradient of ``attention_bwd``, for
    error bounds: the same chain rule with every term replaced by its absolute value.

        A_dq[i] = scale * sum_j |dS_ij| |k_j|       A_dk[j] = scale * sum_i |dS_ij| |q_i|
        E_dq[i] = scale * e_i sum_j P_ij |k_j|       E_dk[j] = scale * sum_i e_i P_ij |q_i|
        A_dv[j] = sum_i P_ij |dO_i|

    (|.| taken element by element along the head dimension). ``delta_err`` [B, H, Sq] is a
    per-row bound e_i on an error in Delta_i (zero when omitted): a change of Delta_i by e
    changes dS_ij by P_ij e. A bounded relative error u on every term of a sum moves it by at
    most u times these magnitudes. Returns (A_dq, E_dq, A_dk, E_dk, A_dv) in the gradients'
    shapes, float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    b_, sq, h_, d = q.shape
    sk, h_kv = k.shape[1], k.shape[2]
    group = h_ // h_kv
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    if causal:
        qpos = np.asarray(qpos, dtype=np.int64)
        kpos = np.asarray(kpos, dtype=np.int64)
    e_all = np.zeros((b_, h_, sq)) if delta_err is None else np.asarray(delta_err, dtype=np.float64)
    a_dq, e_dq = np.zeros_like(q), np.zeros_like(q)
    a_dk, e_dk, a_dv = np.zeros_like(k), np.zeros_like(k), np.zeros_like(v)
    for b in range(b_):
        for h in range(h_):
            hk = h // group
            kk, vv = k[b, :, hk], v[b, :, hk]
            for r0 in range(0, sq, row_chunk):
                r1 = min(sq, r0 + row_chunk)
                mask = visible(qpos[r0:r1], kpos, True) if causal else np.ones((r1 - r0, sk), dtype=bool)
                s = np.where(mask, (q[b, r0:r1, h] @ kk.T) * scale, -np.inf)
                m = s.max(axis=1) if sk else np.full(r1 - r0, -np.inf)
                has = np.isfinite(m)
                p = np.exp(s - np.where(has, m, 0.0)[:, None])
                p /= np.where(has, p.sum(axis=1), 1.0)[:, None]
                g = do[b, r0:r1, h]
                dp = g @ vv.T
                ds = p * (dp - (p * dp).sum(axis=1)[:, None])
                e = e_all[b, h, r0:r1]
                aq = np.abs(q[b, r0:r1, h])
                a_dq[b, r0:r1, h] = scale * (np.abs(ds) @ np.abs(kk))
                e_dq[b, r0:r1, h] = scale * e[:, None] * (p @ np.abs(kk))
                a_dk[b, :, hk] += scale * (np.abs(ds).T @ aq)
                e_dk[b, :, hk] += scale * ((p * e[:, None]).T @ aq)
                a_dv[b, :, hk] += p.T @ np.abs(g)
    return a_dq, e_dq, a_dk, e_dk, a_dv
