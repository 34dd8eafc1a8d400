"""Exact attention by its definition, in fp64, with an explicit boolean mask.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

[Digest] §2 defines Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V. For one
query row i with visible key set V_i:

    s_j   = scale * (q_i . k_j)                        (scale = 1/sqrt(d))
    m     = max_{j in V_i} s_j
    l     = sum_{j in V_i} exp(s_j - m)
    O_i   = sum_{j in V_i} exp(s_j - m) v_j / l
    LSE_i = m + ln l                                   (natural log)

Readings (the pages are silent or brief here):
  * causal visibility is by *global* position, key position <= query position,
    the diagonal included ([Digest] §3.4 causal matrix: token 0 sees itself
    only; [Q14] engineering notes: the mask is decided by ring position);
  * the default scale is 1/sqrt(head dim) ([Digest] §2 and the
    ``softmax_scale=None`` argument of the §10 ring example);
  * LSE is the natural log of the sum of exp of the *scaled* logits over the
    visible keys (the merge formula of [Digest] §6 item 3 uses log and e);
  * a row with no visible key (possible for a single block, never for a whole
    ring) gets O = 0 and LSE = -inf;
  * grouped-query attention ([Digest] §5.3: GQA has fewer KV heads than query
    heads; MQA has one): K and V carry H_kv heads with H_kv dividing H, and query
    head h attends KV head h // (H / H_kv), i.e. each run of H / H_kv consecutive
    query heads shares one KV head (the usual grouping; the pages do not spell it
    out). H_kv = H is plain multi-head attention.
"""
from __future__ import annotations

import math

import numpy as np


def visible(qpos, kpos, causal: bool) -> np.ndarray:
    """Boolean [Sq, Sk] matrix: True where query row i may attend to key j."""
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    if not causal:
        return np.ones((qpos.size, kpos.size), dtype=bool)
    return kpos[None, :] <= qpos[:, None]


def attention_rows(q, k, v, mask, scale):
    """O [Sq, D] and LSE [Sq] for one (batch, head): q [Sq, D], k/v [Sk, D] fp64."""
    s = (q @ k.T) * scale
    s = np.where(mask, s, -np.inf)
    if s.shape[1] == 0:
        m = np.full(s.shape[0], -np.inf)
    else:
        m = s.max(axis=1)
    has = np.isfinite(m)
    m0 = np.where(has, m, 0.0)
    p = np.exp(s - m0[:, None])          # exp(-inf) = 0 for masked keys
    l = p.sum(axis=1)
    o = (p @ v) / np.where(has, l, 1.0)[:, None]
    o[~has] = 0.0
    lse = np.where(has, m0 + np.log(np.where(has, l, 1.0)), -np.inf)
    return o, lse


def attention(q, k, v, qpos=None, kpos=None, causal: bool = False, scale=None,
              row_chunk: int = 256):
    """fp64 attention of q [B, Sq, H, D] against k, v [B, Sk, H_kv, D] (H_kv divides H;
    query head h uses KV head h // (H / H_kv)).

    ``qpos``/``kpos`` are the global positions of the rows (needed when
    ``causal``). Returns O [B, Sq, H, D] and LSE [B, H, Sq], both float64.
    Rows are evaluated ``row_chunk`` at a time only to bound memory; every row
    is computed by the same formula independently of the others.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b_, sq, h_, d = q.shape
    sk = k.shape[1]
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    if causal:
        qpos = np.asarray(qpos, dtype=np.int64)
        kpos = np.asarray(kpos, dtype=np.int64)
        assert qpos.shape == (sq,) and kpos.shape == (sk,)
    o = np.zeros((b_, sq, h_, d), dtype=np.float64)
    lse = np.zeros((b_, h_, sq), dtype=np.float64)
    h_kv = k.shape[2]
    if h_kv < 1 or h_ % h_kv or v.shape[2] != h_kv:
        raise ValueError(f"KV heads {h_kv} must divide query heads {h_}")
    group = h_ // h_kv
    for b in range(b_):
        for h in range(h_):
            kk, vv = k[b, :, h // group, :], v[b, :, h // group, :]
            for r0 in range(0, sq, row_chunk):
                r1 = min(sq, r0 + row_chunk)
                if causal:
                    mask = visible(qpos[r0:r1], kpos, True)
                else:
                    mask = np.ones((r1 - r0, sk), dtype=bool)
                o[b, r0:r1, h, :], lse[b, h, r0:r1] = attention_rows(q[b, r0:r1, h, :], kk, vv, mask,
                                                                      scale)
    return o, lse


def attention_loops(q, k, v, qpos, kpos, causal, scale=None):
    """The same definition with pure-Python loops and the ``math`` module, for
    tiny inputs only (an independent check of the numpy form)."""
    b_, sq, h_, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    sk = len(k[0])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = [[[[0.0] * d for _ in range(h_)] for _ in range(sq)] for _ in range(b_)]
    lse = [[[0.0] * sq for _ in range(h_)] for _ in range(b_)]
    for b in range(b_):
        for h in range(h_):
            for i in range(sq):
                vis = [j for j in range(sk) if (not causal) or kpos[j] <= qpos[i]]
                if not vis:
                    lse[b][h][i] = -math.inf
                    continue
                s = {j: scale * sum(float(q[b][i][h][t]) * float(k[b][j][h][t]) for t in range(d))
                     for j in vis}
                m = max(s.values())
                w = {j: math.exp(s[j] - m) for j in vis}
                den = sum(w.values())
                for t in range(d):
                    out[b][i][h][t] = sum(w[j] * float(v[b][j][h][t]) for j in vis) / den
                lse[b][h][i] = m + math.log(den)
    return out, lse
