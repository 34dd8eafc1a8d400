"""Pins for oracle.attention: library routine on special cases, closed forms, brute force."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import positions as P


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def sdpa_ref(q, k, v, mask, scale):
    # torch's own attention on CPU in float64 with an explicit boolean mask.
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)  # [B,H,S,D]
    kt = torch.from_numpy(k).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3)
    m = torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    logits = (qt @ kt.transpose(-1, -2)) * scale
    logits = logits.masked_fill(~m, float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("assign", ["contiguous", "striped", "zigzag"])
def test_matches_torch_sdpa(causal, assign):
    n, l, d, h = 4, 64, 16, 3
    r = 2
    qpos = P.positions(assign, n, r, l)
    kpos = np.arange(l)
    q, k, v = rnd(1, 2, qpos.size, h, d), rnd(2, 2, l, h, d), rnd(3, 2, l, h, d)
    o, lse = A.attention(q, k, v, qpos, kpos, causal)
    mask = A.visible(qpos, kpos, causal)
    o_ref, lse_ref = sdpa_ref(q, k, v, mask, 1 / math.sqrt(d))
    assert np.max(np.abs(o - o_ref)) < 1e-12
    assert np.max(np.abs(lse - lse_ref)) < 1e-12


@pytest.mark.parametrize("h,h_kv", [(4, 2), (6, 1), (8, 4), (3, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_grouped_query_matches_torch_sdpa(h, h_kv, causal):
    # GQA / MQA against torch's own grouped-query attention (enable_gqa), which shares each
    # KV head among h / h_kv consecutive query heads
    n, l, d = 4, 64, 16
    qpos = P.positions("zigzag", n, 1, l)
    kpos = np.arange(l)
    q, k, v = rnd(7, 2, qpos.size, h, d), rnd(8, 2, l, h_kv, d), rnd(9, 2, l, h_kv, d)
    o, lse = A.attention(q, k, v, qpos, kpos, causal)
    mask = torch.from_numpy(A.visible(qpos, kpos, causal))
    qt, kt, vt = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    o_ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=1 / math.sqrt(d),
                                                             enable_gqa=True).permute(0, 2, 1, 3).numpy()
    assert o.shape == (2, qpos.size, h, d)
    assert np.max(np.abs(o - o_ref)) < 1e-12
    # each query head against its own KV head, one head at a time
    for hq in range(h):
        oh, lh = A.attention(q[:, :, hq:hq + 1], k[:, :, hq * h_kv // h:hq * h_kv // h + 1],
                             v[:, :, hq * h_kv // h:hq * h_kv // h + 1], qpos, kpos, causal)
        assert np.array_equal(oh[:, :, 0], o[:, :, hq]) and np.array_equal(lh[:, 0], lse[:, hq])


def test_grouped_query_rejects_non_divisor():
    with pytest.raises(ValueError):
        A.attention(rnd(1, 1, 4, 6, 8), rnd(2, 1, 4, 4, 8), rnd(3, 1, 4, 4, 8))


def test_matches_python_loops():
    qpos, kpos = np.array([3, 5, 9]), np.array([0, 4, 5, 8, 9, 12])
    q, k, v = rnd(4, 1, 3, 2, 5), rnd(5, 1, 6, 2, 5), rnd(6, 1, 6, 2, 5)
    o, lse = A.attention(q, k, v, qpos, kpos, True)
    o2, lse2 = A.attention_loops(q.tolist(), k.tolist(), v.tolist(), qpos, kpos, True)
    assert np.max(np.abs(o - np.array(o2))) < 1e-13
    assert np.max(np.abs(lse - np.array(lse2))) < 1e-13


def test_zero_logits_closed_form():
    # With Q = 0 every visible logit is 0: LSE_i = ln|V_i| and O_i = mean of the visible V rows.
    n, l, d = 8, 256, 8
    for assign in ["contiguous", "striped", "zigzag"]:
        r = 5
        qpos = P.positions(assign, n, r, l)
        kpos = np.arange(l)
        q = np.zeros((1, qpos.size, 1, d))
        k, v = rnd(7, 1, l, 1, d), rnd(8, 1, l, 1, d)
        o, lse = A.attention(q, k, v, qpos, kpos, True)
        for i, qp in enumerate(qpos):
            cnt = qp + 1  # keys 0..qp, diagonal included
            assert abs(lse[0, 0, i] - math.log(cnt)) < 1e-12
            assert np.max(np.abs(o[0, i, 0] - v[0, :qp + 1, 0].mean(axis=0))) < 1e-12


def test_single_visible_key():
    # Global position 0 sees only key 0: O = v_0 exactly, LSE = scale * q0 . k0.
    d = 32
    q, k, v = rnd(9, 1, 4, 2, d), rnd(10, 1, 4, 2, d), rnd(11, 1, 4, 2, d)
    pos = np.arange(4)
    o, lse = A.attention(q, k, v, pos, pos, True)
    for h in range(2):
        assert np.array_equal(o[0, 0, h], v[0, 0, h])
        assert abs(lse[0, h, 0] - q[0, 0, h] @ k[0, 0, h] / math.sqrt(d)) < 1e-13


def test_two_key_closed_form_and_scale():
    # q = e1, k0 = a*e1, k1 = 0, v0 = e1, v1 = e2: s0 = a*scale, s1 = 0,
    # O = (e^{s0} e1 + e2) / (e^{s0} + 1), LSE = ln(e^{s0} + 1).  Pins scale, sign, V orientation.
    d, a = 4, 3.0
    q = np.zeros((1, 1, 1, d)); q[0, 0, 0, 0] = 1
    k = np.zeros((1, 2, 1, d)); k[0, 0, 0, 0] = a
    v = np.zeros((1, 2, 1, d)); v[0, 0, 0, 0] = 1; v[0, 1, 0, 1] = 1
    for scale in [None, 0.25]:
        sc = 1 / math.sqrt(d) if scale is None else scale
        o, lse = A.attention(q, k, v, scale=scale)
        e = math.exp(a * sc)
        assert np.allclose(o[0, 0, 0], [e / (e + 1), 1 / (e + 1), 0, 0], atol=1e-15, rtol=0)
        assert abs(lse[0, 0, 0] - math.log(e + 1)) < 1e-15


def test_empty_row():
    q, k, v = rnd(12, 1, 2, 1, 4), rnd(13, 1, 3, 1, 4), rnd(14, 1, 3, 1, 4)
    o, lse = A.attention(q, k, v, np.array([0, 10]), np.array([5, 6, 7]), True)
    assert np.all(o[0, 0] == 0) and lse[0, 0, 0] == -np.inf
    assert np.isfinite(lse[0, 0, 1])


def test_causal_rows_page(golden):
    rows = golden("causal_rows.txt")
    L = int(rows[0][0][1])
    mask = A.visible(np.arange(L), np.arange(L), True)
    for (qp,), keys in rows[1:]:
        assert np.flatnonzero(mask[qp]).tolist() == keys
