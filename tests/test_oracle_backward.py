"""Pins for oracle.backward: torch autograd (fp64, CPU) and central finite differences."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import backward as G
from oracle import positions as P


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("h,h_kv", [(3, 3), (4, 2), (4, 1)])
@pytest.mark.parametrize("causal,assign", [(False, "contiguous"), (True, "contiguous"), (True, "striped"),
                                           (True, "zigzag")])
def test_matches_torch_autograd(h, h_kv, causal, assign):
    # torch's own attention (explicit boolean mask, grouped KV heads) differentiated by autograd
    n, l, d = 4, 64, 16
    qpos = P.positions(assign, n, 2, l)
    kpos = np.arange(l)
    q, k, v = rnd(1, 2, qpos.size, h, d), rnd(2, 2, l, h_kv, d), rnd(3, 2, l, h_kv, d)
    do = rnd(4, 2, qpos.size, h, d)
    dq, dk, dv = G.attention_bwd(q, k, v, do, qpos, kpos, causal)
    qt, kt, vt = (torch.from_numpy(x).permute(0, 2, 1, 3).requires_grad_() for x in (q, k, v))
    mask = torch.from_numpy(A.visible(qpos, kpos, causal))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=1 / math.sqrt(d),
                                                         enable_gqa=True)
    o.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    for mine, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        assert np.max(np.abs(mine - ref.permute(0, 2, 1, 3).numpy())) < 1e-12


def test_finite_differences():
    # L = sum(O * dO); dL/dx by central differences on a few entries of q, k and v
    qpos, kpos = np.array([2, 5, 7]), np.array([0, 2, 3, 5, 6, 8])
    q, k, v, do = rnd(5, 1, 3, 2, 4), rnd(6, 1, 6, 1, 4), rnd(7, 1, 6, 1, 4), rnd(8, 1, 3, 2, 4)
    dq, dk, dv = G.attention_bwd(q, k, v, do, qpos, kpos, True)

    def loss(qq, kk, vv):
        o, _ = A.attention(qq, kk, vv, qpos, kpos, True)
        return float((o * do).sum())

    eps = 1e-6
    for arr, grad, idx in ((q, dq, (0, 1, 1, 2)), (q, dq, (0, 2, 0, 0)), (k, dk, (0, 3, 0, 1)),
                           (k, dk, (0, 0, 0, 3)), (v, dv, (0, 2, 0, 0)), (v, dv, (0, 5, 0, 2))):
        plus, minus = arr.copy(), arr.copy()
        plus[idx] += eps
        minus[idx] -= eps
        args_p = [plus if arr is x else x for x in (q, k, v)]
        args_m = [minus if arr is x else x for x in (q, k, v)]
        fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert abs(fd - grad[idx]) < 1e-7, (idx, fd, grad[idx])
    # key 8 is later than every query: no gradient reaches it
    assert np.all(dk[0, 5] == 0) and np.all(dv[0, 5] == 0)


def test_delta_is_row_sum_of_p_dp():
    qpos, kpos = P.positions("zigzag", 2, 1, 32), np.arange(32)
    q, k, v, do = rnd(9, 1, 16, 2, 8), rnd(10, 1, 32, 2, 8), rnd(11, 1, 32, 2, 8), rnd(12, 1, 16, 2, 8)
    o, _ = A.attention(q, k, v, qpos, kpos, True)
    delta = G.delta_rows(o, do)
    s = np.einsum("bqhd,bkhd->bhqk", q, k) / math.sqrt(8)
    s = np.where(A.visible(qpos, kpos, True)[None, None], s, -np.inf)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    dp = np.einsum("bqhd,bkhd->bhqk", do, v)
    assert np.max(np.abs(delta - (p * dp).sum(axis=-1))) < 1e-12


def _inputs(seed, b=1, sq=6, sk=9, h=2, h_kv=1, d=5):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((b, sq, h, d)), rng.standard_normal((b, sk, h_kv, d)),
            rng.standard_normal((b, sk, h_kv, d)), rng.standard_normal((b, sq, h, d)))


def test_magnitudes_bound_the_gradients():
    # triangle inequality: each gradient entry is at most its sum of absolute terms
    q, k, v, do = _inputs(11)
    qpos, kpos = np.array([2, 3, 5, 7, 8, 11]), np.arange(9) * 1.5
    dq, dk, dv = G.attention_bwd(q, k, v, do, qpos, kpos, True)
    a_dq, e_dq, a_dk, e_dk, a_dv = G.attention_bwd_magnitudes(q, k, v, do, qpos, kpos, True)
    assert np.all(np.abs(dq) <= a_dq + 1e-12) and np.all(np.abs(dk) <= a_dk + 1e-12)
    assert np.all(np.abs(dv) <= a_dv + 1e-12)
    assert not e_dq.any() and not e_dk.any()


def test_magnitudes_equal_gradients_for_positive_terms():
    # with dO >= 0 every term of dV is >= 0, so A_dv == dV; with K >= 0, sum_j P_ij k_j is
    # attention with V = K, so E_dq / (scale e_i) is that attention's output
    q, k, v, do = _inputs(12)
    do, k = np.abs(do), np.abs(k)
    _, _, dv = G.attention_bwd(q, k, v, do)
    e = np.full((1, 2, 6), 0.5)
    _, e_dq, _, _, a_dv = G.attention_bwd_magnitudes(q, k, v, do, delta_err=e)
    assert np.allclose(a_dv, dv, rtol=1e-13, atol=1e-13)
    o_kk, _ = A.attention(q, k, k)
    assert np.allclose(e_dq, o_kk * 0.5 / math.sqrt(5), rtol=1e-13, atol=1e-13)


def test_magnitudes_two_key_closed_form():
    # one query, two visible keys: dS_1 = P1 P2 (dP_1 - dP_2) = -dS_2, so with K all ones
    # A_dq = scale * 2 P1 P2 |dP_1 - dP_2| in every column
    rng = np.random.default_rng(13)
    d = 4
    q = rng.standard_normal((1, 1, 1, d))
    k = np.ones((1, 2, 1, d))
    k[0, 1, 0, 0] = 2.0          # make the two logits differ
    v = rng.standard_normal((1, 2, 1, d))
    do = rng.standard_normal((1, 1, 1, d))
    sc = 1 / math.sqrt(d)
    s = sc * np.array([q[0, 0, 0] @ k[0, 0, 0], q[0, 0, 0] @ k[0, 1, 0]])
    p = np.exp(s - s.max())
    p /= p.sum()
    dp = np.array([do[0, 0, 0] @ v[0, 0, 0], do[0, 0, 0] @ v[0, 1, 0]])
    a_dq = G.attention_bwd_magnitudes(q, k, v, do)[0]
    want = sc * p[0] * p[1] * abs(dp[0] - dp[1]) * (np.abs(k[0, 0, 0]) + np.abs(k[0, 1, 0]))
    assert np.allclose(a_dq[0, 0, 0], want, rtol=1e-13)
