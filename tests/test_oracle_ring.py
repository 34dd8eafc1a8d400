"""Pins for oracle.ring: the pages' invariants (exact ring, order and block-count independence)."""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import positions as P
from oracle import ring as R


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def shares_of(x, assign, n, l):
    return [x[:, P.positions(assign, n, r, l)] for r in range(n)]


@pytest.mark.parametrize("assign", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("n", [1, 2, 4, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_ring_equals_one_shot(assign, n, causal):
    # Digest §3.1: after N rounds each rank's result equals single-device attention exactly.
    l, h, d = 64, 2, 8
    q, k, v = rnd(1, 1, l, h, d), rnd(2, 1, l, h, d), rnd(3, 1, l, h, d)
    qs, ks, vs = shares_of(q, assign, n, l), shares_of(k, assign, n, l), shares_of(v, assign, n, l)
    kv_pos = [P.positions(assign, n, r, l) for r in range(n)]
    full = np.arange(l)
    for r in range(n):
        o, lse = R.ring_attention(qs[r], ks, vs, r, kv_pos[r], kv_pos, causal)
        o_ref, lse_ref = A.attention(qs[r], k, v, kv_pos[r], full, causal)
        assert np.max(np.abs(o - o_ref)) < 1e-12
        assert np.max(np.abs(lse - lse_ref)) < 1e-12


def test_ring_order_independence():
    # Digest §3.2: any order of KV blocks gives the same softmax.
    l, n, h, d = 96, 6, 1, 8
    q, k, v = rnd(4, 1, l, h, d), rnd(5, 1, l, h, d), rnd(6, 1, l, h, d)
    assign = "striped"
    ks, vs = shares_of(k, assign, n, l), shares_of(v, assign, n, l)
    kv_pos = [P.positions(assign, n, r, l) for r in range(n)]
    qs = shares_of(q, assign, n, l)
    r = 3
    base = R.ring_attention(qs[r], ks, vs, r, kv_pos[r], kv_pos, True)
    rng = np.random.default_rng(0)
    for _ in range(5):
        order = rng.permutation(n).tolist()
        o, lse = R.ring_attention(qs[r], ks, vs, r, kv_pos[r], kv_pos, True, steps=order)
        assert np.max(np.abs(o - base[0])) < 1e-12 and np.max(np.abs(lse - base[1])) < 1e-12


@pytest.mark.parametrize("nblocks", [1, 2, 4, 8, 16])
def test_online_softmax_block_count(nblocks):
    # Digest §3.2: the recurrence gives the one-shot softmax however many blocks are used.
    sq, sk, d = 16, 64, 8
    q, k, v = rnd(7, sq, d), rnd(8, sk, d), rnd(9, sk, d)
    qpos = np.arange(sq) * 4 + 1
    kpos = np.arange(sk)
    mask = A.visible(qpos, kpos, True)
    edges = np.linspace(0, sk, nblocks + 1).astype(int)
    perm = np.random.default_rng(nblocks).permutation(nblocks)
    kb = [k[edges[i]:edges[i + 1]] for i in perm]
    vb = [v[edges[i]:edges[i + 1]] for i in perm]
    mb = [mask[:, edges[i]:edges[i + 1]] for i in perm]
    o, lse = R.online_softmax(q, kb, vb, mb)
    o_ref, lse_ref = A.attention_rows(q, k, v, mask, 1 / math.sqrt(d))
    assert np.max(np.abs(o - o_ref)) < 1e-12
    assert np.max(np.abs(lse - lse_ref)) < 1e-12


def test_lse_merge_halves():
    sq, sk, d = 8, 40, 4
    q, k, v = rnd(10, sq, d), rnd(11, sk, d), rnd(12, sk, d)
    sc = 1 / math.sqrt(d)
    all_mask = np.ones((sq, sk), bool)
    oa, la = A.attention_rows(q, k[:13], v[:13], all_mask[:, :13], sc)
    ob, lb = A.attention_rows(q, k[13:], v[13:], all_mask[:, 13:], sc)
    o, lse = R.lse_merge(oa, la, ob, lb)
    o_ref, lse_ref = A.attention_rows(q, k, v, all_mask, sc)
    assert np.max(np.abs(o - o_ref)) < 1e-13 and np.max(np.abs(lse - lse_ref)) < 1e-13
    o2, lse2 = R.lse_merge(ob, lb, oa, la)  # commutative
    assert np.max(np.abs(o2 - o)) < 1e-15 and np.max(np.abs(lse2 - lse)) < 1e-15


def test_lse_merge_empty_sides():
    ob = rnd(13, 3, 4)
    lb = np.array([0.5, -2.0, 7.0])
    o, lse = R.lse_merge(np.zeros((3, 4)), np.full(3, -np.inf), ob, lb)
    assert np.array_equal(o, ob) and np.array_equal(lse, lb)
    o, lse = R.lse_merge(ob, lb, np.zeros((3, 4)), np.full(3, -np.inf))
    assert np.array_equal(o, ob) and np.array_equal(lse, lb)
    o, lse = R.lse_merge(np.zeros((2, 4)), np.full(2, -np.inf), np.zeros((2, 4)), np.full(2, -np.inf))
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_lse_merge_closed_form():
    # Two one-key blocks with logits a and b: lse = ln(e^a + e^b), O = (e^a v_a + e^b v_b)/(e^a+e^b).
    a, b = 1.5, -0.25
    va, vb = np.array([[1.0, 0.0]]), np.array([[0.0, 1.0]])
    o, lse = R.lse_merge(va, np.array([a]), vb, np.array([b]))
    z = math.exp(a) + math.exp(b)
    assert abs(lse[0] - math.log(z)) < 1e-15
    assert np.allclose(o[0], [math.exp(a) / z, math.exp(b) / z], atol=1e-15, rtol=0)
