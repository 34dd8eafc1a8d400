"""Pins for oracle.counts: brute force and closed forms of the causal work per share."""
import numpy as np
import pytest

from oracle import counts as C
from oracle import positions as P


@pytest.mark.parametrize("assign", ["contiguous", "striped", "zigzag"])
def test_pairs_match_brute_force(assign):
    n, l = 4, 48
    kpos = np.arange(l)
    for r in range(n):
        qpos = P.positions(assign, n, r, l)
        assert C.visible_pairs(qpos, kpos) == C.visible_pairs_brute(qpos, kpos)


def test_contiguous_closed_form():
    # rank r of contiguous chunks of C: r*C^2 (earlier chunks) + C(C+1)/2 (own triangle).
    n, l = 8, 8192
    c = l // n
    kpos = np.arange(l)
    for r in range(n):
        assert C.visible_pairs(P.positions("contiguous", n, r, l), kpos) == r * c * c + c * (c + 1) // 2
    assert C.visible_pairs(P.positions("contiguous", 8, 7, 8192), kpos) == 7_864_832


def test_striped_closed_form():
    # stripe s <= r: j <= i (S(S+1)/2 pairs); s > r: j <= i-1 (S(S-1)/2 pairs).
    n, l = 8, 32768
    s = l // n
    kpos = np.arange(l)
    for r in [0, 7]:
        want = (r + 1) * s * (s + 1) // 2 + (n - 1 - r) * s * (s - 1) // 2
        assert C.visible_pairs(P.positions("striped", n, r, l), kpos) == want
    assert C.visible_pairs(P.positions("striped", 8, 0, 32768), kpos) == 67_096_576


def test_zigzag_balanced_closed_form():
    # every rank: (2N-1) C^2 + C(C+1)
    n, l = 8, 4096
    c = l // (2 * n)
    kpos = np.arange(l)
    for r in range(n):
        assert C.visible_pairs(P.positions("zigzag", n, r, l), kpos) == (2 * n - 1) * c * c + c * (c + 1)


def test_full_causal():
    l = 65536
    assert C.visible_pairs(np.arange(l), np.arange(l)) == l * (l + 1) // 2


def test_tile_classes_contiguous_rank7():
    # 8 q-tiles x 64 k-tiles of 128: shares 0..6 all full (448), own share: 28 full, 8 partial, 28 skip.
    qpos = P.positions("contiguous", 8, 7, 8192)
    assert C.tile_classes(qpos, np.arange(8192), 128, 128) == (476, 8, 28)


def test_tile_classes_brute():
    qpos = P.positions("zigzag", 2, 1, 32)
    kpos = np.arange(32)
    mask = kpos[None, :] <= qpos[:, None]
    full = partial = skip = 0
    for i0 in range(0, 16, 4):
        for j0 in range(0, 32, 8):
            blk = mask[i0:i0 + 4, j0:j0 + 8]
            full += blk.all(); skip += (~blk).all(); partial += blk.any() and not blk.all()
    assert C.tile_classes(qpos, kpos, 4, 8) == (full, partial, skip)


@pytest.mark.parametrize("assign", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("n,l", [(1, 40), (2, 64), (4, 200), (3, 96)])
@pytest.mark.parametrize("causal", [True, False])
def test_tiled_walk_matches_explicit_masks(assign, n, l, causal):
    # extreme-position decisions against tile-by-tile explicit masks, ragged tiles included
    if assign == "zigzag" and l % (2 * n):
        pytest.skip("zigzag needs L % 2N == 0")
    for r in range(n):
        qpos = P.positions(assign, n, r, l)
        steps = [P.positions(assign, n, (r - s) % n, l) for s in range(n)]
        for bm, bn, wr in ((8, 4, 2), (12, 5, 4), (16, 16, 16)):
            got = C.tiled_walk(qpos, steps, bm, bn, wr, causal)
            want = C.tiled_walk_brute(qpos, steps, bm, bn, wr, causal)
            assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]), (r, bm, bn, wr)


def test_tiled_walk_totals_are_tile_classes():
    # visited tiles = full + partial tiles of the same tiling; the skipped ones are the rest
    n, l = 8, 8192
    qpos = P.positions("contiguous", n, 7, l)
    steps = [P.positions("contiguous", n, s, l) for s in range(n)]
    vis, msk = C.tiled_walk(qpos, steps, 128, 64, 32)
    full = partial = skip = 0
    for k in steps:
        f, p_, s_ = C.tile_classes(qpos, k, 128, 64)
        full, partial, skip = full + f, partial + p_, skip + s_
    assert vis.sum() == full + partial and skip == 8 * 8 * 16 - vis.sum()
    # contiguous rank 7 against itself (shares 0..6 are fully visible): query tile t (rows
    # 128t .. 128t+127 of the share) visits key tiles 0 .. 2t+1; key tile 2t+1 (keys 128t+64 ..
    # 128t+127) is partial for all four 32-row blocks, key tile 2t (keys 128t .. 128t+63) for
    # the first two only
    assert vis.tolist() == [7 * 16 + 2 * t + 2 for t in range(8)]
    assert msk.tolist() == [[2, 2, 1, 1]] * 8
