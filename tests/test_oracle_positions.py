"""Pins for oracle.positions: the pages' literal examples and coverage."""
import numpy as np
import pytest

from oracle import positions as P


def test_contiguous_page_example(golden):
    for (n, l, r), vals in golden("positions_contiguous_n4_l16.txt"):
        assert P.positions("contiguous", n, r, l).tolist() == vals


def test_striped_page_example(golden):
    for (n, l, r), vals in golden("positions_striped_n4_l16.txt"):
        assert P.positions("striped", n, r, l).tolist() == vals


def test_zigzag_page_example(golden):
    L = 16
    for (cp, r), blocks in golden("zigzag_blocks_cp4.txt"):
        c = L // (2 * cp)
        expect = [b * c + t for b in blocks for t in range(c)]
        assert P.positions("zigzag", cp, r, L).tolist() == expect


def test_zigzag_long_share_chunks():
    # 262144 tokens, N=8 -> 16 chunks of 16384; rank 3 holds chunks 3 and 12.
    pos = P.positions("zigzag", 8, 3, 262144)
    assert pos.size == 32768
    assert pos[0] == 3 * 16384 and pos[16383] == 4 * 16384 - 1
    assert pos[16384] == 12 * 16384 and pos[-1] == 13 * 16384 - 1


@pytest.mark.parametrize("assign", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("n,l", [(1, 8), (2, 8), (4, 16), (8, 64), (8, 8192), (3, 24)])
def test_cover_every_token_once(assign, n, l):
    shares = [P.positions(assign, n, r, l) for r in range(n)]
    assert all(s.size == l // n for s in shares)
    allpos = np.concatenate(shares)
    assert np.array_equal(np.sort(allpos), np.arange(l))
    for s in shares:  # local order ascending
        assert np.all(np.diff(s) > 0)


def test_bad_sizes_raise():
    with pytest.raises(ValueError):
        P.positions("zigzag", 4, 0, 12)      # 12 % 8 != 0
    with pytest.raises(ValueError):
        P.positions("contiguous", 4, 4, 16)  # rank out of range
