"""Pins for oracle.permute: index formula on arange payloads, head ownership, exact inverses."""
import numpy as np
import pytest

from oracle import permute as U


def test_head_ownership_page(golden):
    for (p, h, dst), heads in golden("ulysses_heads_p4_h8.txt"):
        s, d = 3, 2
        x = np.zeros((p, 1, s, h, d), dtype=np.int64)
        for hh in range(h):
            x[:, :, :, hh, :] = hh
        y = U.seq2head(x, dst)
        assert sorted(set(y[0, :, :, 0].ravel().tolist())) == heads
        assert y.shape == (1, p * s, h // p, d)


def test_sequence_order_by_source_rank():
    p, b, s, h, d = 4, 2, 3, 8, 5
    x = np.arange(p * b * s * h * d).reshape(p, b, s, h, d)
    for dst in range(p):
        y = U.seq2head(x, dst)
        hp = h // p
        for src in range(p):
            for si in range(s):
                for hh in range(hp):
                    assert np.array_equal(y[:, src * s + si, hh], x[src, :, si, dst * hp + hh])


@pytest.mark.parametrize("p", [2, 4, 8])
@pytest.mark.parametrize("hmul", [1, 2])
@pytest.mark.parametrize("s", [1, 3, 64])
@pytest.mark.parametrize("d", [1, 64, 128])
def test_exact_inverse(p, hmul, s, d):
    h = p * hmul
    b = 1
    x = np.arange(p * b * s * h * d, dtype=np.int64).reshape(p, b, s, h, d)
    y_all = U.seq2head(x, -1)
    back = U.head2seq(y_all, -1, np.full_like(x, -1))
    assert np.array_equal(back, x)
    y_again = U.seq2head(back, -1)
    assert np.array_equal(y_again, y_all)
    # one rank's inverse writes only its own head slice
    dst = p - 1
    part = U.head2seq(U.seq2head(x, dst), dst, np.full_like(x, -1))
    hp = h // p
    assert np.array_equal(part[:, :, :, dst * hp:(dst + 1) * hp], x[:, :, :, dst * hp:(dst + 1) * hp])
    assert np.all(np.delete(part, np.s_[dst * hp:(dst + 1) * hp], axis=3) == -1)


def test_heads_not_divisible():
    with pytest.raises(ValueError):
        U.seq2head(np.zeros((4, 1, 2, 6, 2)), 0)
