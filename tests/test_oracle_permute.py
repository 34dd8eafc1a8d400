"""Pins for oracle.permute: the whole-tensor statement of [Digest] §5.1 (shares of a global
tensor in, head slices of the same global tensor out), head ownership, exact inverses."""
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


@pytest.mark.parametrize("p,hmul,s", [(2, 1, 3), (4, 2, 5), (8, 1, 2)])
def test_global_tensor_identity(p, hmul, s):
    # [Digest] §5.1 stated on a whole tensor: the sequence [B, L, H, D] is cut into P contiguous
    # runs of L/P rows (rank src holds rows src*L/P ..), every head; after the all-to-all, rank p
    # holds the WHOLE sequence in its natural order for heads [p*H/P, (p+1)*H/P). So the
    # layout change of the stacked shares must equal plain slicing of the global tensor.
    b, h, d = 2, p * hmul, 3
    L = p * s
    g = np.random.default_rng(p * 100 + s).integers(-1000, 1000, size=(b, L, h, d))
    stack = np.stack([g[:, src * s:(src + 1) * s] for src in range(p)])   # [P, B, L/P, H, D]
    hp = h // p
    for dst in range(p):
        assert np.array_equal(U.seq2head(stack, dst), g[:, :, dst * hp:(dst + 1) * hp])
    assert np.array_equal(U.seq2head(stack, -1), np.stack([g[:, :, q * hp:(q + 1) * hp] for q in range(p)]))
    # and the reverse: writing rank dst's head slice of the global tensor back yields the shares
    # with exactly that head slice filled in, in sequence order
    for dst in range(p):
        back = U.head2seq(g[:, :, dst * hp:(dst + 1) * hp], dst, np.zeros_like(stack))
        want = np.zeros_like(stack)
        want[:, :, :, dst * hp:(dst + 1) * hp] = stack[:, :, :, dst * hp:(dst + 1) * hp]
        assert np.array_equal(back, want)
    every = U.head2seq(np.stack([g[:, :, q * hp:(q + 1) * hp] for q in range(p)]), -1, np.zeros_like(stack))
    assert np.array_equal(every, stack)


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
