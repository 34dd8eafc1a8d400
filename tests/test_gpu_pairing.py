"""GPU parity of the bf16 causal kernel with paired query tiles (RA_PAIR_TILES=always).

A workgroup then takes query tiles n_qt-1-p and p, the first walked forward over its (step,
key tile) sequence and the second backward. The automatic choice pairs only striped shares on
grids large enough to fill the GPU twice over, which the small parity cases never are; these
tests rerun them with pairing forced, so ragged tails, odd tile counts (a middle tile left
alone), resumed rings, tile-group boundaries, 64-step rings and grouped KV heads all go through
the paired path (the unsplit layout: RA_KV_SPLIT=never, since pairing is not combined with the
key split), with the tile groups of 8 and of 32 tiles (RA_PAIR_GROUP). The oracle comparisons are
those of test_gpu_kernels.
"""
import pytest
import torch

import test_gpu_kernels as K

pytestmark = pytest.mark.gpu

ra = pytest.importorskip("ring_sequence_parallelism_ra_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


@pytest.fixture(autouse=True, params=["short", "long"])
def _always_pair(monkeypatch, request):
    # both paired instantiations: tile groups of 8 (chosen for short shares) and of 32
    monkeypatch.setenv("RA_PAIR_TILES", "always")
    monkeypatch.setenv("RA_KV_SPLIT", "never")
    monkeypatch.setenv("RA_PAIR_GROUP", request.param)


@pytest.mark.parametrize("case", K.RING_CASES, ids=[f"{a}-N{n}-L{l}" for a, n, l in K.RING_CASES])
def test_ring_share_parity_paired(case):
    K.test_ring_share_parity(case, "bf16", True)


@pytest.mark.parametrize("assign", K.ASSIGNS)
def test_ring_share_split_and_resume_paired(assign):
    K.test_ring_share_split_and_resume("bf16", assign)


@pytest.mark.parametrize("assign,n,l", [("contiguous", 3, 300), ("striped", 3, 300), ("zigzag", 2, 300)])
def test_ring_share_batched_ragged_paired(assign, n, l):
    K.test_ring_share_batched_ragged(assign, n, l, "bf16")


@pytest.mark.parametrize("assign,n,l,r", [("contiguous", 3, 7500, 2), ("striped", 2, 5000, 1),
                                          ("zigzag", 2, 5000, 0)])
def test_ring_share_tile_groups_paired(assign, n, l, r):
    K.test_ring_share_tile_groups(assign, n, l, r)


@pytest.mark.parametrize("assign", K.ASSIGNS)
def test_ring_share_64_steps_paired(assign):
    K.test_ring_share_64_steps(assign, True)


@pytest.mark.parametrize("assign", K.ASSIGNS)
@pytest.mark.parametrize("h,h_kv", [(6, 2), (4, 1), (8, 2)])
def test_ring_share_grouped_query_paired(assign, h, h_kv):
    K.test_ring_share_grouped_query(assign, h, h_kv, "bf16")


@pytest.mark.parametrize("case", [c for c in K.BLOCK_CASES if c[0]],
                         ids=[f"c{i}" for i, c in enumerate(K.BLOCK_CASES) if c[0]])
@pytest.mark.parametrize("o_dt", ["bf16", "f32"])
def test_block_attn_parity_paired(case, o_dt):
    K.test_block_attn_parity(case, "bf16", o_dt, 128)


@pytest.mark.parametrize("assign", K.ASSIGNS)
def test_ring_share_zero_logits_closed_form_paired(assign):
    K.test_ring_share_zero_logits_closed_form(assign)


@pytest.mark.parametrize("assign", K.ASSIGNS)
def test_ring_share_single_visible_key_paired(assign):
    K.test_ring_share_single_visible_key(assign)


def test_future_keys_never_read_paired():
    K.test_future_keys_never_read()


def test_deterministic_paired():
    K.test_deterministic()


def test_paired_and_unpaired_agree(monkeypatch):
    # Same inputs, both assignments of query tiles to workgroups: equal up to the rounding of a
    # different fold order. The weights enter the matrix cores rounded to bf16 against the
    # running maximum at the time they are folded, so O may differ by the kernel's own error
    # bound (1e-2); the LSE sums unrounded weights in fp32 and moves only by fp32 rounding.
    assign, n, l = "zigzag", 4, 4 * 520
    gq, gk, gv = (K.gen(970 + i, (1, l, 4, 128), "bf16") for i in range(3))
    kd = [K.dev(x, "bf16") for x in K.shares(gk, assign, n)]
    vd = [K.dev(x, "bf16") for x in K.shares(gv, assign, n)]
    qd = K.dev(K.shares(gq, assign, n)[2], "bf16")
    o1, l1 = ra.ring_share(qd, kd, vd, 2, assign=assign, out_dtype=torch.float32)
    monkeypatch.setenv("RA_PAIR_TILES", "never")
    o2, l2 = ra.ring_share(qd, kd, vd, 2, assign=assign, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert float((o1 - o2).abs().max()) <= 1e-2
    assert float((l1 - l2).abs().max()) <= 1e-5
    # the second query tile of every pair folds its key tiles in reverse order, so some fp32
    # output bits differ: this shows that the two calls ran different layouts
    assert not torch.equal(o1, o2)
