"""GPU parity of both workgroup layouts of the attention kernels (bf16 and fp32).

When one workgroup per query tile would leave a CU with fewer than two workgroups, the launcher
splits each query tile's key tiles between two groups of waves in one workgroup (even and odd
places of the tile sequence) and merges their states through LDS at the end. The small parity
cases of test_gpu_kernels therefore run the split layout by default; here they run again with
RA_KV_SPLIT=never (the layout every large workload uses), and a large share runs with the
split forced, against the oracle and against the unsplit result. The fp32 kernel splits small
grids the same way (four waves on one 64-row query tile, merged in fp64).
"""
import numpy as np
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


@pytest.fixture
def never_split(monkeypatch):
    monkeypatch.setenv("RA_KV_SPLIT", "never")


@pytest.mark.usefixtures("never_split")
@pytest.mark.parametrize("case", K.RING_CASES, ids=[f"{a}-N{n}-L{l}" for a, n, l in K.RING_CASES])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("in_dt", ["bf16", "f32"])
def test_ring_share_parity_unsplit(case, causal, in_dt):
    K.test_ring_share_parity(case, in_dt, causal)


@pytest.mark.usefixtures("never_split")
@pytest.mark.parametrize("assign", K.ASSIGNS)
@pytest.mark.parametrize("in_dt", ["bf16", "f32"])
def test_ring_share_split_and_resume_unsplit(assign, in_dt):
    K.test_ring_share_split_and_resume(in_dt, assign)


@pytest.mark.usefixtures("never_split")
@pytest.mark.parametrize("assign,n,l", [("contiguous", 3, 300), ("striped", 3, 300), ("zigzag", 2, 300)])
def test_ring_share_batched_ragged_unsplit(assign, n, l):
    K.test_ring_share_batched_ragged(assign, n, l, "bf16")


@pytest.mark.usefixtures("never_split")
@pytest.mark.parametrize("assign,n,l,r", [("contiguous", 3, 7500, 2), ("striped", 2, 5000, 1),
                                          ("zigzag", 2, 5000, 0)])
def test_ring_share_tile_groups_unsplit(assign, n, l, r):
    K.test_ring_share_tile_groups(assign, n, l, r)


@pytest.mark.usefixtures("never_split")
@pytest.mark.parametrize("assign", K.ASSIGNS)
@pytest.mark.parametrize("causal", [True, False])
def test_ring_share_64_steps_unsplit(assign, causal):
    K.test_ring_share_64_steps(assign, causal)


@pytest.mark.usefixtures("never_split")
@pytest.mark.parametrize("assign", K.ASSIGNS)
@pytest.mark.parametrize("h,h_kv", [(6, 2), (4, 1), (8, 2)])
def test_ring_share_grouped_query_unsplit(assign, h, h_kv):
    K.test_ring_share_grouped_query(assign, h, h_kv, "bf16")


@pytest.mark.usefixtures("never_split")
@pytest.mark.parametrize("case", K.BLOCK_CASES, ids=[f"c{i}" for i in range(len(K.BLOCK_CASES))])
@pytest.mark.parametrize("o_dt", ["bf16", "f32"])
@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("in_dt", ["bf16", "f32"])
def test_block_attn_parity_unsplit(case, o_dt, d, in_dt):
    K.test_block_attn_parity(case, in_dt, o_dt, d)


@pytest.mark.usefixtures("never_split")
def test_block_attn_all_rows_empty_unsplit():
    K.test_block_attn_all_rows_empty("bf16")


@pytest.mark.usefixtures("never_split")
@pytest.mark.parametrize("assign", K.ASSIGNS)
def test_ring_share_zero_logits_closed_form_unsplit(assign):
    K.test_ring_share_zero_logits_closed_form(assign)


@pytest.mark.usefixtures("never_split")
@pytest.mark.parametrize("assign", K.ASSIGNS)
def test_ring_share_single_visible_key_unsplit(assign):
    K.test_ring_share_single_visible_key(assign)


@pytest.mark.usefixtures("never_split")
def test_future_keys_never_read_unsplit():
    K.test_future_keys_never_read()


@pytest.mark.usefixtures("never_split")
def test_deterministic_unsplit():
    K.test_deterministic()


@pytest.mark.parametrize("assign", K.ASSIGNS)
def test_split_and_unsplit_agree_at_scale(assign, monkeypatch):
    # A share of 16 query tiles x 8 heads on a 4-rank ring, with the split forced on and off:
    # both against the oracle on sampled rows, and against each other.
    # The weights enter the matrix cores rounded to bf16 against the running maximum at the
    # time they are folded, which differs between the layouts, so O may differ by up to the
    # kernel's own error bound; the LSE sums unrounded weights and moves by fp32 rounding only.
    n, l, h, d, r = 4, 4 * 2048, 8, 128, 2
    gq, gk, gv = (K.gen(990 + i, (1, l, h, d), "bf16") for i in range(3))
    qs = K.shares(gq, assign, n)
    kd = [K.dev(x, "bf16") for x in K.shares(gk, assign, n)]
    vd = [K.dev(x, "bf16") for x in K.shares(gv, assign, n)]
    qd = K.dev(qs[r], "bf16")
    res = {}
    for mode in ("never", "always"):
        monkeypatch.setenv("RA_KV_SPLIT", mode)
        K.say(f"kv split {mode}: {assign} N={n} L={l} rank {r}")
        res[mode] = ra.ring_share(qd, kd, vd, r, assign=assign, out_dtype=torch.float32)
    torch.cuda.synchronize()
    (o1, l1), (o2, l2) = res["never"], res["always"]
    assert float((o1 - o2).abs().max()) <= 1e-2
    assert float((l1 - l2).abs().max()) <= 1e-5
    # the split folds the key tiles in another order, so some fp32 output bits differ: this
    # shows that the two calls ran different layouts
    assert not torch.equal(o1, o2)
    rows = np.sort(np.random.default_rng(5).choice(l // n, 96, replace=False))
    qpos = K.OP.positions(assign, n, r, l)
    o_ref, lse_ref = K.OA.attention(K.values(qs[r], "bf16")[:, rows], K.values(gk, "bf16"), K.values(gv, "bf16"),
                                    qpos[rows], np.arange(l), True)
    for o, lse in res.values():
        K.check(K.host(o)[:, rows], K.host(lse)[:, :, rows], o_ref, lse_ref, "bf16", "f32", f"{assign} sampled")
