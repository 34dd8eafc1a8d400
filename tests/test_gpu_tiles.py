"""Device-side tile counts of the bf16 attention kernel against the oracle's tiled walk: the
tiles each wave actually folds in (every tile with a visible pair for its query tile, none of
the skipped upper triangle of the causal matrix, [Digest] §3.4) and the tiles on which it
evaluates the mask, exactly, in every workgroup layout, with the counting copy's outputs
bit-identical to the product call's; the counting copy's own per-tile bounds and visibility
checks report no fault."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, gen, say, shares
from oracle import counts as OC
from oracle import positions as OP

pytestmark = pytest.mark.gpu

ra = pytest.importorskip("ring_sequence_parallelism_ra_amd")

BM, BN, WR = 128, 64, 32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def expected(assign, n, r, L, causal):
    qpos = OP.positions(assign, n, r, L)
    steps = [OP.positions(assign, n, (r - s) % n, L) for s in range(n)]
    return OC.tiled_walk(qpos, steps, BM, BN, WR, causal)


def check_counts(counts, vis, msk, s_loc, what):
    c = counts.cpu().numpy().astype(np.int64)           # [n_qt, B, H, 8, 4]
    n_qt = c.shape[0]
    assert vis.shape == (n_qt,), what
    # the walk's own checks: no copied or folded tile outside its step's visible tiles, no
    # folded tile that the query tile cannot see
    assert not c[..., 2].any(), f"{what}: bounds faults {int(c[..., 2].sum())}"
    assert not c[..., 3].any(), f"{what}: folded tiles no query row sees {int(c[..., 3].sum())}"
    fold = c[..., 0]
    mask = c[..., 1]
    # the two wave groups of a key-split workgroup share the query rows: sum them per wave
    fold_w = fold[..., :4] + fold[..., 4:]
    mask_w = mask[..., :4] + mask[..., 4:]
    live = (np.arange(n_qt)[:, None] * BM + np.arange(4)[None, :] * WR) < s_loc   # [n_qt, 4]
    want_fold = np.where(live, vis[:, None], 0)                                     # [n_qt, 4]
    assert np.array_equal(fold_w, np.broadcast_to(want_fold[:, None, None, :], fold_w.shape)), \
        f"{what}: folded tiles differ from the oracle's visited tiles"
    assert np.array_equal(mask_w, np.broadcast_to(np.where(live, msk, 0)[:, None, None, :], mask_w.shape)), \
        f"{what}: masked tiles differ"
    # a key split gives group 0 the tiles at even places of the walk and group 1 the odd ones
    if fold[..., 4:].any():
        assert np.array_equal(fold[..., :4], (fold_w + 1) // 2) and np.array_equal(fold[..., 4:], fold_w // 2), what
    total = int(vis.sum())
    return total


def run_case(assign, n, s_loc, h, d, causal, b=1, seed=2100):
    L = n * s_loc
    gq, gk, gv = (gen(seed + i, (b, L, h, d), "bf16") for i in range(3))
    qs, ks, vs = shares(gq, assign, n), shares(gk, assign, n), shares(gv, assign, n)
    kd = [dev(x, "bf16") for x in ks]
    vd = [dev(x, "bf16") for x in vs]
    for r in sorted({0, n // 2, n - 1}):
        qd = dev(qs[r], "bf16")
        o, lse, cnt = ra.debug_tile_counts(qd, kd, vd, r, assign=assign, causal=causal)
        o2, lse2 = ra.ring_share(qd, kd, vd, r, assign=assign, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2), \
            "the counting copy must compute exactly what the product kernel does"
        vis, msk = expected(assign, n, r, L, causal)
        check_counts(cnt, vis, msk, s_loc, f"{assign} n={n} s={s_loc} r={r} causal={causal}")


@pytest.mark.parametrize("layout", [{}, {"RA_KV_SPLIT": "always"}, {"RA_KV_SPLIT": "never"},
                                    {"RA_PAIR_TILES": "always", "RA_KV_SPLIT": "never"},
                                    {"RA_PAIR_TILES": "always", "RA_KV_SPLIT": "never", "RA_PAIR_GROUP": "long"}])
@pytest.mark.parametrize("assign", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("n,s_loc,causal", [(4, 256, True), (3, 200, True), (8, 384, True), (1, 520, True),
                                            (4, 200, False)])
def test_tile_counts_small(monkeypatch, layout, assign, n, s_loc, causal):
    for k, v in layout.items():
        monkeypatch.setenv(k, v)
    say(f"tile counts {assign} n={n} s={s_loc} causal={causal} layout={layout}")
    run_case(assign, n, s_loc, 2, 128, causal, b=2)


@pytest.mark.parametrize("assign", ["striped", "zigzag"])
def test_tile_counts_head_dim_64(assign):
    run_case(assign, 4, 320, 3, 64, True)


@pytest.mark.parametrize("name", ["contig_rank7", "striped_rank0", "zigzag_rank3"])
def test_tile_counts_workloads(name):
    # the workloads' shapes and launch layouts (key split for the short contiguous share, paired
    # tiles for the striped one, one tile per workgroup for the long zigzag share); the counts do
    # not depend on the values, which are drawn on the device
    import synth
    w = synth.get(name)
    n, r, L, s = w.world, w.rank, w.global_len, w.share_len
    g = torch.Generator(device="cuda").manual_seed(w.number)
    shape = (w.batch, s, w.heads, w.head_dim)
    q = torch.randn(shape, device="cuda", generator=g).to(torch.bfloat16)
    kd = [torch.randn(shape, device="cuda", generator=g).to(torch.bfloat16) for _ in range(n)]
    vd = [torch.randn(shape, device="cuda", generator=g).to(torch.bfloat16) for _ in range(n)]
    say(f"tile counts {name}")
    o, lse, cnt = ra.debug_tile_counts(q, kd, vd, r, assign=w.assign)
    o2, lse2 = ra.ring_share(q, kd, vd, r, assign=w.assign)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)
    vis, msk = expected(w.assign, n, r, L, True)
    total = check_counts(cnt, vis, msk, s, name)
    # against the tile classes of the same tiling: visited = full + partial, the rest skipped
    qpos = OP.positions(w.assign, n, r, L)
    cls = [OC.tile_classes(qpos, OP.positions(w.assign, n, src, L), BM, BN) for src in range(n)]
    full, part, skip = (sum(x[i] for x in cls) for i in range(3))
    assert total == full + part
    say(f"  {name}: {total} tiles visited, {skip} skipped per head; "
        f"{int(cnt[..., 1].sum().item()) // (w.batch * w.heads)} wave-tiles masked per head")
