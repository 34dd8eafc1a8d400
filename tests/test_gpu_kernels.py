"""GPU parity of every entry point against the fp64 oracle, at sizes the oracle finishes in
seconds (several tiles, ragged tails, every assignment, empty rows, both dtypes)."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import (TOL, check, check_grad_entries, delta_error, dev, gen, half_ulp_bf16, host, say,
                         shares, values)
from oracle import attention as OA
from oracle import backward as OB
from oracle import permute as OU
from oracle import positions as OP
from oracle import ring as OR

pytestmark = pytest.mark.gpu

ra = pytest.importorskip("ring_sequence_parallelism_ra_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


ASSIGNS = ["contiguous", "striped", "zigzag"]


def test_positions_at_the_length_limit():
    # the largest global length accepted (the last multiple of 2N = 128 below 2^31) with the
    # largest ring: 32-bit position arithmetic must not overflow anywhere along the share
    n = 64
    l = ((1 << 31) - 1) // (2 * n) * (2 * n)
    for assign in ASSIGNS:
        for r in (0, 17, n - 1):
            say(f"positions {assign} N={n} L={l} rank {r}")
            got = ra.debug_positions(ra.Shard(assign, n, r, l)).cpu().numpy()
            want = OP.positions(assign, n, r, l)
            assert got.shape == want.shape and np.array_equal(got, want)
            assert got.max() < l and got.min() >= 0


@pytest.mark.parametrize("assign", ASSIGNS)
@pytest.mark.parametrize("n,l", [(1, 64), (4, 256), (8, 8192), (8, 262144), (3, 600)])
def test_positions_bit_exact(assign, n, l):
    if assign == "zigzag" and l % (2 * n):
        pytest.skip("zigzag needs L % 2N == 0")
    for r in range(n):
        got = ra.debug_positions(ra.Shard(assign, n, r, l)).cpu().numpy()
        assert np.array_equal(got, OP.positions(assign, n, r, l))


@pytest.mark.parametrize("assign", ASSIGNS)
def test_mask_bit_exact(assign):
    n, l = 4, 512
    s = l // n
    for r in range(n):
        for src in range(n):
            got = ra.debug_mask(ra.Shard(assign, n, r, l), ra.Shard(assign, n, src, l), s, s).cpu().numpy()
            want = OA.visible(OP.positions(assign, n, r, l), OP.positions(assign, n, src, l), True)
            assert np.array_equal(got.astype(bool), want), (r, src)


BLOCK_CASES = [
    # (causal, assign, N, L, q_rank, kv_rank, Sq, Sk) ; non-causal cases use Sq/Sk directly
    (False, None, 0, 0, 0, 0, 300, 200),
    (False, None, 0, 0, 0, 0, 1, 1),
    (False, None, 0, 0, 0, 0, 130, 1000),
    (False, None, 0, 0, 0, 0, 64, 64),
    (True, "contiguous", 4, 1200, 2, 2, 300, 300),
    (True, "contiguous", 4, 1200, 3, 1, 300, 300),
    (True, "striped", 3, 600, 1, 2, 200, 200),
    (True, "striped", 3, 600, 2, 0, 200, 200),
    (True, "zigzag", 2, 520, 0, 1, 260, 260),
    (True, "zigzag", 2, 520, 1, 0, 260, 260),
    (True, "contiguous", 1, 333, 0, 0, 333, 333),
]


@pytest.mark.parametrize("case", BLOCK_CASES, ids=[f"c{i}" for i in range(len(BLOCK_CASES))])
@pytest.mark.parametrize("in_dt,o_dt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"), ("f32", "bf16")])
@pytest.mark.parametrize("d", [128, 64])
def test_block_attn_parity(case, in_dt, o_dt, d):
    causal, assign, n, l, qr, kr, sq, sk = case
    b, h = 2, 3
    seed = 17 + sq + 3 * sk + d
    say(f"block_attn case={case} in={in_dt} out={o_dt} D={d} seed={seed}")
    q, k, v = gen(seed, (b, sq, h, d), in_dt), gen(seed + 1, (b, sk, h, d), in_dt), gen(seed + 2, (b, sk, h, d), in_dt)
    qs = ks = None
    qpos = kpos = None
    if causal:
        qs, ks = ra.Shard(assign, n, qr, l), ra.Shard(assign, n, kr, l)
        qpos, kpos = OP.positions(assign, n, qr, l), OP.positions(assign, n, kr, l)
    o, lse = ra.block_attn_fwd(dev(q, in_dt), dev(k, in_dt), dev(v, in_dt), causal=causal, q_shard=qs, kv_shard=ks,
                               out_dtype=torch.bfloat16 if o_dt == "bf16" else torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = OA.attention(values(q, in_dt), values(k, in_dt), values(v, in_dt), qpos, kpos, causal)
    check(o, lse, o_ref, lse_ref, in_dt, o_dt, what=str(case))


@pytest.mark.parametrize("in_dt", ["bf16", "f32"])
def test_block_attn_all_rows_empty(in_dt):
    # contiguous rank 0's queries precede every key of rank 3: no visible key at all
    n, l = 4, 512
    s = l // n
    q, k, v = (gen(i, (1, s, 2, 128), in_dt) for i in (1, 2, 3))
    o, lse = ra.block_attn_fwd(dev(q, in_dt), dev(k, in_dt), dev(v, in_dt), causal=True,
                               q_shard=ra.Shard("contiguous", n, 0, l), kv_shard=ra.Shard("contiguous", n, 3, l))
    torch.cuda.synchronize()
    assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("in_dt", ["bf16", "f32"])
def test_block_attn_scale(in_dt):
    sq = sk = 96
    q, k, v = (gen(40 + i, (1, sq, 2, 64), in_dt) for i in range(3))
    o, lse = ra.block_attn_fwd(dev(q, in_dt), dev(k, in_dt), dev(v, in_dt), scale=0.3)
    torch.cuda.synchronize()
    o_ref, lse_ref = OA.attention(values(q, in_dt), values(k, in_dt), values(v, in_dt), scale=0.3)
    check(o, lse, o_ref, lse_ref, in_dt, in_dt, "scale=0.3")


RING_CASES = [
    ("contiguous", 4, 4 * 200), ("striped", 4, 4 * 200), ("zigzag", 4, 4 * 200),
    ("contiguous", 8, 8 * 130), ("striped", 8, 8 * 136), ("zigzag", 8, 8 * 130),
    ("zigzag", 2, 2 * 384), ("striped", 1, 300), ("contiguous", 3, 3 * 128),
]


@pytest.mark.parametrize("case", RING_CASES, ids=[f"{a}-N{n}-L{l}" for a, n, l in RING_CASES])
@pytest.mark.parametrize("in_dt", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [True, False])
def test_ring_share_parity(case, in_dt, causal):
    assign, n, l = case
    b, h, d = 1, 2, 128
    seed = 100 + n + l
    say(f"ring_share {case} in={in_dt} causal={causal} seed={seed}")
    gq, gk, gv = (gen(seed + i, (b, l, h, d), in_dt) for i in range(3))
    qs, ks, vs = shares(gq, assign, n), shares(gk, assign, n), shares(gv, assign, n)
    kd = [dev(x, in_dt) for x in ks]
    vd = [dev(x, in_dt) for x in vs]
    kv_full, vv_full = values(gk, in_dt), values(gv, in_dt)
    for r in range(n):
        o, lse = ra.ring_share(dev(qs[r], in_dt), kd, vd, r, assign=assign, causal=causal)
        torch.cuda.synchronize()
        qpos = OP.positions(assign, n, r, l)
        o_ref, lse_ref = OA.attention(values(qs[r], in_dt), kv_full, vv_full, qpos, np.arange(l), causal)
        check(o, lse, o_ref, lse_ref, in_dt, in_dt, what=f"rank {r}")


@pytest.mark.parametrize("in_dt", ["bf16", "f32"])
@pytest.mark.parametrize("assign", ASSIGNS)
def test_ring_share_split_and_resume(in_dt, assign):
    # The state after any prefix of the steps is complete: [0,k) then [k,N), or one step per
    # call, reaches the one-call result (order/block independence, Digest §3.2).
    n, l, b, h, d = 4, 4 * 192, 1, 2, 64
    gq, gk, gv = (gen(300 + i, (b, l, h, d), in_dt) for i in range(3))
    qs, ks, vs = shares(gq, assign, n), shares(gk, assign, n), shares(gv, assign, n)
    kd = [dev(x, in_dt) for x in ks]
    vd = [dev(x, in_dt) for x in vs]
    r = 2
    qd = dev(qs[r], in_dt)
    o1, lse1 = ra.ring_share(qd, kd, vd, r, assign=assign)
    ws = ra.ring_share_workspace(b, h, l // n, d)
    ra.ring_share(qd, kd, vd, r, assign=assign, start_step=0, num_steps=1, ws=ws)
    o2, lse2 = ra.ring_share(qd, kd, vd, r, assign=assign, start_step=1, num_steps=3, ws=ws)
    for st in range(n - 1):
        ra.ring_share(qd, kd, vd, r, assign=assign, start_step=st, num_steps=1, ws=ws)
    o3, lse3 = ra.ring_share(qd, kd, vd, r, assign=assign, start_step=n - 1, num_steps=1, ws=ws)
    torch.cuda.synchronize()
    qpos = OP.positions(assign, n, r, l)
    o_ref, lse_ref = OA.attention(values(qs[r], in_dt), values(gk, in_dt), values(gv, in_dt), qpos, np.arange(l), True)
    for o, lse in ((o1, lse1), (o2, lse2), (o3, lse3)):
        check(o, lse, o_ref, lse_ref, in_dt, in_dt, what="split")


def test_resume_rejects_a_state_stored_by_another_call():
    # the running state's layout depends on the input dtype (log2 units in the bf16 kernel,
    # natural units in the fp32 one); a resume must match the call that stored the state
    n, l, b, h, d = 4, 4 * 128, 1, 2, 64
    gq, gk, gv = (gen(320 + i, (b, l, h, d), "bf16") for i in range(3))
    qs, ks, vs = shares(gq, "zigzag", n), shares(gk, "zigzag", n), shares(gv, "zigzag", n)
    kd, vd = [dev(x, "bf16") for x in ks], [dev(x, "bf16") for x in vs]
    qd = dev(qs[1], "bf16")
    ws = ra.ring_share_workspace(b, h, l // n, d)
    ra.ring_share(qd, kd, vd, 1, assign="zigzag", start_step=0, num_steps=2, ws=ws)
    kf, vf, qf = [x.float() for x in kd], [x.float() for x in vd], qd.float()
    bad = [dict(q=qf, k=kf, v=vf, start_step=2, num_steps=2),                   # other dtype
           dict(q=qd, k=kd, v=vd, start_step=2, num_steps=2, scale=0.3),        # other scale
           dict(q=qd, k=kd, v=vd, start_step=1, num_steps=3),                   # wrong step
           dict(q=qd, k=kd, v=vd, start_step=2, num_steps=2, assign="striped")]  # other ring
    for kw in bad:
        q_, k_, v_ = kw.pop("q"), kw.pop("k"), kw.pop("v")
        kw.setdefault("assign", "zigzag")
        with pytest.raises(ra.RaError) as e:
            ra.ring_share(q_, k_, v_, 1, ws=ws, **kw)
        assert e.value.code == -1 and "resume" in str(e.value), kw
    o, lse = ra.ring_share(qd, kd, vd, 1, assign="zigzag", start_step=2, num_steps=2, ws=ws)
    torch.cuda.synchronize()
    qpos = OP.positions("zigzag", n, 1, l)
    o_ref, lse_ref = OA.attention(values(qs[1], "bf16"), values(gk, "bf16"), values(gv, "bf16"), qpos,
                                  np.arange(l), True)
    check(o, lse, o_ref, lse_ref, "bf16", "bf16", what="matching resume")


@pytest.mark.parametrize("assign,n,l", [("contiguous", 3, 300), ("striped", 3, 300), ("zigzag", 2, 300)])
@pytest.mark.parametrize("in_dt", ["bf16", "f32"])
def test_ring_share_batched_ragged(assign, n, l, in_dt):
    # B > 1, an odd head count, D = 64 and a share length that is no multiple of the tiles, run
    # in one call and resumed over two calls through the workspace state
    b, h, d = 2, 3, 64
    gq, gk, gv = (gen(700 + i, (b, l, h, d), in_dt) for i in range(3))
    qs, ks, vs = shares(gq, assign, n), shares(gk, assign, n), shares(gv, assign, n)
    kd = [dev(x, in_dt) for x in ks]
    vd = [dev(x, in_dt) for x in vs]
    for r in range(n):
        say(f"batched ragged ring {assign} N={n} L={l} rank {r} in={in_dt}")
        qd = dev(qs[r], in_dt)
        o1, l1 = ra.ring_share(qd, kd, vd, r, assign=assign)
        ws = ra.ring_share_workspace(b, h, l // n, d)
        ra.ring_share(qd, kd, vd, r, assign=assign, start_step=0, num_steps=1, ws=ws)
        o2, l2 = ra.ring_share(qd, kd, vd, r, assign=assign, start_step=1, num_steps=n - 1, ws=ws)
        torch.cuda.synchronize()
        qpos = OP.positions(assign, n, r, l)
        o_ref, lse_ref = OA.attention(values(qs[r], in_dt), values(gk, in_dt), values(gv, in_dt), qpos,
                                      np.arange(l), True)
        check(o1, l1, o_ref, lse_ref, in_dt, in_dt, what=f"one call rank {r}")
        check(o2, l2, o_ref, lse_ref, in_dt, in_dt, what=f"resumed rank {r}")


@pytest.mark.parametrize("assign,n,l,r", [("contiguous", 3, 7500, 2), ("striped", 2, 5000, 1),
                                          ("zigzag", 2, 5000, 0)])
def test_ring_share_tile_groups(assign, n, l, r):
    # Shares of 2500 rows (40 tiles of 64 keys): the kernel folds 32-tile groups round-robin
    # over the steps, so these runs cross a group boundary inside fully visible, partially
    # visible and ragged steps; one call and a call resumed after the first step.
    b, h, d = 1, 2, 64
    gq, gk, gv = (gen(1100 + i, (b, l, h, d), "bf16") for i in range(3))
    qs, ks, vs = shares(gq, assign, n), shares(gk, assign, n), shares(gv, assign, n)
    kd = [dev(x, "bf16") for x in ks]
    vd = [dev(x, "bf16") for x in vs]
    say(f"tile groups {assign} N={n} L={l} rank {r}")
    qd = dev(qs[r], "bf16")
    o1, l1 = ra.ring_share(qd, kd, vd, r, assign=assign)
    ws = ra.ring_share_workspace(b, h, l // n, d)
    ra.ring_share(qd, kd, vd, r, assign=assign, start_step=0, num_steps=1, ws=ws)
    o2, l2 = ra.ring_share(qd, kd, vd, r, assign=assign, start_step=1, num_steps=n - 1, ws=ws)
    torch.cuda.synchronize()
    qpos = OP.positions(assign, n, r, l)
    o_ref, lse_ref = OA.attention(values(qs[r], "bf16"), values(gk, "bf16"), values(gv, "bf16"), qpos,
                                  np.arange(l), True)
    check(o1, l1, o_ref, lse_ref, "bf16", "bf16", what="one call")
    check(o2, l2, o_ref, lse_ref, "bf16", "bf16", what="resumed")


@pytest.mark.parametrize("assign", ASSIGNS)
@pytest.mark.parametrize("causal", [True, False])
def test_ring_share_64_steps(assign, causal):
    # The largest ring: one step per lane of the kernel's step table, the last in lane 63.
    n, l, b, h, d = 64, 64 * 64, 1, 2, 64
    gq, gk, gv = (gen(1200 + i, (b, l, h, d), "bf16") for i in range(3))
    qs, ks, vs = shares(gq, assign, n), shares(gk, assign, n), shares(gv, assign, n)
    kd = [dev(x, "bf16") for x in ks]
    vd = [dev(x, "bf16") for x in vs]
    for r in (0, 37, 63):
        say(f"64-step ring {assign} causal={causal} rank {r}")
        o, lse = ra.ring_share(dev(qs[r], "bf16"), kd, vd, r, assign=assign, causal=causal)
        torch.cuda.synchronize()
        qpos = OP.positions(assign, n, r, l)
        o_ref, lse_ref = OA.attention(values(qs[r], "bf16"), values(gk, "bf16"), values(gv, "bf16"), qpos,
                                      np.arange(l), causal)
        check(o, lse, o_ref, lse_ref, "bf16", "bf16", what=f"rank {r}")


@pytest.mark.parametrize("h,h_kv", [(4, 2), (4, 1), (6, 3), (16, 4)])
@pytest.mark.parametrize("in_dt", ["bf16", "f32"])
@pytest.mark.parametrize("d", [128, 64])
def test_block_attn_grouped_query(h, h_kv, in_dt, d):
    # (16 query heads: the bf16 kernel renumbers heads across the XCDs when 8 divides H)
    # GQA / MQA: K and V carry h_kv heads; causal zigzag shards with a ragged-free share and a
    # non-causal ragged block (200 queries, 136 keys)
    b = 2
    n, l = 4, 4 * 96
    qs, ks = OP.positions("zigzag", n, 1, l), OP.positions("zigzag", n, 2, l)
    for causal, sq, sk in ((True, l // n, l // n), (False, 200, 136)):
        say(f"gqa block h={h} h_kv={h_kv} in={in_dt} d={d} causal={causal}")
        q = gen(1400 + h, (b, sq, h, d), in_dt)
        k = gen(1410 + h_kv, (b, sk, h_kv, d), in_dt)
        v = gen(1420 + h_kv, (b, sk, h_kv, d), in_dt)
        kw = dict(causal=True, q_shard=ra.Shard("zigzag", n, 1, l), kv_shard=ra.Shard("zigzag", n, 2, l)) if causal else {}
        o, lse = ra.block_attn_fwd(dev(q, in_dt), dev(k, in_dt), dev(v, in_dt), **kw)
        torch.cuda.synchronize()
        o_ref, lse_ref = OA.attention(values(q, in_dt), values(k, in_dt), values(v, in_dt),
                                      qs if causal else None, ks if causal else None, causal)
        check(o, lse, o_ref, lse_ref, in_dt, in_dt, what=f"causal={causal}")


@pytest.mark.parametrize("assign", ASSIGNS)
@pytest.mark.parametrize("h,h_kv,in_dt", [(6, 2, "bf16"), (4, 1, "bf16"), (6, 2, "f32"), (8, 2, "bf16")])
def test_ring_share_grouped_query(assign, h, h_kv, in_dt):
    n, l, b, d = 4, 4 * 200, 1, 128
    gq = gen(1500, (b, l, h, d), in_dt)
    gk, gv = gen(1501, (b, l, h_kv, d), in_dt), gen(1502, (b, l, h_kv, d), in_dt)
    qs, ks, vs = shares(gq, assign, n), shares(gk, assign, n), shares(gv, assign, n)
    kd = [dev(x, in_dt) for x in ks]
    vd = [dev(x, in_dt) for x in vs]
    for r in (0, n - 1):
        say(f"gqa ring {assign} h={h} h_kv={h_kv} in={in_dt} rank {r}")
        qd = dev(qs[r], in_dt)
        o1, l1 = ra.ring_share(qd, kd, vd, r, assign=assign)
        ws = ra.ring_share_workspace(b, h, l // n, d)
        ra.ring_share(qd, kd, vd, r, assign=assign, start_step=0, num_steps=2, ws=ws)
        o2, l2 = ra.ring_share(qd, kd, vd, r, assign=assign, start_step=2, num_steps=n - 2, ws=ws)
        torch.cuda.synchronize()
        qpos = OP.positions(assign, n, r, l)
        o_ref, lse_ref = OA.attention(values(qs[r], in_dt), values(gk, in_dt), values(gv, in_dt), qpos,
                                      np.arange(l), True)
        check(o1, l1, o_ref, lse_ref, in_dt, in_dt, what=f"one call rank {r}")
        check(o2, l2, o_ref, lse_ref, in_dt, in_dt, what=f"resumed rank {r}")


# Backward tolerance, entry by entry, from the arithmetic (grad_bound in gpu_helpers): P and dS
# enter the matrix cores rounded to bf16 (relative error at most u = 2^-8 per term) and Delta uses
# the bf16 forward output, so each gradient entry may move by u times the sum of the absolute
# values of its terms, plus the Delta error carried through P. The bound is that, doubled.

@pytest.mark.parametrize("assign", ASSIGNS)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("h,h_kv,d", [(2, 2, 128), (4, 2, 64), (4, 1, 128)])
def test_ring_share_bwd_parity(assign, causal, h, h_kv, d):
    # every rank of a 4-rank ring with 200-row shares (ragged against the 64- and 128-row tiles)
    n, l, b = 4, 4 * 200, 1
    gq, gdo = gen(1600, (b, l, h, d), "bf16"), gen(1603, (b, l, h, d), "bf16")
    gk, gv = gen(1601, (b, l, h_kv, d), "bf16"), gen(1602, (b, l, h_kv, d), "bf16")
    qs, ks, vs, dos = (shares(x, assign, n) for x in (gq, gk, gv, gdo))
    kd = [dev(x, "bf16") for x in ks]
    vd = [dev(x, "bf16") for x in vs]
    for r in range(n):
        say(f"ring bwd {assign} causal={causal} h={h} h_kv={h_kv} d={d} rank {r}")
        qpos = OP.positions(assign, n, r, l)
        args = (values(qs[r], "bf16"), values(gk, "bf16"), values(gv, "bf16"), values(dos[r], "bf16"), qpos,
                np.arange(l), causal)
        # the backward's forward inputs come from the oracle (O rounded to bf16, LSE to fp32), so
        # nothing the expected values depend on comes from the GPU
        o_ref, lse_ref = OA.attention(*args[:3], qpos, np.arange(l), causal)
        o_bits = synth.f32_to_bf16_bits(o_ref.astype(np.float32))
        qd, dod = dev(qs[r], "bf16"), dev(dos[r], "bf16")
        o_in, lse_in = dev(o_bits, "bf16"), dev(lse_ref.astype(np.float32), "f32")
        dq, dk, dv = ra.ring_share_bwd(qd, kd, vd, o_in, lse_in, dod, r, assign=assign, causal=causal)
        torch.cuda.synchronize()
        dq_ref, dk_ref, dv_ref = OB.attention_bwd(*args)
        mags = OB.attention_bwd_magnitudes(*args, delta_err=delta_error(values(o_bits, "bf16"), o_ref, args[3]))
        worst = check_grad_entries(dq, dq_ref, mags[0], mags[1], "dq")
        for i in range(n):
            p = OP.positions(assign, n, i, l)
            worst = max(worst, check_grad_entries(dk[i], dk_ref[:, p], mags[2][:, p], mags[3][:, p], f"dk share {i}"),
                        check_grad_entries(dv[i], dv_ref[:, p], mags[4][:, p], 0.0, f"dv share {i}"))
        say(f"  largest error / its entry bound: {worst:.2e}")


def usp_stack(g, ring_pos, u, n):
    """The Ulysses group of one ring rank: that rank's ring share [B, L/r, H, D] (positions
    ring_pos) cut into u consecutive slices of L/N rows, stacked [u, B, L/N, H, D]."""
    b, _, h, d = g.shape
    share = g[:, ring_pos]
    return np.ascontiguousarray(share.reshape(b, u, share.shape[1] // u, h, d).transpose(1, 0, 2, 3, 4))


@pytest.mark.parametrize("u,r,l,h,d", [(2, 2, 1024, 4, 64), (4, 2, 2048, 8, 128), (2, 4, 2048, 4, 64)])
def test_usp_local_step(u, r, l, h, d):
    # USP (Digest §7.2) on one GPU, every device of a u x r mesh: the device's head group of its
    # ring share attends the whole sequence; its O goes back into the group's sequence slices,
    # other heads untouched.
    b, n, hg = 1, u * r, h // u
    gq, gk, gv = (gen(1300 + i, (b, l, h, d), "bf16") for i in range(3))
    ring_pos = [OP.positions("zigzag", r, k, l) for k in range(r)]
    qst = [usp_stack(gq, p, u, n) for p in ring_pos]
    kst = [usp_stack(gk, p, u, n) for p in ring_pos]
    vst = [usp_stack(gv, p, u, n) for p in ring_pos]
    for k in range(r):
        for p in range(u):
            say(f"usp u={u} r={r} L={l} ulysses rank {p} ring rank {k}")
            k_heads = [ra.seq2head_permute(dev(x, "bf16"), p) for x in kst]
            v_heads = [ra.seq2head_permute(dev(x, "bf16"), p) for x in vst]
            fill = np.full((u, b, l // n, h, d), 0x40E0, dtype=np.uint16)  # 7.0
            out, o, lse = ra.usp_local_step(dev(qst[k], "bf16"), k_heads, v_heads, p, k, out=dev(fill, "bf16"))
            torch.cuda.synchronize()
            heads = slice(p * hg, (p + 1) * hg)
            o_ref, lse_ref = OA.attention(values(gq[:, ring_pos[k]][:, :, heads], "bf16"),
                                          values(gk[:, :, heads], "bf16"), values(gv[:, :, heads], "bf16"),
                                          ring_pos[k], np.arange(l), True)
            check(o, lse, o_ref, lse_ref, "bf16", "bf16", what=f"p={p} k={k}")
            want = OU.head2seq(o.cpu().view(torch.int16).numpy(), p, fill.view(np.int16).copy())
            assert np.array_equal(out.cpu().view(torch.int16).numpy(), want)


@pytest.mark.parametrize("assign", ASSIGNS)
def test_ring_share_zero_logits_closed_form(assign):
    # Q = 0 makes every logit 0, so the whole ring reduces to counting and averaging: the row at
    # global position p sees exactly the p + 1 keys at positions 0..p (the N shares cover the
    # sequence), hence LSE = ln(p + 1) and O = mean of V over positions 0..p. This pins the causal
    # mask, the ring order and the online update on the GPU without the oracle's attention code.
    n, l, b, h, d = 4, 4 * 256, 1, 2, 128
    gk, gv = (gen(800 + i, (b, l, h, d), "bf16") for i in range(2))
    gq = np.zeros((b, l, h, d), dtype=np.uint16)
    kd = [dev(x, "bf16") for x in shares(gk, assign, n)]
    vd = [dev(x, "bf16") for x in shares(gv, assign, n)]
    vcum = np.cumsum(values(gv, "bf16").astype(np.float64), axis=1)  # [b, l, h, d] prefix sums
    for r in range(n):
        qpos = OP.positions(assign, n, r, l)
        qd = dev(np.ascontiguousarray(gq[:, qpos]), "bf16")
        o, lse = ra.ring_share(qd, kd, vd, r, assign=assign, out_dtype=torch.float32)
        torch.cuda.synchronize()
        cnt = (qpos + 1).astype(np.float64)
        lse_want = np.broadcast_to(np.log(cnt)[None, None, :], (b, h, qpos.size))
        o_want = vcum[:, qpos] / cnt[None, :, None, None]
        assert np.abs(host(lse) - lse_want).max() < 5e-6, f"rank {r} LSE"
        assert np.abs(host(o) - o_want).max() < 2e-5, f"rank {r} O"


@pytest.mark.parametrize("assign", ASSIGNS)
def test_ring_share_single_visible_key(assign):
    # The row at global position 0 (local row 0 of rank 0 in every assignment) sees only its own
    # key: O = v_0 and LSE = scale * q_0 . k_0, whatever the other keys hold.
    n, l, b, h, d = 4, 4 * 128, 1, 2, 128
    gq, gk, gv = (gen(900 + i, (b, l, h, d), "bf16") for i in range(3))
    qpos = OP.positions(assign, n, 0, l)
    assert qpos[0] == 0
    o, lse = ra.ring_share(dev(np.ascontiguousarray(gq[:, qpos]), "bf16"), [dev(x, "bf16") for x in shares(gk, assign, n)],
                           [dev(x, "bf16") for x in shares(gv, assign, n)], 0, assign=assign, out_dtype=torch.float32)
    torch.cuda.synchronize()
    q0, k0, v0 = (values(x, "bf16")[:, 0].astype(np.float64) for x in (gq, gk, gv))  # [b, h, d]
    lse_want = (q0 * k0).sum(-1) / np.sqrt(d)
    assert np.abs(host(lse)[:, :, 0] - lse_want).max() < 1e-5
    assert np.abs(host(o)[:, 0] - v0).max() < 1e-6


@pytest.mark.parametrize("acc_dt,blk_dt", [("f32", "f32"), ("f32", "bf16"), ("bf16", "f32"), ("bf16", "bf16")])
@pytest.mark.parametrize("d", [128, 64, 8])
def test_lse_merge_parity(acc_dt, blk_dt, d):
    b, s, h = 2, 77, 3
    rng = np.random.default_rng(d)
    oa, ob = gen(500 + d, (b, s, h, d), acc_dt), gen(600 + d, (b, s, h, d), blk_dt)
    la = rng.standard_normal((b, h, s)).astype(np.float32) * 5
    lb = rng.standard_normal((b, h, s)).astype(np.float32) * 5
    la[0, 0, :5] = -np.inf
    lb[0, 0, 3:8] = -np.inf     # rows 3, 4 are empty on both sides
    lb[1, 2, 10] = la[1, 2, 10]  # a tie
    oad, lad = dev(oa, acc_dt), torch.from_numpy(la).cuda()
    ra.lse_merge(oad, lad, dev(ob, blk_dt), torch.from_numpy(lb).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = OR.lse_merge(values(oa, acc_dt), np.transpose(la, (0, 2, 1)), values(ob, blk_dt),
                                np.transpose(lb, (0, 2, 1)))
    l_ref = np.transpose(l_ref, (0, 2, 1))
    bound = 2e-6 + (half_ulp_bf16(o_ref) if acc_dt == "bf16" else 0.0)
    assert np.all(np.abs(host(oad) - o_ref) <= bound)
    got_l = host(lad)
    assert np.array_equal(np.isneginf(got_l), np.isneginf(l_ref))
    fin = np.isfinite(l_ref)
    assert np.max(np.abs(got_l[fin] - l_ref[fin])) <= 2e-6
    assert np.all(host(oad)[0, 3:5, 0] == 0)


@pytest.mark.parametrize("p", [2, 4, 8])
@pytest.mark.parametrize("hmul", [1, 2])
@pytest.mark.parametrize("s", [1, 3, 64])
@pytest.mark.parametrize("d,dt", [(128, "bf16"), (64, "bf16"), (64, "f32"), (1, "bf16"), (3, "f32")])
def test_permute_bit_exact(p, hmul, s, d, dt):
    h, b = p * hmul, 2
    x = gen(700 + p + s + d, (p, b, s, h, d), dt)
    xd = dev(x, dt)
    for dst in (0, p - 1, -1):
        y = ra.seq2head_permute(xd, dst)
        torch.cuda.synchronize()
        want = OU.seq2head(x, dst)
        got = y.cpu().view(torch.int16 if dt == "bf16" else torch.int32).numpy()
        assert np.array_equal(got, want.view(np.int16 if dt == "bf16" else np.int32))
        fill = np.full_like(x, 0x3f80 if dt == "bf16" else 7)
        out = dev(fill, dt)
        ra.head2seq_permute(y, dst, out)
        torch.cuda.synchronize()
        want_back = OU.head2seq(want, dst, fill.copy())
        got_back = out.cpu().view(torch.int16 if dt == "bf16" else torch.int32).numpy()
        assert np.array_equal(got_back, want_back.view(np.int16 if dt == "bf16" else np.int32))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("p,hmul,s,d,nt", [(8, 1, 64, 128, 3), (4, 2, 3, 64, 2), (2, 3, 5, 1, 8), (8, 4, 17, 8, 1)])
def test_permute_n_bit_exact(p, hmul, s, d, nt, dt):
    # several tensors in one launch, each exactly as the one-tensor permute (and the oracle)
    h, b = p * hmul, 2
    xs = [gen(760 + i, (p, b, s, h, d), dt) for i in range(nt)]
    xd = [dev(x, dt) for x in xs]
    iv = torch.int16 if dt == "bf16" else torch.int32
    nv = np.int16 if dt == "bf16" else np.int32
    for dst in (p - 1, -1):
        ys = ra.seq2head_permute_n(xd, dst)
        torch.cuda.synchronize()
        for x, y in zip(xs, ys):
            assert np.array_equal(y.cpu().view(iv).numpy(), OU.seq2head(x, dst).view(nv))
        fills = [np.full_like(x, 0x3f80 if dt == "bf16" else 7) for x in xs]
        outs = [dev(f, dt) for f in fills]
        ra.seq2head_permute_n(ys, dst, outs, inverse=True)
        torch.cuda.synchronize()
        for f, x, o in zip(fills, xs, outs):
            want = OU.head2seq(OU.seq2head(x, dst), dst, f.copy())
            assert np.array_equal(o.cpu().view(iv).numpy(), want.view(nv))


def test_future_keys_never_read():
    # Keys later than every query of the share are invisible: filling them with +-1e4 garbage
    # must leave O and LSE bit-identical (tile skipping and masking together).
    assign, n, l, b, h, d = "striped", 4, 1024, 1, 2, 128
    gq, gk, gv = (gen(900 + i, (b, l, h, d), "bf16") for i in range(3))
    r = 1
    qpos = OP.positions(assign, n, r, l)
    qs = shares(gq, assign, n)
    o1, lse1 = ra.ring_share(dev(qs[r], "bf16"), [dev(x, "bf16") for x in shares(gk, assign, n)],
                             [dev(x, "bf16") for x in shares(gv, assign, n)], r, assign=assign)
    for x in (gk, gv):
        late = np.arange(l) > qpos.max()
        junk = np.where(np.random.default_rng(0).random(x[:, late].shape) < 0.5, 0x461C, 0xC61C)  # +-1e4
        x[:, late] = junk.astype(np.uint16)
    o2, lse2 = ra.ring_share(dev(qs[r], "bf16"), [dev(x, "bf16") for x in shares(gk, assign, n)],
                             [dev(x, "bf16") for x in shares(gv, assign, n)], r, assign=assign)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32))


def test_deterministic():
    assign, n, l = "zigzag", 8, 8 * 256
    gq, gk, gv = (gen(950 + i, (1, l, 4, 128), "bf16") for i in range(3))
    kd = [dev(x, "bf16") for x in shares(gk, assign, n)]
    vd = [dev(x, "bf16") for x in shares(gv, assign, n)]
    qd = dev(shares(gq, assign, n)[5], "bf16")
    o1, l1 = ra.ring_share(qd, kd, vd, 5, assign=assign)
    o2, l2 = ra.ring_share(qd, kd, vd, 5, assign=assign)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
