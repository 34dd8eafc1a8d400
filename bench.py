#!/usr/bin/env python3
"""Throughput of the per-device Ring Attention inner loop on one MI355X.

A step is one ``ra_ring_share`` call: every ring step of one rank's share (token positions,
tile classification, QK^T, causal mask, online softmax, PV, epilogue) on the long zigzag
workload -- B=1, H=16, D=128, L=262144 over N=8 ranks in 16 chunks of 16384, rank 3's
32768 queries against all 8 KV shares, bf16 inputs, fp32 accumulation. The value is
causal-adjusted TFLOP/s: 4*D FLOPs per visible (query, key) pair per head, the pairs counted
by the library's planner from the same position rule the kernel uses.

Also reported in the same JSON line (``secondary``): the other workloads (contiguous
rank 7 of L=8192, striped rank 0 of L=32768 at std 1 and 4, grouped-query attention with 64
query heads on 8 KV heads on a zigzag ring of L=65536, the Ulysses local step of
L=65536 with its permutes, one device of a 128K-token USP mesh with Ulysses degree 4 and a
zigzag ring of 2, the backward pass of the headline share, the heaviest rank of each token
assignment at the pages' Striped Attention sizes, the tiny exact fp32 ring), the LSE-merge
bandwidth, the
roofline of the attention kernel and the oracle timed on the host cores (``cpu_baseline``).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary | --secondary a,b,...]
                       [--no-cpu-baseline]

``--secondary`` runs only the named secondary workloads (for short profiling runs); their
names are the keys of ``secondary`` in the JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal-adjusted attention TFLOP/s per GPU share; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
HEADLINE = "zigzag_rank3"
SETTLE_S = 0.3              # warm-up and minimum timed span of the short secondary workloads
KERNEL_SRC = [os.path.join(ROOT, "ring_sequence_parallelism_ra_amd", "csrc", f)
              for f in ("attn_bf16.hip", "attn_bf16_tile.inc")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_zigzag_rank3_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def to_dev(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def ring_inputs(w):
    """Q share and the N K/V shares of a ring workload, gathered on the device by the
    library's own position rule."""
    import torch

    import ring_sequence_parallelism_ra_amd as ra
    import synth
    gq, gk, gv = synth.global_qkv(w)
    n, L = w.world, w.global_len
    pos = [ra.debug_positions(ra.Shard(w.assign, n, s, L)) for s in range(n)]
    out = {}
    for name, g in (("q", gq), ("k", gk), ("v", gv)):
        t = to_dev(g)
        if name == "q":
            out["q"] = torch.index_select(t, 1, pos[w.rank]).contiguous()
        else:
            out[name] = [torch.index_select(t, 1, p).contiguous() for p in pos]
        del t
    torch.cuda.synchronize()
    return out, (gq, gk, gv)


def ring_pairs(w) -> int:
    import ring_sequence_parallelism_ra_amd as ra
    n, L, s = w.world, w.global_len, w.share_len
    q_sh = ra.Shard(w.assign, n, w.rank, L)
    return sum(ra.share_work(q_sh, ra.Shard(w.assign, n, src, L), s, s, True)[0] for src in range(n))


TIMES = {}  # event statistics of the last time_calls of each callable: min, median, mean, count


def time_calls(fn, steps, warmup, settle_s=0.0):
    """(wall ms per call over ``steps`` back-to-back calls, mean event ms per call, median); the
    minimum, median, mean and count of the per-call events are also left in TIMES[id(fn)].

    With ``settle_s`` > 0 (the short secondary workloads) the warm-up goes on for at least that
    many seconds and at least that many seconds are timed: a call of a millisecond or two right
    after an idle spell runs before the shader clock has ramped up (measured in-kernel: 1.38 GHz
    on a first call vs 1.70 GHz after ~50 ms of back-to-back calls)."""
    import torch
    t0 = time.perf_counter()
    n_warm = 0
    while n_warm < warmup or time.perf_counter() - t0 < settle_s:
        fn()
        n_warm += 1
        if settle_s > 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    if settle_s > 0 and n_warm:
        per_call = (time.perf_counter() - t0) / n_warm
        steps = max(steps, int(settle_s / max(per_call, 1e-6)) + 1)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ev = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    TIMES[id(fn)] = {"min": min(ev), "median": sorted(ev)[len(ev) // 2], "mean": sum(ev) / len(ev), "n": len(ev)}
    return wall, sum(ev) / len(ev), sorted(ev)[len(ev) // 2]


def tile_walk(inp, w):
    """Tiles the kernel really visits on a ring workload, counted on the device by the
    tile-counting copy of the kernel (one untimed call), next to the planner's tile classes:
    the skipped upper triangle of the causal matrix."""
    import ring_sequence_parallelism_ra_amd as ra
    _, _, cnt = ra.debug_tile_counts(inp["q"], inp["k"], inp["v"], w.rank, assign=w.assign)
    c = cnt.cpu().long()
    folded = int(c[..., 0].sum()) // 4           # each of the 4 waves of a query tile folds every tile
    masked = int(c[..., 1].sum())
    faults = int(c[..., 2].sum()) + int(c[..., 3].sum())
    n, L, s = w.world, w.global_len, w.share_len
    bm, bn = ra.tile_shape(ra.BF16, w.head_dim)
    q_sh = ra.Shard(w.assign, n, w.rank, L)
    cls = [ra.share_work(q_sh, ra.Shard(w.assign, n, src, L), s, s, True, bm, bn) for src in range(n)]
    full, part, skip = (sum(x[i] for x in cls) * w.batch * w.heads for i in (1, 2, 3))
    return {"visited_tiles": folded, "planner_full_plus_partial": full + part, "skipped_tiles": skip,
            "skipped_fraction": round(skip / (full + part + skip), 4), "masked_wave_tiles": masked,
            "masked_fraction_of_wave_tiles": round(masked / max(1, 4 * folded), 5), "walk_faults": faults}


def bench_ring(name, steps, warmup, settle_s=0.0, tiles=False):
    import torch

    import ring_sequence_parallelism_ra_amd as ra
    import synth
    w = synth.get(name)
    t0 = time.perf_counter()
    inp, host = ring_inputs(w)
    log(f"[bench] {name}: inputs ready in {time.perf_counter() - t0:.1f}s")
    call, o, lse = ra.prepare_ring_share(inp["q"], inp["k"], inp["v"], w.rank, assign=w.assign, causal=True)
    flops = 4 * w.head_dim * w.batch * w.heads * ring_pairs(w)
    wall, ev_mean, ev_med = time_calls(call, steps, warmup, settle_s)
    res = {"tflops": flops / (wall * 1e-3) / 1e12, "kernel_ms_mean": ev_mean, "kernel_ms_median": ev_med,
           "kernel_ms_min": TIMES[id(call)]["min"], "ms_per_step": wall, "flops": flops}
    if tiles:
        res["tile_walk"] = tile_walk(inp, w)
    del inp, o, lse
    torch.cuda.empty_cache()
    return res, host, w


def bench_ulysses(steps, warmup):
    import torch

    import ring_sequence_parallelism_ra_amd as ra
    import synth
    w = synth.get("ulysses_local")
    gq, gk, gv = synth.global_qkv(w)
    P, L, H, D, B = w.world, w.global_len, w.heads, w.head_dim, w.batch
    s_loc = L // P
    stacks = [to_dev(g).view(B, P, s_loc, H, D).transpose(0, 1).contiguous() for g in (gq, gk, gv)]
    del gq, gk, gv
    moved = 2 * B * L * (H // P) * D * 2  # read + write bytes of one tensor's permute
    # Bandwidth with rotated buffers, so that successive calls read and write different regions
    # (no Infinity Cache reuse between calls): the destination rank rotates over the 8 head slices
    # of the three 256 MiB stacks, the outputs over 4 buffers per tensor.
    outs = [[torch.empty((B, L, H // P, D), dtype=torch.bfloat16, device="cuda") for _ in range(3)] for _ in range(4)]
    idx = [0]

    def perm_one():
        i = idx[0]
        ra.seq2head_permute(stacks[i % 3], (i // 3) % P, out=outs[i % 4][i % 3])
        idx[0] += 1

    def perm_qkv():
        i = idx[0]
        ra.seq2head_permute_n(stacks, i % P, outs=outs[i % 4])
        idx[0] += 1

    nperm = max(steps, 24)
    time_calls(perm_one, nperm, 3, SETTLE_S)
    t_one = TIMES[id(perm_one)]
    time_calls(perm_qkv, nperm, 3, SETTLE_S)
    t_qkv = TIMES[id(perm_qkv)]
    # context for the HBM roofline: a plain device copy (torch) of 64 MiB with the same rotation
    flat = [x.view(-1)[: B * L * (H // P) * D] for x in stacks]
    cidx = [0]

    def copy():
        outs[cidx[0] % 4][cidx[0] % 3].view(-1).copy_(flat[cidx[0] % 3])
        cidx[0] += 1

    _, ev_copy, _ = time_calls(copy, nperm, 3, SETTLE_S)
    # the local step itself: permute Q, K, V for rank 0 (one launch), causal attention, inverse of O
    q, k, v = ra.seq2head_permute_n(stacks, w.rank)
    full = ra.Shard("contiguous", 1, 0, L)
    o = torch.empty_like(q)
    lse = torch.empty((B, H // P, L), dtype=torch.float32, device="cuda")

    def attn():
        ra.block_attn_fwd(q, k, v, causal=True, q_shard=full, kv_shard=full, o=o, lse=lse)

    pairs = ra.share_work(full, full, L, L, True)[0]
    flops = 4 * D * B * (H // P) * pairs
    wall_a, ev_a, _ = time_calls(attn, steps, warmup, SETTLE_S)
    t_attn = TIMES[id(attn)]
    # inverse permute with rotated sources (12 distinct 64 MiB head-sharded tensors) and targets
    # (the head slice of dst in one of the three stacks)
    srcs = [t for grp in outs for t in grp]
    iidx = [0]

    def inv():
        i = iidx[0]
        ra.head2seq_permute(srcs[i % len(srcs)], (i // 3) % P, stacks[i % 3])
        iidx[0] += 1

    time_calls(inv, nperm, 3, SETTLE_S)
    t_inv = TIMES[id(inv)]
    del stacks, outs, q, k, v, o, lse, srcs
    torch.cuda.empty_cache()
    gbs = lambda ms, nbytes: nbytes / (ms * 1e-3) / 1e9  # noqa: E731
    return {"attention_tflops": flops / (t_attn["mean"] * 1e-3) / 1e12, "attention_ms": t_attn["mean"],
            "attention_ms_min": t_attn["min"], "attention_ms_median": t_attn["median"],
            "permute_gbs": gbs(t_one["mean"], moved), "permute_pct_hbm": 100 * gbs(t_one["mean"], moved) / PEAK_HBM_GBS,
            "permute_qkv_gbs": gbs(t_qkv["mean"], 3 * moved),
            "permute_qkv_pct_hbm": 100 * gbs(t_qkv["mean"], 3 * moved) / PEAK_HBM_GBS,
            "permute_qkv_ms": t_qkv["mean"], "permute_qkv_ms_min": t_qkv["min"],
            "device_copy_gbs": gbs(ev_copy, moved),
            "inverse_permute_gbs": gbs(t_inv["mean"], moved), "inverse_permute_ms": t_inv["mean"],
            "step_ms": t_qkv["mean"] + t_attn["mean"] + t_inv["mean"]}


def bench_usp(steps, warmup):
    """One device of the USP mesh (Ulysses degree u inside a group, zigzag ring of r groups):
    its step is the permute of its Ulysses group's Q, K and V for its head group, the ring over
    the r groups' K/V of that head group (the other groups' permuted K/V are prepared untimed:
    on a real mesh they arrive over the ring), and the inverse permute of O."""
    import torch

    import ring_sequence_parallelism_ra_amd as ra
    import synth
    w = synth.get("usp_u4r2")
    gq, gk, gv = synth.global_qkv(w)
    u, p, r, k, L, H, D, B = w.ulysses, w.ulysses_rank, w.world, w.rank, w.global_len, w.heads, w.head_dim, w.batch
    n = u * r
    pos = [ra.debug_positions(ra.Shard("zigzag", r, s, L)) for s in range(r)]

    def stacks(g):
        t = to_dev(g)
        out = [torch.index_select(t, 1, ps).view(B, u, L // n, H, D).transpose(0, 1).contiguous() for ps in pos]
        del t
        return out

    qs, ks, vs = stacks(gq), stacks(gk), stacks(gv)
    del gq, gk, gv
    kh = [ra.seq2head_permute(x, p) for x in ks]
    vh = [ra.seq2head_permute(x, p) for x in vs]
    qh = torch.empty_like(kh[0])
    call, o, lse = ra.prepare_ring_share(qh, kh, vh, k, assign="zigzag", causal=True)
    o_seq = torch.zeros_like(qs[k])

    def step():
        ra.seq2head_permute(qs[k], p, out=qh)
        ra.seq2head_permute(ks[k], p, out=kh[k])
        ra.seq2head_permute(vs[k], p, out=vh[k])
        call()
        ra.head2seq_permute(o, p, o_seq)

    q_sh = ra.Shard("zigzag", r, k, L)
    pairs = sum(ra.share_work(q_sh, ra.Shard("zigzag", r, s, L), L // r, L // r, True)[0] for s in range(r))
    flops = 4 * D * B * (H // u) * pairs
    _, ev_ring, _ = time_calls(call, steps, warmup, SETTLE_S)
    _, ev_step, _ = time_calls(step, steps, warmup, SETTLE_S)
    del qs, ks, vs, kh, vh, qh, o, lse, o_seq
    torch.cuda.empty_cache()
    return {"attention_tflops": flops / (ev_ring * 1e-3) / 1e12, "attention_ms": ev_ring,
            "step_ms": ev_step, "step_tflops": flops / (ev_step * 1e-3) / 1e12}


def bench_backward(steps, warmup):
    """ra_ring_share_bwd on the headline share (dO drawn like the inputs). Algorithmic work:
    5 matrix products per visible pair (S, dP, dV, dQ, dK) = 10*D FLOP; the kernels recompute S
    and dP once more (14*D executed)."""
    import torch

    import ring_sequence_parallelism_ra_amd as ra
    import synth
    w = synth.get(HEADLINE)
    inp, _ = ring_inputs(w)
    do = to_dev(synth.gaussian_bf16_bits(1000 * w.number + 3, tuple(inp["q"].shape)))
    o, lse = ra.ring_share(inp["q"], inp["k"], inp["v"], w.rank, assign=w.assign)

    def step():
        ra.ring_share_bwd(inp["q"], inp["k"], inp["v"], o, lse, do, w.rank, assign=w.assign)

    pairs = ring_pairs(w)
    flops = 10 * w.head_dim * w.batch * w.heads * pairs
    _, ev, _ = time_calls(step, max(2, steps // 3), 1, 0.0)
    del inp, do, o, lse
    torch.cuda.empty_cache()
    return {"tflops": flops / (ev * 1e-3) / 1e12, "ms": ev,
            "pct_bf16_peak_executed": 100 * 1.4 * flops / (ev * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def bench_balance(steps, warmup):
    """The pages' Striped Attention comparison, projected from one GPU.

    A ring of N devices finishes when its slowest rank does, so the time of the heaviest rank's
    whole share (one ra_ring_share call over all N steps) bounds the ring's attention time. For
    each token assignment (contiguous, striped, zigzag) this times the heaviest rank's share --
    the rank with the most visible pairs by the library's planner -- at the pages' two sizes
    (256K tokens on 8 devices, 786K on 16), B=1, H=16, D=128, causal, bf16 N(0,1) inputs drawn on
    the device. The contiguous/striped ratio is the compute-only counterpart of the pages'
    end-to-end 1.45x (256K, A100/TPUv4) and 1.65x (786K, 16x TPUv4); communication is not
    modelled."""
    import torch

    import ring_sequence_parallelism_ra_amd as ra
    H, D = 16, 128
    out = {}
    for L, n in ((262144, 8), (786432, 16)):
        g = torch.Generator(device="cuda").manual_seed(L + n)
        glob = [torch.randn((1, L, H, D), device="cuda", generator=g).to(torch.bfloat16) for _ in range(3)]
        s_loc = L // n
        res = {}
        for assign in ("contiguous", "striped", "zigzag"):
            sh = [ra.Shard(assign, n, r, L) for r in range(n)]
            pairs = [sum(ra.share_work(sh[r], sh[src], s_loc, s_loc, True)[0] for src in range(n)) for r in range(n)]
            rank = max(range(n), key=lambda r: pairs[r])
            pos = [ra.debug_positions(x) for x in sh]
            q = torch.index_select(glob[0], 1, pos[rank]).contiguous()
            ks = [torch.index_select(glob[1], 1, p).contiguous() for p in pos]
            vs = [torch.index_select(glob[2], 1, p).contiguous() for p in pos]
            call, o, lse = ra.prepare_ring_share(q, ks, vs, rank, assign=assign, causal=True)
            _, ev, _ = time_calls(call, steps, warmup)
            flops = 4 * D * H * pairs[rank]
            res[assign] = {"rank": rank, "ms": round(ev, 3), "tflops": round(flops / (ev * 1e-3) / 1e12, 1),
                           "pairs_per_head": pairs[rank], "lightest_rank_pairs_per_head": min(pairs)}
            del q, ks, vs, o, lse, call
            torch.cuda.empty_cache()
        c = res["contiguous"]
        res["striped_speedup"] = round(c["ms"] / res["striped"]["ms"], 3)
        res["zigzag_speedup"] = round(c["ms"] / res["zigzag"]["ms"], 3)
        res["striped_pair_ratio"] = round(c["pairs_per_head"] / res["striped"]["pairs_per_head"], 3)
        out[f"L{L}_N{n}"] = res
        del glob
        torch.cuda.empty_cache()
    out["pages_context"] = ("Striped over contiguous Ring Attention, end to end: 1.45x at 256K tokens "
                            "(A100 / TPUv4), 1.65x at 786K tokens (16x TPUv4); other hardware, with "
                            "communication; context only")
    return out


def bench_tiny(steps, warmup):
    """The tiny exact fp32 workload (B1 H1 L256 D64, 4 contiguous ranks, non-causal): one
    ra_ring_share per rank, each 4 ring steps of 64 keys. Reported for completeness, not held to
    the matrix-core roofline: the fp32 path gives every query row one lane and computes logits,
    maximum and sum in fp64 on the vector ALUs; a 64-query share is one workgroup whose four
    waves fold a quarter of the keys each, so its time is the latency of 64 keys' fp64 work per
    lane plus the merge (about a hundred microseconds)."""
    import torch

    import ring_sequence_parallelism_ra_amd as ra
    import synth
    w = synth.get("tiny_exact")
    gq, gk, gv = (torch.from_numpy(x).cuda() for x in synth.global_qkv(w))
    n, L = w.world, w.global_len
    pos = [ra.debug_positions(ra.Shard(w.assign, n, r, L)) for r in range(n)]
    ks = [torch.index_select(gk, 1, p).contiguous() for p in pos]
    vs = [torch.index_select(gv, 1, p).contiguous() for p in pos]
    calls = [ra.prepare_ring_share(torch.index_select(gq, 1, pos[r]).contiguous(), ks, vs, r, assign=w.assign,
                                   causal=False)[0] for r in range(n)]

    def all_ranks():
        for c in calls:
            c()

    _, ev, _ = time_calls(all_ranks, steps, warmup, SETTLE_S)
    flops = 4 * w.head_dim * w.heads * w.batch * L * L  # every rank's 64 queries against all 256 keys
    return {"us_per_rank_call": 1e3 * ev / n, "tflops": flops / (ev * 1e-3) / 1e12, "dtype": "f32"}


def bench_merge(steps, warmup):
    import torch

    import ring_sequence_parallelism_ra_amd as ra
    B, S, H, D = 1, 32768, 16, 128  # one share of the long zigzag workload, fp32 state
    sets = []
    for i in range(3):
        g = torch.Generator(device="cuda").manual_seed(i)
        sets.append((torch.randn((B, S, H, D), device="cuda", generator=g),
                     torch.randn((B, H, S), device="cuda", generator=g),
                     torch.randn((B, S, H, D), device="cuda", generator=g),
                     torch.randn((B, H, S), device="cuda", generator=g)))
    idx = [0]

    def merge():
        a = sets[idx[0] % 3]
        ra.lse_merge(*a)
        idx[0] += 1

    _, ev, _ = time_calls(merge, max(steps, 12), warmup, SETTLE_S)
    moved = B * S * H * (3 * 4 * D + 3 * 4)
    del sets
    torch.cuda.empty_cache()
    return {"gbs": moved / (ev * 1e-3) / 1e9, "pct_hbm": 100 * moved / (ev * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "ms": ev, "shape": [B, S, H, D]}


def cpu_baseline(host, w, budget_s):
    """The fp64 oracle timed on this host: batches of sampled query rows (all heads) of the
    headline share, each against every key up to its position, until ``budget_s`` is used."""
    import numpy as np

    import synth
    from oracle import attention as OA
    from oracle import positions as OP
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max(i["num_threads"] for i in blas) if blas else 1
    except Exception:
        cores = os.cpu_count() or 1
    gq, gk, gv = host
    n, r, L = w.world, w.rank, w.global_len
    pos = OP.positions(w.assign, n, r, L)
    rows = synth.sample_rows(1000 * w.number, w.share_len, chunk_len=L // (2 * n))
    rows = np.random.default_rng(0).permutation(rows)
    batch = 16
    done_rows, pairs, t0 = 0, 0, time.perf_counter()
    for i in range(0, len(rows), batch):
        rb = np.sort(rows[i:i + batch])
        qpos = pos[rb]
        kmax = int(qpos.max()) + 1
        q = synth.bf16_bits_to_f32(np.ascontiguousarray(gq[:, qpos]))
        k = synth.bf16_bits_to_f32(gk[:, :kmax])
        v = synth.bf16_bits_to_f32(gv[:, :kmax])
        OA.attention(q, k, v, qpos, np.arange(kmax), True)
        done_rows += len(rb)
        pairs += int((qpos + 1).sum()) * w.heads * w.batch
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 4 * w.head_dim * pairs
    full_pairs = ring_pairs(w) * w.heads * w.batch
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done_rows} sampled query rows x {w.heads} heads of {w.name} ({pairs} visible pairs, "
                      f"fp64 numpy, {dt:.1f}s incl. bf16->fp64 conversion)",
            "cpu_count": os.cpu_count(), "blas_threads": int(cores),
            "per_row_head_ms": 1e3 * dt / (done_rows * w.heads * w.batch),
            "full_share_s_extrapolated": dt * full_pairs / pairs}


def oracle_configs():
    """Wall time of the oracle, as it stands, on the other workloads: every row of the tiny exact
    ring (all four ranks), of the contiguous rank-7 share and of the striped rank-0 share (one
    OA.attention call each, the share against the whole sequence); for the Ulysses attention,
    32 sampled rows x its 4 heads, reported per row-head and extrapolated (by visible pairs) to
    the full attention. The headline share's figures are in the cpu_baseline entry."""
    import numpy as np

    import synth
    from oracle import attention as OA
    from oracle import positions as OP
    out = {"full_s": {}, "per_row_head_ms": {}, "full_s_extrapolated": {}}
    for name in ("tiny_exact", "contig_rank7", "striped_rank0"):
        w = synth.get(name)
        gq, gk, gv = synth.global_qkv(w)
        conv = (lambda x: x) if w.dtype == "f32" else synth.bf16_bits_to_f32
        k, v = conv(gk), conv(gv)
        ranks = range(w.world) if w.rank < 0 else [w.rank]
        t0 = time.perf_counter()
        for r in ranks:
            qpos = OP.positions(w.assign, w.world, r, w.global_len)
            OA.attention(conv(np.ascontiguousarray(gq[:, qpos])), k, v, qpos, np.arange(w.global_len), w.causal)
        out["full_s"][name] = round(time.perf_counter() - t0, 3)
        log(f"[bench] oracle {name}: {out['full_s'][name]:.1f}s for the whole share")
    w = synth.get("ulysses_local")
    gq, gk, gv = synth.global_qkv(w)
    P, L, H, D = w.world, w.global_len, w.heads, w.head_dim
    heads = slice(w.rank * H // P, (w.rank + 1) * H // P)   # the destination rank's head slice
    rows = np.sort(np.random.default_rng(1).choice(L, 32, replace=False))
    kmax = int(rows.max()) + 1
    t0 = time.perf_counter()
    OA.attention(synth.bf16_bits_to_f32(np.ascontiguousarray(gq[:, rows, heads])),
                 synth.bf16_bits_to_f32(np.ascontiguousarray(gk[:, :kmax, heads])),
                 synth.bf16_bits_to_f32(np.ascontiguousarray(gv[:, :kmax, heads])), rows, np.arange(kmax), True)
    dt = time.perf_counter() - t0
    pairs = int((rows + 1).sum()) * (H // P)
    out["per_row_head_ms"]["ulysses_local"] = round(1e3 * dt / (len(rows) * (H // P)), 3)
    out["full_s_extrapolated"]["ulysses_local"] = round(dt * (L * (L + 1) // 2) * (H // P) / pairs, 1)
    return out


def traffic_for(kernel_ms_launch):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, if they were taken on the
    current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256_16") != kernel_hash():
        return None
    return t.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary", default="", help="comma-separated subset of the secondary workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-oracle-configs", action="store_true",
                    help="skip the oracle wall times of the other workloads (about a minute of host time)")
    args = ap.parse_args()
    every = ("contig_rank7", "striped_rank0", "striped_rank0_std4", "gqa_zigzag_rank3", "ulysses_local", "usp_u4r2",
             "backward_zigzag_rank3", "lse_merge", "striped_vs_contiguous", "tiny_exact")
    chosen = () if args.no_secondary else (tuple(args.secondary.split(",")) if args.secondary else every)
    unknown = [c for c in chosen if c not in every]
    if unknown:
        ap.error(f"unknown secondary workload(s) {unknown}; choose from {list(every)}")
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share only: this build runs on a single MI355X and has no "
              "multi-GPU path (each rank would run the same ra_ring_share on its own share). "
              "Run with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import ring_sequence_parallelism_ra_amd as ra  # noqa: F401  (fails loudly if libra.so is missing)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    head, host, w = bench_ring(HEADLINE, args.steps, args.warmup, tiles=True)
    log(f"[bench] {HEADLINE}: {head['tflops']:.1f} TFLOP/s, kernel {head['kernel_ms_mean']:.3f} ms")
    achieved = head["flops"] / (head["kernel_ms_mean"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic_for(head["kernel_ms_mean"]),
                "kernel": "attn_bf16_kernel<128, OutBf16, 1, 0, 0>", "kernel_ms": round(head["kernel_ms_mean"], 4),
                "kernel_ms_min": round(head["kernel_ms_min"], 4), "kernel_ms_median": round(head["kernel_ms_median"], 4),
                "flops_per_launch": head["flops"], "tile_walk": head["tile_walk"]}

    secondary = {}
    if chosen:
        for name in [n for n in every[:4] if n in chosen]:
            r, _, _ = bench_ring(name, args.steps, args.warmup, SETTLE_S)
            secondary[name] = {"tflops": round(r["tflops"], 2), "pct_bf16_peak": round(100 * r["tflops"] / PEAK_BF16_TFLOPS, 2),
                               "kernel_ms": round(r["kernel_ms_mean"], 4), "kernel_ms_min": round(r["kernel_ms_min"], 4),
                               "kernel_ms_median": round(r["kernel_ms_median"], 4)}
            log(f"[bench] {name}: {r['tflops']:.1f} TFLOP/s")
        if "ulysses_local" in chosen:
            u = bench_ulysses(args.steps, args.warmup)
            secondary["ulysses_local"] = {k: round(v, 3) for k, v in u.items()}
            log(f"[bench] ulysses_local: attention {u['attention_tflops']:.1f} TFLOP/s, permute {u['permute_gbs']:.0f} GB/s "
                f"(plain device copy of the same bytes: {u['device_copy_gbs']:.0f} GB/s)")
        if "usp_u4r2" in chosen:
            us = bench_usp(args.steps, args.warmup)
            secondary["usp_u4r2"] = {k: round(v, 3) for k, v in us.items()}
            log(f"[bench] usp_u4r2: attention {us['attention_tflops']:.1f} TFLOP/s, device step {us['step_ms']:.3f} ms "
                f"({us['step_tflops']:.1f} TFLOP/s incl. permutes)")
        if "backward_zigzag_rank3" in chosen:
            bw = bench_backward(args.steps, args.warmup)
            secondary["backward_zigzag_rank3"] = {k: round(v, 3) for k, v in bw.items()}
            log(f"[bench] backward {HEADLINE}: {bw['tflops']:.1f} TFLOP/s (10*D FLOP per pair), {bw['ms']:.1f} ms")
        if "striped_vs_contiguous" in chosen:
            sb = bench_balance(min(args.steps, 3), 1)
            secondary["striped_vs_contiguous"] = sb
            for k, v in sb.items():
                if isinstance(v, dict):
                    log(f"[bench] striped_vs_contiguous {k}: heaviest-rank share contiguous {v['contiguous']['ms']:.1f} ms, "
                        f"striped {v['striped']['ms']:.1f} ms, zigzag {v['zigzag']['ms']:.1f} ms -> striped "
                        f"{v['striped_speedup']}x, zigzag {v['zigzag_speedup']}x over contiguous")
        if "tiny_exact" in chosen:
            t = bench_tiny(args.steps, args.warmup)
            secondary["tiny_exact"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in t.items()}
            log(f"[bench] tiny_exact: {t['us_per_rank_call']:.1f} us per rank's ring call (fp32, latency-bound)")
        if "lse_merge" in chosen:
            m = bench_merge(args.steps, args.warmup)
            secondary["lse_merge"] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in m.items()}
            log(f"[bench] lse_merge: {m['gbs']:.0f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(host, w, args.cpu_seconds)
        log(f"[bench] cpu_baseline: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads")
        if not args.no_oracle_configs:
            cpu["oracle_configs"] = oracle_configs()

    line = {"metric": METRIC, "value": round(head["tflops"], 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["ms_per_step"], 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": HEADLINE, "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim,
                       "global_len": w.global_len, "world": w.world, "rank": w.rank, "assign": w.assign,
                       "share_len": w.share_len, "causal": True,
                       "pct_bf16_peak": round(100 * head["tflops"] / PEAK_BF16_TFLOPS, 2)},
            "roofline": roofline, "cpu_baseline": cpu, "secondary": secondary}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
