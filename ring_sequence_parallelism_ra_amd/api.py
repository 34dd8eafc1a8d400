"""torch-facing wrappers of the C ABI (same names as ``include/ra.h`` without the ``ra_`` prefix).

PyTorch supplies device memory and streams only; the wrappers check tensor shapes/dtypes,
allocate outputs when none are given, and pass raw pointers to the HIP library.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import ASSIGN, BF16, F32, Shard, check, lib

_DT = {torch.float32: F32, torch.bfloat16: BF16}
_TORCH_DT = {F32: torch.float32, BF16: torch.bfloat16}


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16") from None


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else None


def _need(t, name):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


def _expect(t, name, shape, dtype):
    """Shape and dtype of a caller-supplied tensor, checked before anything is launched: the
    library reads and writes exactly these extents in these element sizes."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    dts = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dts:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dts)}, got {t.dtype}")


def _shard(sh):
    if sh is None:
        return None
    if not isinstance(sh, Shard):
        sh = Shard(*sh)
    return ctypes.byref(sh)


def block_attn_fwd(q, k, v, *, causal=False, q_shard=None, kv_shard=None, scale=0.0, out_dtype=None,
                   o=None, lse=None, stream=None):
    """O, LSE of q [B,Sq,H,D] against one KV block k, v [B,Sk,H_kv,D] (H_kv dividing H: grouped-
    query attention); see ra_block_attn_fwd."""
    b, sq, h, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    _expect(q, "q", q.shape, tuple(_DT))
    _expect(k, "k", (b, sk, hkv, d), q.dtype)
    _expect(v, "v", k.shape, q.dtype)
    od = out_dtype or (o.dtype if o is not None else q.dtype)
    if o is not None:
        _expect(o, "o", (b, sq, h, d), od)
    if lse is not None:
        _expect(lse, "lse", (b, h, sq), torch.float32)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (lse, "lse")):
        if t is not None:
            _need(t, n)
    if o is None:
        o = torch.empty((b, sq, h, d), dtype=od, device=q.device)
    if lse is None:
        lse = torch.empty((b, h, sq), dtype=torch.float32, device=q.device)
    check(lib.ra_block_attn_fwd(_p(q), _p(k), _p(v), _p(o), _p(lse), b, h, hkv, sq, sk, d, _dt(q), _dt(o),
                                1 if causal else 0, _shard(q_shard), _shard(kv_shard), float(scale),
                                _stream(stream)))
    return o, lse


def ring_share_workspace_bytes(B, H, S_loc, D) -> int:
    return int(lib.ra_ring_share_workspace_bytes(B, H, S_loc, D))


def ring_share_workspace(B, H, S_loc, D, device="cuda"):
    return torch.empty(ring_share_workspace_bytes(B, H, S_loc, D), dtype=torch.uint8, device=device)


def prepare_ring_share(q, k_shares, v_shares, rank, *, assign="contiguous", causal=True, scale=0.0,
                       out_dtype=None, start_step=0, num_steps=None, ws=None, o=None, lse=None,
                       stream=None):
    """Marshal the arguments of ra_ring_share once; returns (call, o, lse) where ``call()``
    enqueues the whole ring loop on the stream (for repeated launches)."""
    b, s, h, d = q.shape
    _expect(q, "q", q.shape, tuple(_DT))
    n = len(k_shares)
    if len(v_shares) != n:
        raise ValueError("k_shares and v_shares differ in length")
    hkv = k_shares[0].shape[2] if n else h
    for t in list(k_shares) + list(v_shares):
        _expect(t, "every K/V share", (b, s, hkv, d), q.dtype)
    num = n - start_step if num_steps is None else num_steps
    od = out_dtype or (o.dtype if o is not None else q.dtype)
    if o is not None:
        _expect(o, "o", (b, s, h, d), od)
    if lse is not None:
        _expect(lse, "lse", (b, h, s), torch.float32)
    for t in [q, o, lse, ws] + list(k_shares) + list(v_shares):
        if t is not None:
            _need(t, "q/o/lse/ws/share")
    if o is None:
        o = torch.empty((b, s, h, d), dtype=od, device=q.device)
    if lse is None:
        lse = torch.empty((b, h, s), dtype=torch.float32, device=q.device)
    kp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in k_shares])
    vp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in v_shares])
    ws_p, ws_n = (_p(ws), ws.numel() * ws.element_size()) if ws is not None else (None, 0)
    args = (_p(q), kp, vp, _p(o), _p(lse), b, h, hkv, s, d, n, rank, ASSIGN.get(assign, assign),
            1 if causal else 0, _dt(q), _dt(o), float(scale), start_step, num, ws_p, ws_n,
            _stream(stream))
    keep = (k_shares, v_shares, ws)

    def call():
        _ = keep
        check(lib.ra_ring_share(*args))

    return call, o, lse


def ring_share(q, k_shares, v_shares, rank, **kw):
    """Every ring step of ``rank``'s share; see ra_ring_share. Returns (O, LSE)."""
    call, o, lse = prepare_ring_share(q, k_shares, v_shares, rank, **kw)
    call()
    return o, lse


def ring_share_bwd(q, k_shares, v_shares, o, lse, dout, rank, *, assign="contiguous", causal=True,
                   scale=0.0, stream=None):
    """Gradients of ``ring_share``'s output: returns (dq [B,S,H,D], dk list, dv list), fp32, where
    dk[i] / dv[i] [B,S,H_kv,D] are the gradients with respect to rank i's K/V share from this
    rank's queries; see ra_ring_share_bwd."""
    b, s, h, d = q.shape
    n = len(k_shares)
    if len(v_shares) != n or n == 0:
        raise ValueError("k_shares and v_shares must be non-empty and of equal length")
    hkv = k_shares[0].shape[2]
    # the library reads q, o, dout and the shares as bf16 and lse as fp32: a forward output
    # kept in fp32 must be rounded to bf16 by the caller first
    _expect(q, "q", (b, s, h, d), torch.bfloat16)
    _expect(o, "o", (b, s, h, d), torch.bfloat16)
    _expect(dout, "dout", (b, s, h, d), torch.bfloat16)
    _expect(lse, "lse", (b, h, s), torch.float32)
    for t in list(k_shares) + list(v_shares):
        _expect(t, "every K/V share", (b, s, hkv, d), torch.bfloat16)
    for t in [q, o, lse, dout] + list(k_shares) + list(v_shares):
        _need(t, "q/o/lse/dout/share")
    dq = torch.empty((b, s, h, d), dtype=torch.float32, device=q.device)
    dk = [torch.empty((b, s, hkv, d), dtype=torch.float32, device=q.device) for _ in range(n)]
    dv = [torch.empty((b, s, hkv, d), dtype=torch.float32, device=q.device) for _ in range(n)]
    ws_n = int(lib.ra_ring_share_bwd_workspace_bytes(b, h, s))
    ws = torch.empty((max(ws_n, 16) + 3) // 4, dtype=torch.float32, device=q.device)
    kp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in k_shares])
    vp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in v_shares])
    dkp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in dk])
    dvp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in dv])
    check(lib.ra_ring_share_bwd(_p(q), kp, vp, _p(o), _p(lse), _p(dout), _p(dq), dkp, dvp, b, h, hkv, s, d, n,
                                rank, ASSIGN.get(assign, assign), 1 if causal else 0, _dt(q), float(scale),
                                _p(ws), ws.numel() * 4, _stream(stream)))
    return dq, dk, dv


def usp_local_step(q_stack, k_heads, v_heads, ulysses_rank, ring_rank, *, out=None, scale=0.0,
                   out_dtype=None, stream=None):
    """One device's USP attention ([Digest] §7.2: Ulysses all-to-all inside the Ulysses group,
    zigzag ring attention across the ring groups, reverse all-to-all), with the collectives'
    data already local. Three library calls, nothing computed here:

      1. ra_seq2head_permute of q_stack [u, B, L/N, H, D] (the Q slices of the Ulysses group of
         ring rank ``ring_rank``, in Ulysses-rank order) for head group ``ulysses_rank``:
         Q [B, L/r, H/u, D], i.e. the ring share of ``ring_rank`` for heads
         [ulysses_rank*H/u, (ulysses_rank+1)*H/u);
      2. ra_ring_share over the r ring shares (zigzag, causal, global length L = r * L/r):
         k_heads / v_heads are the r tensors [B, L/r, H/u, D] of the same head group, entry k
         from ring rank k (each is that ring group's own step-1 permute; on several GPUs the
         ring passes them along);
      3. the inverse permute of O into ``out`` [u, B, L/N, H, D], writing only this head group.

    Returns (out, O [B, L/r, H/u, D], LSE [B, H/u, L/r]).
    """
    u, b, s, h, d = q_stack.shape
    od = out_dtype or q_stack.dtype
    if out is not None:
        _expect(out, "out", (u, b, s, h, d), od)
    _need(q_stack, "q_stack")
    qh = seq2head_permute(q_stack, ulysses_rank, stream=stream)
    o, lse = ring_share(qh, k_heads, v_heads, ring_rank, assign="zigzag", causal=True, scale=scale,
                        out_dtype=out_dtype, stream=stream)
    if out is None:
        out = torch.zeros((u, b, s, h, d), dtype=od, device=q_stack.device)
    head2seq_permute(o, ulysses_rank, out, stream=stream)
    return out, o, lse


def lse_merge(o_acc, lse_acc, o_blk, lse_blk, stream=None):
    """In-place merge of (o_blk, lse_blk) into (o_acc, lse_acc); see ra_lse_merge."""
    b, s, h, d = o_acc.shape
    _expect(o_acc, "o_acc", o_acc.shape, tuple(_DT))
    _expect(o_blk, "o_blk", o_acc.shape, tuple(_DT))
    _expect(lse_acc, "lse_acc", (b, h, s), torch.float32)
    _expect(lse_blk, "lse_blk", (b, h, s), torch.float32)
    for t, nme in ((o_acc, "o_acc"), (lse_acc, "lse_acc"), (o_blk, "o_blk"), (lse_blk, "lse_blk")):
        _need(t, nme)
    check(lib.ra_lse_merge(_p(o_acc), _p(lse_acc), _p(o_blk), _p(lse_blk), b, h, s, d, _dt(o_acc),
                           _dt(o_blk), _stream(stream)))
    return o_acc, lse_acc


def seq2head_permute(x, dst_rank, out=None, stream=None):
    """x [P, B, S_loc, H, D] -> [B, P*S_loc, H/P, D] for dst_rank (or the stack of all ranks
    [P, B, P*S_loc, H/P, D] for dst_rank=-1); see ra_seq2head_permute."""
    p, b, s, h, d = x.shape
    _expect(x, "x", x.shape, tuple(_DT))
    if h % p:
        raise ValueError(f"P={p} does not divide H={h}")
    shape = (b, p * s, h // p, d) if dst_rank >= 0 else (p, b, p * s, h // p, d)
    if out is not None:
        _expect(out, "out", shape, x.dtype)
        _need(out, "out")
    _need(x, "x")
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    check(lib.ra_seq2head_permute(_p(x), _p(out), b, p, s, h, d, _dt(x), dst_rank, 0, _stream(stream)))
    return out


def seq2head_permute_n(xs, dst_rank, outs=None, inverse=False, stream=None):
    """ra_seq2head_permute_n: the permute (or, with ``inverse``, its inverse) of several tensors of
    one shape and dtype in one launch. Forward: xs are [P, B, S_loc, H, D] stacks, outs (allocated
    when None) their head-sharded results. Inverse: xs are head-sharded tensors, outs the
    [P, B, S_loc, H, D] stacks to write (only dst_rank's heads are written)."""
    xs = list(xs)
    if not xs:
        return []
    if outs is None:
        if inverse:
            raise ValueError("the inverse writes into caller-supplied outs")
        p, b, s, h, d = xs[0].shape
        shape = (b, p * s, h // p, d) if dst_rank >= 0 else (p, b, p * s, h // p, d)
        outs = [torch.empty(shape, dtype=xs[0].dtype, device=xs[0].device) for _ in xs]
    outs = list(outs)
    if len(outs) != len(xs):
        raise ValueError("xs and outs differ in length")
    seq = outs if inverse else xs
    p, b, s, h, d = seq[0].shape
    _expect(seq[0], "stack", seq[0].shape, tuple(_DT))
    if h % p:
        raise ValueError(f"P={p} does not divide H={h}")
    head_shape = (b, p * s, h // p, d) if dst_rank >= 0 else (p, b, p * s, h // p, d)
    for i, (x, y) in enumerate(zip(xs, outs)):
        src_shape, dst_shape = ((head_shape, (p, b, s, h, d)) if inverse else ((p, b, s, h, d), head_shape))
        _expect(x, f"xs[{i}]", src_shape, seq[0].dtype)
        _expect(y, f"outs[{i}]", dst_shape, seq[0].dtype)
        _need(x, f"xs[{i}]")
        _need(y, f"outs[{i}]")
    n = len(xs)
    ip = (ctypes.c_void_p * n)(*[t.data_ptr() for t in xs])
    op = (ctypes.c_void_p * n)(*[t.data_ptr() for t in outs])
    check(lib.ra_seq2head_permute_n(ip, op, n, b, p, s, h, d, _dt(seq[0]), dst_rank, 1 if inverse else 0,
                                    _stream(stream)))
    return outs


def head2seq_permute(y, dst_rank, out, stream=None):
    """Inverse: write y (dst_rank's head-sharded tensor, or the stack) back into
    out [P, B, S_loc, H, D], touching only dst_rank's heads (all for -1)."""
    p, b, s, h, d = out.shape
    _expect(out, "out", out.shape, tuple(_DT))
    if h % p:
        raise ValueError(f"P={p} does not divide H={h}")
    _expect(y, "y", (b, p * s, h // p, d) if dst_rank >= 0 else (p, b, p * s, h // p, d), out.dtype)
    _need(y, "y")
    _need(out, "out")
    check(lib.ra_seq2head_permute(_p(y), _p(out), b, p, s, h, d, _dt(out), dst_rank, 1, _stream(stream)))
    return out


def share_work(q_shard, kv_shard, Sq, Sk, causal=True, block_m=128, block_n=64):
    """(visible pairs, full tiles, partial tiles, skip tiles); host only, no GPU."""
    out = (ctypes.c_int64 * 4)()
    check(lib.ra_share_work(_shard(q_shard), _shard(kv_shard), Sq, Sk, 1 if causal else 0, block_m,
                            block_n, out))
    return tuple(out)


def tile_shape(in_dtype=BF16, D=128):
    bm, bn = ctypes.c_int64(), ctypes.c_int64()
    check(lib.ra_tile_shape(in_dtype, D, ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value


def debug_positions(shard, device="cuda", stream=None):
    sh = shard if isinstance(shard, Shard) else Shard(*shard)
    out = torch.empty(sh.global_len // sh.world, dtype=torch.int64, device=device)
    check(lib.ra_debug_positions(ctypes.byref(sh), _p(out), _stream(stream)))
    return out


def debug_mask(q_shard, kv_shard, Sq, Sk, device="cuda", stream=None):
    out = torch.empty((Sq, Sk), dtype=torch.uint8, device=device)
    check(lib.ra_debug_mask(_shard(q_shard), _shard(kv_shard), Sq, Sk, _p(out), _stream(stream)))
    return out


def debug_tile_counts(q, k_shares, v_shares, rank, *, assign="contiguous", causal=True, scale=0.0,
                      out_dtype=None, stream=None):
    """ring_share through the tile-counting copy of the bf16 kernel; returns (O, LSE, counts) with
    counts int32 [ceil(S_loc/128), B, H, 8, 4] (per wave slot: tiles folded in, tiles masked,
    bounds faults, skip faults); see ra_debug_tile_counts."""
    b, s, h, d = q.shape
    _expect(q, "q", q.shape, torch.bfloat16)
    n = len(k_shares)
    if len(v_shares) != n or n == 0:
        raise ValueError("k_shares and v_shares must be non-empty and of equal length")
    hkv = k_shares[0].shape[2]
    for t in list(k_shares) + list(v_shares):
        _expect(t, "every K/V share", (b, s, hkv, d), torch.bfloat16)
    for t in [q] + list(k_shares) + list(v_shares):
        _need(t, "q/share")
    od = out_dtype or q.dtype
    o = torch.empty((b, s, h, d), dtype=od, device=q.device)
    lse = torch.empty((b, h, s), dtype=torch.float32, device=q.device)
    slots = int(lib.ra_debug_tile_count_slots(b, h, s))
    counts = torch.empty(max(slots, 4), dtype=torch.int32, device=q.device)
    kp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in k_shares])
    vp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in v_shares])
    check(lib.ra_debug_tile_counts(_p(q), kp, vp, _p(o), _p(lse), b, h, hkv, s, d, n, rank, ASSIGN.get(assign, assign),
                                   1 if causal else 0, _dt(o), float(scale), _p(counts), counts.numel(),
                                   _stream(stream)))
    return o, lse, counts[:slots].view(-1, b, h, 8, 4)


def torch_dtype(code: int):
    return _TORCH_DT[code]
