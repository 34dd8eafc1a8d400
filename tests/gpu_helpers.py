"""Helpers for the GPU parity tests: moving seeded inputs to the device, gathering shares
by the oracle's positions, and the tolerance checks."""
from __future__ import annotations

import numpy as np
import torch

import synth
from oracle import attention as OA
from oracle import positions as OP

# Tolerances (max-abs): fp32 I/O O 1e-5, LSE 1e-6; bf16 I/O with fp32 accumulation O 1e-2,
# LSE 2e-3. A bf16 *output* adds half a bf16 ulp for the rounding of the stored result itself
# (which alone can exceed 1e-2 once |O| >= 4), taken in the binade the unrounded result can
# fall in: that of |O_ref| + (kernel tolerance), since a value just below a power of two may
# round up into the next binade.
TOL = {"f32": (1e-5, 1e-6), "bf16": (1e-2, 2e-3)}


def say(*a):
    print(*a, flush=True)


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def values(x: np.ndarray, dtype: str) -> np.ndarray:
    """The exact values an input array stands for (bf16 bits widen exactly)."""
    return synth.bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def gen(seed, shape, dtype, std=1.0):
    return synth.gaussian_bf16_bits(seed, shape, std) if dtype == "bf16" else synth.gaussian_f32(seed, shape, std)


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def half_ulp_bf16(ref: np.ndarray) -> np.ndarray:
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def check(o_gpu, lse_gpu, o_ref, lse_ref, in_dtype, o_dtype, what=""):
    """Max-abs check of O and LSE against the fp64 oracle; returns (err_o, err_lse)."""
    to, tl = TOL[in_dtype]
    o = host(o_gpu) if isinstance(o_gpu, torch.Tensor) else o_gpu
    lse = host(lse_gpu) if isinstance(lse_gpu, torch.Tensor) else lse_gpu
    bound = to + (half_ulp_bf16(np.abs(o_ref) + to) if o_dtype == "bf16" else 0.0)
    err = np.abs(o - o_ref)
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    bad = err > bound
    assert not bad.any(), f"{what}: O error {err.max():.3e} > bound at {np.argwhere(bad)[:3].tolist()}"
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: -inf LSE rows differ"
    el = np.abs(lse[~empty] - lse_ref[~empty]) if (~empty).any() else np.zeros(1)
    assert el.max() <= tl, f"{what}: LSE error {el.max():.3e} > {tl}"
    return float(err.max()), float(el.max())


def shares(x: np.ndarray, assign: str, n: int) -> list:
    """Gather each rank's share [B, S_loc, H, D] of a global [B, L, H, D] array."""
    L = x.shape[1]
    return [np.ascontiguousarray(x[:, OP.positions(assign, n, r, L)]) for r in range(n)]


def oracle_rows(q_share_vals, k_glob_vals, v_glob_vals, qpos_rows, rows, causal=True):
    """Oracle O [B, len(rows), H, D] and LSE [B, H, len(rows)] of selected local rows of a share
    against the whole global sequence (keys beyond the largest query position are invisible to
    every selected row and are left out)."""
    q = q_share_vals[:, rows]
    qpos = qpos_rows
    kmax = int(qpos.max()) + 1 if causal else k_glob_vals.shape[1]
    kpos = np.arange(kmax)
    return OA.attention(q, k_glob_vals[:, :kmax], v_glob_vals[:, :kmax], qpos, kpos, causal)


def oracle_share(q_share_vals, k_glob_vals, v_glob_vals, qpos, causal=True, rows_per_job=512, threads=None):
    """Oracle O [B, S, H, D] and LSE [B, H, S] of every row of a share against the global
    sequence. Jobs of ``rows_per_job`` rows of one (batch, head) run on a thread pool (the
    numpy work releases the GIL; BLAS is held to one thread per job); a job passes only the
    keys up to its largest query position, since the later ones are invisible to all its rows.
    Each row is still evaluated by the oracle's own definition, independently of the others."""
    import concurrent.futures as cf
    import os

    from threadpoolctl import threadpool_limits

    b_, s_, h_, d_ = q_share_vals.shape
    group = h_ // k_glob_vals.shape[2]
    o = np.zeros((b_, s_, h_, d_))
    lse = np.zeros((b_, h_, s_))
    jobs = [(b, h, r0) for b in range(b_) for h in range(h_) for r0 in range(0, s_, rows_per_job)]

    def run(job):
        b, h, r0 = job
        r1 = min(s_, r0 + rows_per_job)
        qp = qpos[r0:r1]
        kmax = int(qp.max()) + 1 if causal else k_glob_vals.shape[1]
        hk = h // group
        oo, ll = OA.attention(q_share_vals[b:b + 1, r0:r1, h:h + 1], k_glob_vals[b:b + 1, :kmax, hk:hk + 1],
                              v_glob_vals[b:b + 1, :kmax, hk:hk + 1], qp, np.arange(kmax), causal)
        o[b, r0:r1, h] = oo[0, :, 0]
        lse[b, h, r0:r1] = ll[0, 0]

    n = threads or min(16, os.cpu_count() or 1)
    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(n) as ex:
            list(ex.map(run, jobs))
    return o, lse


U_BF16 = 2.0 ** -8  # unit roundoff of bf16 (8 significant bits): |round(x) - x| <= u |x|


def delta_error(o_used, o_ref, do_vals):
    """Per-row bound [B, H, S] on the error of the backward's Delta_i = dO_i . O_i, which the
    kernels take from the stored forward output ``o_used`` (values, e.g. the oracle's O rounded
    to bf16) instead of the exact O: the difference it makes, plus fp32 rounding of the dot
    product."""
    diff = np.abs(np.einsum("bshd,bshd->bhs", do_vals, o_used - o_ref))
    mag = np.einsum("bshd,bshd->bhs", np.abs(do_vals), np.abs(o_ref))
    return diff + 1e-6 * mag


def check_grad_entries(got, want, mag, err_delta, what):
    """Entry-wise check of a gradient against the oracle: |got - want| <= 2 (u * mag + err_delta)
    + 1e-7, where mag is the entry's sum of absolute terms and err_delta what a bounded error in
    Delta moves it by (oracle.backward.attention_bwd_magnitudes). Returns the largest ratio of an
    error to its bound."""
    got = host(got) if isinstance(got, torch.Tensor) else got
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    bound = 2.0 * (U_BF16 * mag + err_delta) + 1e-7
    err = np.abs(got - want)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} entries beyond their bound, e.g. {np.argwhere(bad)[:3].tolist()} "
                           f"error {err[bad][:3].tolist()} bound {bound[bad][:3].tolist()}")
    return float((err / bound).max())


def per_head(fn, q, k, v, *rest, delta_err=None, threads=None, **kw):
    """Run an oracle function once per head on a thread pool (BLAS held to one thread per job)
    and stack the results along the head axis: [B, S, H, D] outputs on axis 2, [B, H, S] on
    axis 1. Heads are independent in the definition (multi-head: K/V heads = query heads)."""
    import concurrent.futures as cf
    import os

    from threadpoolctl import threadpool_limits

    h_ = q.shape[2]
    assert k.shape[2] == h_, "per-head split needs as many K/V heads as query heads"
    do = rest[0] if rest and isinstance(rest[0], np.ndarray) and rest[0].ndim == 4 else None
    tail = rest[1:] if do is not None else rest

    def run(h):
        sl = slice(h, h + 1)
        args = [q[:, :, sl], k[:, :, sl], v[:, :, sl]] + ([do[:, :, sl]] if do is not None else []) + list(tail)
        extra = dict(kw)
        if delta_err is not None:
            extra["delta_err"] = delta_err[:, sl]
        return fn(*args, **extra)

    n = threads or min(16, os.cpu_count() or 1)
    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(n) as ex:
            parts = list(ex.map(run, range(h_)))
    out = []
    for i in range(len(parts[0])):
        xs = [p_[i] for p_ in parts]
        out.append(np.concatenate(xs, axis=2 if xs[0].ndim == 4 else 1))
    return tuple(out)


class Guarded:
    """A device tensor of ``shape`` / ``dtype`` placed between two pads of canary bytes, to
    catch writes before or after an output (pads of 4 KiB keep the view 16-byte aligned)."""
    PAD = 4096
    BYTE = 0xA5

    def __init__(self, shape, dtype, fill=None):
        esize = torch.tensor([], dtype=dtype).element_size()
        n = int(np.prod(shape))
        self.buf = torch.full((2 * self.PAD + n * esize,), self.BYTE, dtype=torch.uint8, device="cuda")
        self.t = self.buf[self.PAD:self.PAD + n * esize].view(dtype).view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def check(self, what=""):
        torch.cuda.synchronize()
        head = self.buf[:self.PAD]
        tail = self.buf[-self.PAD:]
        assert bool((head == self.BYTE).all()), f"{what}: write before the output"
        assert bool((tail == self.BYTE).all()), f"{what}: write past the output"
