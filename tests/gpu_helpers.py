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
