"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds data generation only: Gaussian draws from a named seed, the
float32 -> bfloat16 storage conversion, the workload descriptions and the
choice of sampled query rows. It computes nothing of the attention method
itself (no positions, no masks, no softmax), so both the oracle and the HIP
path can take their inputs from here without sharing any of the method's
arithmetic.

Recipe (the pages give none; this is the stated reading):
  * generator: numpy PCG64, ``standard_normal(dtype=float32)`` multiplied by ``std``; a
    tensor is filled in blocks of ``GEN_ROWS`` leading-dimension rows (all dimensions but
    the first flattened), block ``j`` drawn from ``numpy.random.default_rng([seed, j])``,
    so blocks can be generated in parallel threads with a fixed result;
  * bf16 inputs are those float32 values rounded to nearest-even bfloat16;
  * a workload's Q, K and V are drawn as one *global* tensor ``[B, L, H, D]``
    each, from seeds ``1000*k + 0, 1, 2`` for workload number ``k``; a rank's
    share is then gathered from the global tensor by its token positions;
  * the "std 4" variant scales Q and K (not V) by 4 before rounding.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import CONFIGS, Workload, get  # noqa: F401

GEN_ROWS = 4096          # rows of the flattened leading dimension per generator block
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _blocks(shape):
    shape = tuple(int(x) for x in shape)
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    inner = shape[-1] if len(shape) > 1 else (shape[0] if shape else 1)
    return rows, inner


def _fill(seed: int, shape, std: float, convert):
    rows, inner = _blocks(shape)
    out = np.empty((rows, inner), dtype=np.uint16 if convert else np.float32)
    nblk = (rows + GEN_ROWS - 1) // GEN_ROWS

    def work(j):
        r0, r1 = j * GEN_ROWS, min(rows, (j + 1) * GEN_ROWS)
        x = np.random.default_rng([seed, j]).standard_normal(size=(r1 - r0, inner), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[r0:r1] = f32_to_bf16_bits(x) if convert else x

    if nblk <= 1:
        for j in range(nblk):
            work(j)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(work, range(nblk)))
    return out.reshape(shape)


def gaussian_f32(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """float32 array of iid N(0, std^2) values (see the module recipe)."""
    return _fill(seed, shape, std, convert=False)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returns uint16 bit patterns.

    Inputs here are finite Gaussian draws, so NaN/Inf handling is not needed and
    is rejected rather than silently mangled.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("f32_to_bf16_bits: non-finite input")
    u = x.view(np.uint32).copy()
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)   # finite inputs stay below 2^32 after both additions
    u += lsb
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def gaussian_bf16_bits(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """uint16 bfloat16 bit patterns of iid N(0, std^2) draws (see module recipe)."""
    return _fill(seed, shape, std, convert=True)


def global_qkv(w: "Workload"):
    """Global Q, K, V of a workload, as stored (uint16 bf16 bits or float32).

    Shapes are ``[B, L, H, D]`` for Q and ``[B, L, H_kv, D]`` for K and V. Seeds are
    ``1000*w.number + {0, 1, 2}``.
    """
    q_shape = (w.batch, w.global_len, w.heads, w.head_dim)
    kv_shape = (w.batch, w.global_len, w.heads_kv, w.head_dim)
    shapes = [q_shape, kv_shape, kv_shape]
    seeds = [1000 * w.number + i for i in range(3)]
    stds = [w.qk_std, w.qk_std, 1.0]
    if w.dtype == "bf16":
        return tuple(gaussian_bf16_bits(s, sh, sd) for s, sh, sd in zip(seeds, shapes, stds))
    if w.dtype == "f32":
        return tuple(gaussian_f32(s, sh, sd) for s, sh, sd in zip(seeds, shapes, stds))
    raise ValueError(w.dtype)


def sample_rows(seed: int, n_rows: int, n_random: int = 480, *, chunk_len: int | None = None,
                tile: int = 128) -> np.ndarray:
    """The checked local query rows of a large share: ``n_random`` drawn without
    replacement from ``default_rng(seed + 7)`` plus fixed edge rows (local row 0,
    the first and last row of every chunk of ``chunk_len`` rows, and the first and
    last row of every ``tile``-row tile, evenly thinned to 32 rows). Sorted, unique.
    """
    rng = np.random.default_rng(seed + 7)
    rnd = rng.choice(n_rows, size=min(n_random, n_rows), replace=False)
    edges = {0, n_rows - 1}
    if chunk_len:
        for c0 in range(0, n_rows, chunk_len):
            edges.update({c0, min(c0 + chunk_len, n_rows) - 1})
    tile_edges = sorted({t for t0 in range(0, n_rows, tile) for t in (t0, min(t0 + tile, n_rows) - 1)})
    need = max(0, 32 - len(edges))
    if tile_edges and need:
        idx = np.linspace(0, len(tile_edges) - 1, num=min(need, len(tile_edges))).round().astype(int)
        edges.update(tile_edges[i] for i in idx)
    rows = np.union1d(rnd, np.array(sorted(edges), dtype=np.int64))
    return rows.astype(np.int64)
