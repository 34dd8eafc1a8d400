"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds data generation only: Gaussian draws from a named seed, the
float32 -> bfloat16 storage conversion, the five workload descriptions and the
choice of sampled query rows. It computes nothing of the attention method
itself (no positions, no masks, no softmax), so both the oracle and the HIP
path can take their inputs from here without sharing any of the method's
arithmetic.

Recipe (the pages give none; this is the stated reading):
  * generator: ``numpy.random.default_rng(seed)`` (PCG64),
    ``standard_normal(dtype=float32)``, multiplied by ``std``;
  * bf16 inputs are those float32 values rounded to nearest-even bfloat16;
  * a workload's Q, K and V are drawn as one *global* tensor ``[B, L, H, D]``
    each, from seeds ``1000*k + 0, 1, 2`` for workload number ``k``; a rank's
    share is then gathered from the global tensor by its token positions;
  * the "std 4" variant scales Q and K (not V) by 4 before rounding.
"""
from __future__ import annotations

import numpy as np

from .configs import CONFIGS, Workload, get  # noqa: F401


def gaussian_f32(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """float32 array of iid N(0, std^2) values from PCG64 seeded with ``seed``."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returns uint16 bit patterns.

    Inputs here are finite Gaussian draws, so NaN/Inf handling is not needed and
    is rejected rather than silently mangled.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("f32_to_bf16_bits: non-finite input")
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def gaussian_bf16_bits(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """uint16 bfloat16 bit patterns of iid N(0, std^2) draws (see module recipe)."""
    return f32_to_bf16_bits(gaussian_f32(seed, shape, std))


def global_qkv(w: "Workload"):
    """Global Q, K, V of a workload, as stored (uint16 bf16 bits or float32).

    Shapes are ``[B, L, H, D]``. Seeds are ``1000*w.number + {0, 1, 2}``.
    """
    shape = (w.batch, w.global_len, w.heads, w.head_dim)
    seeds = [1000 * w.number + i for i in range(3)]
    stds = [w.qk_std, w.qk_std, 1.0]
    if w.dtype == "bf16":
        return tuple(gaussian_bf16_bits(s, shape, sd) for s, sd in zip(seeds, stds))
    if w.dtype == "f32":
        return tuple(gaussian_f32(s, shape, sd) for s, sd in zip(seeds, stds))
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
