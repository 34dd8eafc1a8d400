"""ctypes binding of ``libra.so`` (the C ABI in ``include/ra.h``).

Argument marshalling only: tensors become device pointers and sizes, streams become
``hipStream_t`` handles, statuses become exceptions. Every step of the computation runs in
the HIP library; there is no fallback. If the library has not been built, importing this
module raises ``ImportError``.
"""
from __future__ import annotations

import ctypes
import os

# torch ships its own HIP runtime with the same soname (libamdhip64.so.7) as the system one that
# libra.so links against; the dynamic loader serves the whole process from whichever copy is
# loaded first. Importing torch first makes the library and torch share torch's runtime (one
# device context, one set of streams).
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libra.so")

RA_OK = 0
F32, BF16 = 0, 1
CONTIGUOUS, STRIPED, ZIGZAG = 0, 1, 2
ASSIGN = {"contiguous": CONTIGUOUS, "striped": STRIPED, "zigzag": ZIGZAG}
STATUS = {0: "RA_OK", -1: "RA_ERR_INVALID_ARG", -2: "RA_ERR_UNSUPPORTED", -3: "RA_ERR_SHAPE",
          -4: "RA_ERR_MISALIGNED", -5: "RA_ERR_HIP"}

# Every function the header declares, in declaration order.
EXPORTS = ["ra_block_attn_fwd", "ra_lse_merge", "ra_ring_share_workspace_bytes", "ra_ring_share",
           "ra_ring_share_bwd_workspace_bytes", "ra_ring_share_bwd", "ra_ring_share_bwd_noalloc", "ra_seq2head_permute", "ra_seq2head_permute_n", "ra_last_error",
           "ra_share_work", "ra_tile_shape", "ra_debug_positions", "ra_debug_mask", "ra_debug_tile_count_slots",
           "ra_debug_tile_counts"]


class RaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class Shard(ctypes.Structure):
    """``ra_shard``: token assignment of a global sequence over ``world`` ranks."""
    _fields_ = [("assign", ctypes.c_int32), ("world", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("global_len", ctypes.c_int64)]

    def __init__(self, assign, world, rank, global_len):
        super().__init__(ASSIGN.get(assign, assign), world, rank, global_len)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I, F, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    SH = ctypes.POINTER(Shard)
    sig = {
        "ra_block_attn_fwd": (I, [P, P, P, P, P, I64, I64, I64, I64, I64, I64, I, I, I, SH, SH, F, P]),
        "ra_lse_merge": (I, [P, P, P, P, I64, I64, I64, I64, I, I, P]),
        "ra_ring_share_workspace_bytes": (SZ, [I64, I64, I64, I64]),
        "ra_ring_share": (I, [P, P, P, P, P, I64, I64, I64, I64, I64, I, I, I, I, I, I, F, I, I, P, SZ, P]),
        "ra_ring_share_bwd_workspace_bytes": (SZ, [I64, I64, I64]),
        "ra_ring_share_bwd": (I, [P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I, I, I, I, I, F, P, SZ, P]),
        "ra_ring_share_bwd_noalloc": (I, [P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I, I, I, I, I, F, P]),
        "ra_seq2head_permute": (I, [P, P, I64, I64, I64, I64, I64, I, I, I, P]),
        "ra_seq2head_permute_n": (I, [P, P, I, I64, I64, I64, I64, I64, I, I, I, P]),
        "ra_last_error": (ctypes.c_char_p, []),
        "ra_share_work": (I, [SH, SH, I64, I64, I, I64, I64, ctypes.POINTER(I64)]),
        "ra_tile_shape": (I, [I, I64, ctypes.POINTER(I64), ctypes.POINTER(I64)]),
        "ra_debug_positions": (I, [SH, P, P]),
        "ra_debug_mask": (I, [SH, SH, I64, I64, P, P]),
        "ra_debug_tile_count_slots": (I64, [I64, I64, I64]),
        "ra_debug_tile_counts": (I, [P, P, P, P, P, I64, I64, I64, I64, I64, I, I, I, I, I, F, P, I64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def check(code: int) -> None:
    if code != RA_OK:
        raise RaError(code, lib.ra_last_error().decode(errors="replace"))


def last_error() -> str:
    return lib.ra_last_error().decode(errors="replace")
