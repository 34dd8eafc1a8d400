"""MI355X-native per-device Ring Attention inner loop.

Blockwise causal attention of one local Q share against the ring's KV shares with the
online-softmax / LSE update, under contiguous, striped and zigzag token assignments, plus
the Ulysses sequence->head permute. The computation runs in hand-written HIP kernels for
gfx950 behind the C ABI of ``include/ra.h`` (``libra.so``, built in-tree); this package is
the thin ctypes binding over it. Importing fails if the library has not been built.
"""
from ._lib import (ASSIGN, BF16, CONTIGUOUS, EXPORTS, F32, LIB_PATH, STRIPED, ZIGZAG, RaError,  # noqa: F401
                   Shard, last_error, lib)
from .api import (block_attn_fwd, debug_mask, debug_positions, debug_tile_counts, head2seq_permute,  # noqa: F401
                  lse_merge, prepare_ring_share, ring_share, ring_share_bwd, ring_share_workspace,
                  ring_share_workspace_bytes, seq2head_permute, seq2head_permute_n, share_work, tile_shape,
                  torch_dtype, usp_local_step)
