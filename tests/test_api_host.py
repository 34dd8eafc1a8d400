"""Host-side checks of the Python binding (no GPU): every wrapper that accepts a caller tensor
rejects a wrong shape or dtype before anything reaches the library, so the kernels never read
or write past a buffer or in the wrong element size."""
import pytest
import torch

ra = pytest.importorskip("ring_sequence_parallelism_ra_amd", reason="libra.so not built")

BF, F32 = torch.bfloat16, torch.float32


def t(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def test_block_attn_rejects_caller_outputs_of_wrong_shape_or_dtype():
    q, k = t(1, 64, 2, 128), t(1, 64, 2, 128)
    with pytest.raises(ValueError, match="o must have shape"):
        ra.block_attn_fwd(q, k, k, o=t(1, 32, 2, 128))
    with pytest.raises(ValueError, match="o must be"):
        ra.block_attn_fwd(q, k, k, o=t(1, 64, 2, 128), out_dtype=F32)
    with pytest.raises(ValueError, match="lse must be"):
        ra.block_attn_fwd(q, k, k, lse=t(1, 2, 64, dtype=torch.float64))
    with pytest.raises(ValueError, match="k must be"):
        ra.block_attn_fwd(q, t(1, 64, 2, 128, dtype=F32), k)
    with pytest.raises(ValueError, match="v must have shape"):
        ra.block_attn_fwd(q, k, t(1, 63, 2, 128))


def test_ring_share_rejects_caller_outputs_of_wrong_shape_or_dtype():
    q = t(1, 64, 2, 128)
    ks = [t(1, 64, 2, 128) for _ in range(2)]
    with pytest.raises(ValueError, match="o must have shape"):
        ra.prepare_ring_share(q, ks, ks, 0, o=t(1, 64, 4, 128))
    with pytest.raises(ValueError, match="lse must have shape"):
        ra.prepare_ring_share(q, ks, ks, 0, lse=t(1, 64, 2, dtype=F32))
    with pytest.raises(ValueError, match="every K/V share"):
        ra.prepare_ring_share(q, [ks[0], t(1, 64, 2, 128, dtype=F32)], ks, 0)


def test_ring_share_bwd_rejects_fp32_forward_output():
    # the backward reads o and dout as bf16 and lse as fp32: an fp32 forward output must not
    # reach it (half of each fp32 row would be read as bf16)
    q = t(1, 64, 2, 128)
    ks = [t(1, 64, 2, 128) for _ in range(2)]
    lse = t(1, 2, 64, dtype=F32)
    with pytest.raises(ValueError, match="o must be"):
        ra.ring_share_bwd(q, ks, ks, t(1, 64, 2, 128, dtype=F32), lse, q, 0)
    with pytest.raises(ValueError, match="dout must be"):
        ra.ring_share_bwd(q, ks, ks, q, lse, t(1, 64, 2, 128, dtype=F32), 0)
    with pytest.raises(ValueError, match="lse must be"):
        ra.ring_share_bwd(q, ks, ks, q, t(1, 2, 64), q, 0)
    with pytest.raises(ValueError, match="q must be"):
        ra.ring_share_bwd(t(1, 64, 2, 128, dtype=F32), ks, ks, q, lse, q, 0)


def test_permutes_reject_mismatched_buffers():
    x = t(4, 1, 8, 8, 64)
    with pytest.raises(ValueError, match="out must have shape"):
        ra.seq2head_permute(x, 1, out=t(1, 32, 4, 64))
    with pytest.raises(ValueError, match="out must be"):
        ra.seq2head_permute(x, 1, out=t(1, 32, 2, 64, dtype=F32))
    with pytest.raises(ValueError, match="does not divide"):
        ra.seq2head_permute(t(4, 1, 8, 6, 64), 0)
    # inverse: y read with out's element size, so both must agree (an fp32 out with a bf16 y
    # would read twice y's bytes)
    with pytest.raises(ValueError, match="y must be"):
        ra.head2seq_permute(t(1, 32, 2, 64), 1, t(4, 1, 8, 8, 64, dtype=F32))
    with pytest.raises(ValueError, match="y must have shape"):
        ra.head2seq_permute(t(1, 16, 2, 64), 1, x)
    with pytest.raises(ValueError, match="y must have shape"):
        ra.head2seq_permute(t(1, 32, 2, 64), -1, x)


def test_merge_rejects_mismatched_buffers():
    o = t(1, 16, 2, 64, dtype=F32)
    lse = t(1, 2, 16, dtype=F32)
    with pytest.raises(ValueError, match="lse_blk must be"):
        ra.lse_merge(o, lse, o, t(1, 2, 16, dtype=torch.float64))
    with pytest.raises(ValueError, match="o_blk must have shape"):
        ra.lse_merge(o, lse, t(1, 16, 2, 32, dtype=F32), lse)


def test_usp_step_rejects_out_of_another_dtype():
    with pytest.raises(ValueError, match="out must be"):
        ra.usp_local_step(t(4, 1, 8, 8, 64), [], [], 0, 0, out=t(4, 1, 8, 8, 64, dtype=F32))
