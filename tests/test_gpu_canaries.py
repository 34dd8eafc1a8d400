"""Output guard canaries: every entry point writes its outputs into buffers framed by canary
bytes, on ragged shapes (sizes that are no multiple of the tiles or vector widths), and the
canaries must be intact afterwards, with the outputs still matching the oracle."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_helpers import Guarded, check, dev, gen, say, shares, values
from oracle import attention as OA
from oracle import permute as OU
from oracle import positions as OP

pytestmark = pytest.mark.gpu

ra = pytest.importorskip("ring_sequence_parallelism_ra_amd")
from ring_sequence_parallelism_ra_amd._lib import ASSIGN, BF16, lib  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


@pytest.mark.parametrize("in_dt,o_dt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32")])
@pytest.mark.parametrize("assign", ["contiguous", "striped", "zigzag"])
def test_ring_share_outputs_guarded(in_dt, o_dt, assign):
    n, s, b, h, d = 3, 130, 2, 3, 64       # ragged against the 128-row and 64-key tiles
    l = n * s
    gq, gk, gv = (gen(5100 + i, (b, l, h, d), in_dt) for i in range(3))
    qs, ks, vs = shares(gq, assign, n), shares(gk, assign, n), shares(gv, assign, n)
    kd, vd = [dev(x, in_dt) for x in ks], [dev(x, in_dt) for x in vs]
    odt = torch.bfloat16 if o_dt == "bf16" else torch.float32
    for r in range(n):
        go, gl = Guarded((b, s, h, d), odt), Guarded((b, h, s), torch.float32)
        ws = Guarded((ra.ring_share_workspace_bytes(b, h, s, d),), torch.uint8)
        qd = dev(qs[r], in_dt)
        ra.ring_share(qd, kd, vd, r, assign=assign, start_step=0, num_steps=1, ws=ws.t)
        ws.check("workspace")
        ra.ring_share(qd, kd, vd, r, assign=assign, start_step=1, num_steps=n - 1, ws=ws.t, o=go.t, lse=gl.t)
        go.check("o")
        gl.check("lse")
        ws.check("workspace")
        qpos = OP.positions(assign, n, r, l)
        o_ref, lse_ref = OA.attention(values(qs[r], in_dt), values(gk, in_dt), values(gv, in_dt), qpos,
                                      np.arange(l), True)
        check(go.t, gl.t, o_ref, lse_ref, in_dt, o_dt, f"guarded rank {r}")


def test_block_attn_and_merge_guarded():
    b, sq, sk, h, d = 1, 77, 45, 2, 128
    q, k, v = (gen(5200 + i, (b, n, h, d), "bf16") for i, n in enumerate((sq, sk, sk)))
    acc_o, acc_l = Guarded((b, sq, h, d), torch.float32), Guarded((b, h, sq), torch.float32)
    ra.block_attn_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), out_dtype=torch.float32, o=acc_o.t,
                      lse=acc_l.t)
    acc_o.check("block o")
    acc_l.check("block lse")
    k2, v2 = gen(5210, (b, sk, h, d), "bf16"), gen(5211, (b, sk, h, d), "bf16")
    bo, bl = ra.block_attn_fwd(dev(q, "bf16"), dev(k2, "bf16"), dev(v2, "bf16"))
    ra.lse_merge(acc_o.t, acc_l.t, bo, bl)
    acc_o.check("merged o")
    acc_l.check("merged lse")
    kk = np.concatenate([values(k, "bf16"), values(k2, "bf16")], axis=1)
    vv = np.concatenate([values(v, "bf16"), values(v2, "bf16")], axis=1)
    o_ref, lse_ref = OA.attention(values(q, "bf16"), kk, vv)
    check(acc_o.t, acc_l.t, o_ref, lse_ref, "bf16", "bf16", "block + merge")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("p,s,hmul,d", [(4, 3, 1, 8), (8, 5, 2, 1), (2, 7, 3, 64)])
def test_permutes_guarded(dt, p, s, hmul, d):
    h, b = p * hmul, 2
    x = gen(5300 + p + s, (p, b, s, h, d), dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    iv, nv = (torch.int16, np.int16) if dt == "bf16" else (torch.int32, np.int32)
    for dst in (p - 1, -1):
        shape = (b, p * s, h // p, d) if dst >= 0 else (p, b, p * s, h // p, d)
        y = Guarded(shape, tdt)
        ra.seq2head_permute(dev(x, dt), dst, out=y.t)
        y.check("permute")
        assert np.array_equal(y.t.cpu().view(iv).numpy(), OU.seq2head(x, dst).view(nv))
        back = Guarded(x.shape, tdt, fill=torch.zeros(x.shape, dtype=tdt))
        ra.head2seq_permute(y.t, dst, back.t)
        back.check("inverse permute")


def test_backward_outputs_guarded():
    assign, n, s, h, d = "zigzag", 2, 130, 2, 128
    l = n * s
    g = [gen(5400 + i, (1, l, h, d), "bf16") for i in range(4)]
    qs, ks, vs, dos = (shares(x, assign, n) for x in g)
    kd, vd = [dev(x, "bf16") for x in ks], [dev(x, "bf16") for x in vs]
    qd, dod = dev(qs[1], "bf16"), dev(dos[1], "bf16")
    o, lse = ra.ring_share(qd, kd, vd, 1, assign=assign)
    dq = Guarded((1, s, h, d), torch.float32)
    dk = [Guarded((1, s, h, d), torch.float32) for _ in range(n)]
    dv = [Guarded((1, s, h, d), torch.float32) for _ in range(n)]
    arr = lambda ts: (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.ra_ring_share_bwd_noalloc(ctypes.c_void_p(qd.data_ptr()), arr(kd), arr(vd), ctypes.c_void_p(o.data_ptr()),
                                       ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(dod.data_ptr()),
                                       ctypes.c_void_p(dq.t.data_ptr()), arr([x.t for x in dk]),
                                       arr([x.t for x in dv]), 1, h, h, s, d, n, 1, ASSIGN[assign], 1, BF16, 0.0,
                                       stream)
    assert rc == 0, lib.ra_last_error()
    dq.check("dq")
    for i in range(n):
        dk[i].check(f"dk {i}")
        dv[i].check(f"dv {i}")
    say("backward outputs guarded")
