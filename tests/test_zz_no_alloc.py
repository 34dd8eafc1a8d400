"""The allocation-free backward entry point (ra_ring_share_bwd_noalloc) against the existing one
(ra_ring_share_bwd with a caller workspace), both called through the C ABI: two calls in a row,
the second on a smaller share, each bit-identical to the workspace form (same kernels, same
inputs) and therefore within the backward's parity bound."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_helpers import dev, gen, say, shares

pytestmark = pytest.mark.gpu

ra = pytest.importorskip("ring_sequence_parallelism_ra_amd")
from ring_sequence_parallelism_ra_amd._lib import ASSIGN, BF16, lib  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def ptrs(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def both(assign, n, s_loc, h, d, seed):
    b, L = 1, n * s_loc
    g = [gen(seed + i, (b, L, h, d), "bf16") for i in range(4)]
    qs, ks, vs, dos = (shares(x, assign, n) for x in g)
    kd, vd = [dev(x, "bf16") for x in ks], [dev(x, "bf16") for x in vs]
    r = n - 1
    qd, dod = dev(qs[r], "bf16"), dev(dos[r], "bf16")
    o, lse = ra.ring_share(qd, kd, vd, r, assign=assign)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    outs = []
    for noalloc in (False, True):
        dq = torch.full((b, s_loc, h, d), float("nan"), device="cuda")
        dk = [torch.full((b, s_loc, h, d), float("nan"), device="cuda") for _ in range(n)]
        dv = [torch.full((b, s_loc, h, d), float("nan"), device="cuda") for _ in range(n)]
        common = (ctypes.c_void_p(qd.data_ptr()), ptrs(kd), ptrs(vd), ctypes.c_void_p(o.data_ptr()),
                  ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(dod.data_ptr()), ctypes.c_void_p(dq.data_ptr()),
                  ptrs(dk), ptrs(dv), b, h, h, s_loc, d, n, r, ASSIGN[assign], 1, BF16, 0.0)
        if noalloc:
            rc = lib.ra_ring_share_bwd_noalloc(*common, stream)
        else:
            wsb = int(lib.ra_ring_share_bwd_workspace_bytes(b, h, s_loc))
            ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
            rc = lib.ra_ring_share_bwd(*common, ctypes.c_void_p(ws.data_ptr()), ws.numel(), stream)
        assert rc == 0, lib.ra_last_error()
        torch.cuda.synchronize()
        outs.append((dq, dk, dv))
    (dq0, dk0, dv0), (dq1, dk1, dv1) = outs
    assert torch.equal(dq0, dq1), "dq differs"
    for i in range(n):
        assert torch.equal(dk0[i], dk1[i]) and torch.equal(dv0[i], dv1[i]), f"share {i} differs"
    assert torch.isfinite(dq1).all()


def test_noalloc_matches_workspace_form_twice():
    say("noalloc bwd: zigzag N=4 S=1024 H=8 D=128")
    both("zigzag", 4, 1024, 8, 128, 4100)
    say("noalloc bwd: striped N=3 S=200 H=2 D=64 (smaller, after the larger call)")
    both("striped", 3, 200, 2, 64, 4200)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    # 8 * B * H * S_loc bytes of row terms must fit the 16 MiB array
    fake = ctypes.c_void_p(0x10000)
    arr = (ctypes.c_void_p * 2)(0x10000, 0x10000)
    rc = lib.ra_ring_share_bwd_noalloc(fake, arr, arr, fake, fake, fake, fake, arr, arr, 1, 32, 32, 65536 + 64, 128,
                                       2, 0, 0, 1, BF16, 0.0, None)
    assert rc == -2 and "scratch" in lib.ra_last_error().decode()
