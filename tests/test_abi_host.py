"""Host-side checks of the C ABI (no GPU): symbols, argument validation, planner counts."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ra = pytest.importorskip("ring_sequence_parallelism_ra_amd", reason="libra.so not built")
from ring_sequence_parallelism_ra_amd import _lib  # noqa: E402
from ring_sequence_parallelism_ra_amd._lib import Shard, lib  # noqa: E402

from oracle import counts as OC  # noqa: E402
from oracle import positions as OP  # noqa: E402

OK, INVALID, UNSUP, SHAPE, MISALIGNED = 0, -1, -2, -3, -4
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first


def header_functions():
    text = open(os.path.join(ROOT, "include", "ra.h")).read()
    return re.findall(r"^\s*(?:const\s+)?[\w\*\s]+?\b(ra_\w+)\s*\(", text, flags=re.M)


def test_exports_every_declared_symbol():
    declared = set(header_functions())
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_exported_symbols_in_dynamic_table():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in header_functions():
        assert name in syms, name


def test_no_undefined_library_symbols():
    # Every symbol the library itself defines must resolve: a kernel whose host launch stub
    # went missing shows up as an undefined ra:: symbol (the dynamic loader only fails lazily).
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    own = [ln for ln in out.splitlines() if "_ZN2ra" in ln or " ra_" in ln]
    assert not own, own


def call_block(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=2, Sq=64, Sk=64, D=128, ind=1, od=1, causal=0,
             qs=None, ks=None, scale=0.0)
    a.update(over)
    hkv = a.get("Hkv", a["H"])
    return lib.ra_block_attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], hkv, a["Sq"], a["Sk"],
                                 a["D"], a["ind"], a["od"], a["causal"], a["qs"], a["ks"], a["scale"], None)


def test_block_attn_validation():
    assert call_block(D=96) == UNSUP
    assert call_block(ind=3) == UNSUP
    assert call_block(q=None) == INVALID
    assert call_block(k=ctypes.c_void_p(0x10008)) == MISALIGNED
    assert call_block(B=-1) == INVALID
    assert call_block(scale=float("nan")) == INVALID
    # grouped-query attention: KV heads must be >= 1 and divide the query heads
    assert call_block(H=4, Hkv=0) == INVALID
    assert call_block(H=6, Hkv=4) == SHAPE
    assert "divide" in _lib.last_error()
    assert call_block(H=4, Hkv=-1) == INVALID
    # 32-bit limits: byte offsets inside a 64-row K/V tile, and the launch grid
    assert call_block(H=1 << 16) == UNSUP                 # 2^16 heads x 128 x 2 B = 2^24-byte rows
    assert "2^24" in _lib.last_error()
    assert call_block(H=(1 << 16) - 8, B=0, q=None, k=None, v=None, o=None, lse=None) == OK
    assert call_block(B=1 << 14, H=1 << 10, Sq=1 << 13, Sk=64) == UNSUP   # 128 x 2^24 workgroups
    assert "grid" in _lib.last_error()
    # causal needs shard descriptors matching the sizes
    assert call_block(causal=1) == INVALID
    qs = Shard("zigzag", 4, 1, 256)   # share 64
    ks = Shard("zigzag", 4, 5, 256)   # rank out of range
    assert call_block(causal=1, qs=ctypes.byref(qs), ks=ctypes.byref(ks)) == INVALID
    ks = Shard("zigzag", 4, 0, 250)   # 250 % 8 != 0
    assert call_block(causal=1, qs=ctypes.byref(qs), ks=ctypes.byref(ks)) == SHAPE
    ks = Shard("contiguous", 2, 0, 256)  # share 128 != Sk 64
    assert call_block(causal=1, qs=ctypes.byref(qs), ks=ctypes.byref(ks)) == SHAPE
    assert "share length" in _lib.last_error()
    # empty inputs are valid and launch nothing (so they succeed without a GPU)
    assert call_block(B=0, q=None, k=None, v=None, o=None, lse=None) == OK
    assert call_block(Sq=0, q=None, o=None, lse=None) == OK


def call_ring(**over):
    n = over.pop("N", 4)
    arr = (ctypes.c_void_p * max(n, 1))(*([0x10000] * max(n, 1)))
    a = dict(q=FAKE, ks=arr, vs=arr, o=FAKE, lse=FAKE, B=1, H=2, S=64, D=128, N=n, rank=0, assign=0, causal=1,
             ind=1, od=1, scale=0.0, start=0, num=n, ws=None, wsb=0)
    a.update(over)
    hkv = a.get("Hkv", a["H"])
    return lib.ra_ring_share(a["q"], a["ks"], a["vs"], a["o"], a["lse"], a["B"], a["H"], hkv, a["S"], a["D"], a["N"],
                             a["rank"], a["assign"], a["causal"], a["ind"], a["od"], a["scale"], a["start"],
                             a["num"], a["ws"], a["wsb"], None)


def test_ring_share_validation():
    assert call_ring(N=0, num=1) == INVALID
    assert call_ring(N=65, num=65) == UNSUP
    assert call_ring(rank=4) == INVALID
    assert call_ring(assign=7) == INVALID
    assert call_ring(start=2, num=3) == INVALID           # past N
    assert call_ring(num=0) == INVALID
    assert call_ring(assign=2, S=63) == SHAPE              # zigzag needs even share
    nulls = (ctypes.c_void_p * 4)(0x10000, 0, 0x10000, 0x10000)
    assert call_ring(ks=nulls) == INVALID
    mis = (ctypes.c_void_p * 4)(0x10000, 0x10004, 0x10000, 0x10000)
    assert call_ring(vs=mis) == MISALIGNED
    # partial runs need a workspace of the right size
    assert call_ring(start=0, num=2) == INVALID
    need = lib.ra_ring_share_workspace_bytes(1, 2, 64, 128)
    assert need == 4 * 64 * 2 * 128 + 16 * 2 * 64
    assert call_ring(start=1, num=3, ws=FAKE, wsb=need - 4) == INVALID
    # a resume needs a state this process stored in that workspace
    assert call_ring(start=1, num=3, ws=ctypes.c_void_p(0x20000), wsb=need) == INVALID
    assert "no running state" in _lib.last_error()
    assert call_ring(D=64, ind=5) == UNSUP
    assert call_ring(H=4, Hkv=3) == SHAPE
    assert call_ring(H=4, Hkv=0) == INVALID
    assert call_ring(B=0, q=None) == OK


def call_bwd(**over):
    n = over.pop("N", 4)
    arr = (ctypes.c_void_p * max(n, 1))(*([0x10000] * max(n, 1)))
    a = dict(q=FAKE, ks=arr, vs=arr, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dks=arr, dvs=arr, B=1, H=2, Hkv=2, S=64,
             D=128, N=n, rank=0, assign=0, causal=1, ind=1, scale=0.0, ws=FAKE, wsb=1 << 20)
    a.update(over)
    return lib.ra_ring_share_bwd(a["q"], a["ks"], a["vs"], a["o"], a["lse"], a["do"], a["dq"], a["dks"], a["dvs"],
                                 a["B"], a["H"], a["Hkv"], a["S"], a["D"], a["N"], a["rank"], a["assign"], a["causal"],
                                 a["ind"], a["scale"], a["ws"], a["wsb"], None)


def test_ring_share_bwd_validation():
    assert lib.ra_ring_share_bwd_workspace_bytes(2, 3, 100) == 8 * 2 * 3 * 100
    assert call_bwd(ind=0) == UNSUP                       # fp32 inputs: forward only
    assert call_bwd(D=96) == UNSUP
    assert call_bwd(N=0) == INVALID
    assert call_bwd(rank=4) == INVALID
    assert call_bwd(Hkv=3, H=4) == SHAPE
    assert call_bwd(assign=2, S=63) == SHAPE
    assert call_bwd(ws=None) == INVALID
    assert call_bwd(wsb=8 * 2 * 64 - 4) == INVALID
    assert call_bwd(dq=ctypes.c_void_p(0x10004)) == MISALIGNED
    nulls = (ctypes.c_void_p * 4)(0x10000, 0x10000, 0, 0x10000)
    assert call_bwd(dvs=nulls) == INVALID
    assert call_bwd(B=0, q=None, o=None) == OK            # empty: nothing launched


def test_ring_share_bwd_noalloc_validation():
    # same checks as the workspace form, plus the size of the static device scratch (16 MiB of
    # row terms, 8 bytes per (batch, head, row)), all on the host
    f = lib.ra_ring_share_bwd_noalloc
    arr = (ctypes.c_void_p * 2)(0x10000, 0x10000)
    args = lambda **o: [o.get(k, v) for k, v in (("q", FAKE), ("ks", arr), ("vs", arr), ("o", FAKE), ("lse", FAKE),
                                                 ("do", FAKE), ("dq", FAKE), ("dks", arr), ("dvs", arr), ("B", 1),
                                                 ("H", 32), ("Hkv", 32), ("S", 65536), ("D", 128), ("N", 2), ("rank", 0),
                                                 ("assign", 0), ("causal", 1), ("ind", 1), ("scale", 0.0), ("st", None))]
    assert f(*args(S=65536 + 64)) == UNSUP and "scratch" in _lib.last_error()
    assert f(*args(ind=0)) == UNSUP
    assert f(*args(rank=2)) == INVALID
    assert f(*args(dq=ctypes.c_void_p(0x10004))) == MISALIGNED
    assert f(*args(B=0, q=None)) == OK


def test_permute_validation():
    f = lib.ra_seq2head_permute
    assert f(FAKE, FAKE, 1, 4, 8, 6, 128, 1, 0, 0, None) == SHAPE          # 4 does not divide 6
    assert f(FAKE, FAKE, 1, 4, 8, 8, 128, 1, 4, 0, None) == INVALID        # dst rank
    assert f(FAKE, FAKE, 1, 0, 8, 8, 128, 1, 0, 0, None) == INVALID        # P < 1
    assert f(FAKE, FAKE, 1, 4, 8, 8, 128, 9, 0, 0, None) == UNSUP
    assert f(ctypes.c_void_p(0x10002), FAKE, 1, 4, 8, 8, 128, 1, 0, 0, None) == MISALIGNED
    assert f(None, None, 1, 4, 0, 8, 128, 1, 0, 0, None) == OK              # empty


def test_permute_n_validation():
    f = lib.ra_seq2head_permute_n
    arr = (ctypes.c_void_p * 3)(0x10000, 0x10000, 0x10000)
    assert f(arr, arr, 9, 1, 4, 8, 8, 128, 1, 0, 0, None) == INVALID     # more than RA_MAX_PERMUTE
    assert f(arr, arr, -1, 1, 4, 8, 8, 128, 1, 0, 0, None) == INVALID
    assert f(arr, arr, 3, 1, 4, 8, 6, 128, 1, 0, 0, None) == SHAPE       # 4 does not divide 6
    nulls = (ctypes.c_void_p * 3)(0x10000, 0, 0x10000)
    assert f(arr, nulls, 3, 1, 4, 8, 8, 128, 1, 0, 0, None) == INVALID
    mis = (ctypes.c_void_p * 3)(0x10000, 0x10000, 0x10008)
    assert f(mis, arr, 3, 1, 4, 8, 8, 128, 1, 0, 0, None) == MISALIGNED
    assert f(None, None, 0, 1, 4, 8, 8, 128, 1, 0, 0, None) == OK         # nothing to move


def test_merge_validation():
    f = lib.ra_lse_merge
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 4, 12, 1, 1, None) == UNSUP      # D % 8
    assert f(FAKE, FAKE, None, FAKE, 1, 2, 4, 16, 1, 1, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 4, 16, 1, 2, None) == UNSUP
    assert f(None, None, None, None, 0, 2, 4, 16, 1, 1, None) == OK


def test_last_error_cleared_on_success():
    assert call_block(D=96) == UNSUP and _lib.last_error()
    assert call_block(B=0, q=None, k=None, v=None, o=None, lse=None) == OK
    assert _lib.last_error() == ""


def test_tile_shape():
    assert ra.tile_shape(1, 128) == (128, 64)
    assert ra.tile_shape(0, 64) == (64, 32)
    with pytest.raises(ra.RaError):
        ra.tile_shape(1, 80)


@pytest.mark.parametrize("assign", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("n,l", [(1, 256), (2, 320), (4, 1024), (8, 8192)])
@pytest.mark.parametrize("bm,bn", [(128, 64), (64, 32), (128, 128), (7, 5)])
def test_share_work_matches_oracle(assign, n, l, bm, bn):
    s = l // n
    for r in sorted({0, n // 2, n - 1}):
        qpos = OP.positions(assign, n, r, l)
        for src in sorted({0, (r - 1) % n, r, n - 1}):
            kpos = OP.positions(assign, n, src, l)
            got = ra.share_work(Shard(assign, n, r, l), Shard(assign, n, src, l), s, s, True, bm, bn)
            want = (OC.visible_pairs(qpos, kpos),) + OC.tile_classes(qpos, kpos, bm, bn)
            assert got == want, (r, src)


@pytest.mark.parametrize("assign", ["contiguous", "striped", "zigzag"])
def test_share_work_at_the_length_limit(assign):
    # The host planner runs the kernels' own position and prefix-count functions (32-bit
    # arithmetic): at the largest accepted global length and ring size they must still count
    # every visible pair exactly.
    n = 64
    l = ((1 << 31) - 1) // (2 * n) * (2 * n)
    s = l // n
    r, src = 45, 12
    got = ra.share_work(Shard(assign, n, r, l), Shard(assign, n, src, l), s, s, True, 128, 64)
    assert got[0] == OC.visible_pairs(OP.positions(assign, n, r, l), OP.positions(assign, n, src, l))
    assert got[1] + got[2] + got[3] == ((s + 127) // 128) * ((s + 63) // 64)


def test_share_work_noncausal_ragged():
    assert ra.share_work(None, None, 100, 70, False, 64, 32) == (7000, 2 * 3, 0, 0)
