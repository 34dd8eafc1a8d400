"""Plain, slow, fp64 CPU oracle for the per-device Ring Attention inner loop.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(the HIP library and its Python binding) never imports, links or calls it, and
this package imports nothing from the product.

Sources (cited by page title and section, never by line):
  * [Digest]  "从 Ring Attention 到 DeepSpeed Ulysses，再到 USP 统一框架"
              (jsqmd.com technology digest on sequence parallelism).
  * [Notes]   "主流序列并行(SP)方案对比 + 大模型通信原语"
              (hzhuang.org notes: SP schemes compared, communication primitives).
  * [Q14]     "序列并行（Sequence Parallelism）解决了什么问题？和 TP 是什么关系？"
              (model.playoffer.cn interview answer 14).

What each module follows:
  * ``positions``  -- token -> rank assignment: contiguous ([Digest] §3.4 and the
    "original Ring Attention" listing of §4), striped ([Digest] §4), zigzag
    ([Digest] §6 item 1).
  * ``attention``  -- the definition softmax(Q K^T / sqrt(d)) V of [Digest] §2,
    with the causal visibility of [Digest] §3.4 / [Q14] engineering notes taken
    by global position (key position <= query position).
  * ``ring``       -- the online-softmax recurrence of [Digest] §3.2, the LSE
    merge of [Digest] §6 item 3, and the ring loop of [Digest] §3.1/§3.3.
  * ``permute``    -- the Ulysses sequence-sharded -> head-sharded layout change
    of [Digest] §5.1 (and [Notes] §3), by its index formula.
  * ``counts``     -- brute-force counts of visible (q, k) pairs and of tile
    classes, used for FLOP accounting and to pin the library's planner.
  * ``backward``   -- dQ, dK, dV of the ``attention`` definition by the chain rule
    (the pages train with ring attention but print no backward formulas).

Every function is pinned by ``tests/test_oracle_*.py`` against values fixed by
the pages or by mathematics (page examples, closed forms, a library routine on
special cases, invariants). Readings of silent or garbled passages are listed
in the design notes and repeated at the function that takes them.
"""
from . import positions, attention, ring, permute, counts  # noqa: F401
from .positions import CONTIGUOUS, STRIPED, ZIGZAG  # noqa: F401
