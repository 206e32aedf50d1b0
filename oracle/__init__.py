"""The oracle: a plain, slow, obviously correct fp64 CPU attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (different language, no common helpers or tables).

What it computes is the plain definition of scaled dot-product attention,
softmax(Q K^T / sqrt(d_k)) V, as written in "FlashAttention — フラッシュ
アテンション" (section 標準的なアテンションの問題点, the display equation),
evaluated the slow three-step way that "Flash Attention 2 / 3 とは 2026年版"
describes in its section on what is wrong with standard attention: form the
score matrix, take a row softmax, multiply by V.  There is no online softmax
and no tiling over keys: scores are materialised for whole rows.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (closed forms, invariants, brute force on tiny
inputs, finite differences, a library cross-check); none is unpinned.
"""
from .attention import (  # noqa: F401
    kv_head_of,
    scores_rows,
    softmax_rows,
    forward_head,
    forward,
    forward_rows,
    forward_kvcache,
    forward_masked,
    forward_masked_rows,
    backward_masked,
    block_mask_dense,
    forward_dense_mask,
    backward_dense_mask,
    forward_blocksparse,
    forward_blocksparse_rows,
    backward_blocksparse,
    visible_range,
    backward_head,
    backward,
)
