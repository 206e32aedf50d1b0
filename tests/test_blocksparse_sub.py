"""The sub-problem reduction behind the full-size block-sparse backward test
(tests/blocksparse_sub.py) gives exactly the oracle's whole-problem
gradients for every key block, so a GPU result checked against it is checked
against the oracle."""
import numpy as np

import blocksparse_sub as bsub
import oracle


def test_key_block_grads_match_the_whole_problem():
    H, H_kv, N, d = 4, 2, 700, 16
    rng = np.random.default_rng(3)
    q = rng.standard_normal((H, N, d))
    k = rng.standard_normal((H_kv, N, d))
    v = rng.standard_normal((H_kv, N, d))
    do = rng.standard_normal((H, N, d))
    nb = (N + 127) // 128
    bm = bsub.sparse_causal_mask(H, nb, 2, 9).numpy() != 0
    assert 0.2 < bm.mean() < 0.6
    scale = 0.3
    gq, gk, gv = oracle.backward_blocksparse(q[None], k[None], v[None], do[None], bm, 128, scale, True)
    seen_rows = 0
    for kv in range(H_kv):
        for kb in range(nb):
            dqs, dk, dv = bsub.key_block_grads(q, k, v, do, bm, kv, kb, scale)
            keys = bsub.span([kb], N)
            np.testing.assert_allclose(dk, gk[0, kv, keys], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(dv, gv[0, kv, keys], rtol=1e-10, atol=1e-12)
            for h, rows, g in dqs:
                np.testing.assert_allclose(g, gq[0, h, rows], rtol=1e-10, atol=1e-12)
                seen_rows += rows.size
    assert seen_rows > 0
