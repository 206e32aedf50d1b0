"""Exact gradients of a few key blocks of a large block-sparse problem from a
small sub-problem (test helper; only the oracle does arithmetic here).

The dK, dV rows of key block kb depend only on the query rows that see kb,
and those rows' probabilities depend only on the key blocks they see.  So
attention restricted to those query blocks and the union of their key
blocks, with the visibility of the full problem, gives exactly those rows'
dQ and the key block's dK, dV."""
import numpy as np
import torch

import oracle


def sparse_causal_mask(H, nb, per_row, seed):
    """The diagonal block plus per_row random earlier blocks in each query block row."""
    g = torch.Generator().manual_seed(seed)
    m = torch.zeros(H, nb, nb, dtype=torch.uint8)
    idx = torch.arange(nb)
    m[:, idx, idx] = 1
    cols = (torch.rand(H, nb, per_row, generator=g) * (idx[None, :, None] + 1)).long()
    m.scatter_(2, cols, torch.ones_like(cols, dtype=torch.uint8))
    return m


def span(blocks, n, block=128):
    return np.concatenate([np.arange(qb * block, min(qb * block + block, n)) for qb in blocks])


def key_block_grads(q, k, v, do, bm, kv, kb, scale, causal=True, block=128):
    """For K/V head kv (q, do [H, N, d], k, v [H_kv, N, d], fp64; bm [H, nb, nb]
    bool): a list of (head, query rows, their dQ) for the heads that see key
    block kb, and kb's dK, dV rows summed over the group's heads."""
    H, n = q.shape[0], q.shape[1]
    g = H // k.shape[0]
    keys_kb = span([kb], n, block)
    dk = np.zeros((keys_kb.size, k.shape[2]))
    dv = np.zeros((keys_kb.size, v.shape[2]))
    dqs = []
    for h in range(kv * g, (kv + 1) * g):
        qbs = np.flatnonzero(bm[h, :, kb])
        if qbs.size == 0:
            continue
        kbs = np.flatnonzero(bm[h, qbs].any(axis=0))
        rows, keys = span(qbs, n, block), span(kbs, n, block)
        vis = bm[h][np.ix_(rows // block, keys // block)]
        if causal:
            vis = vis & (keys[None, :] <= rows[:, None])
        gq, gk, gv = oracle.backward_dense_mask(q[h, rows][None, None], k[kv, keys][None, None],
                                                v[kv, keys][None, None], do[h, rows][None, None], vis[None], scale)
        dqs.append((h, rows, gq[0, 0]))
        at = np.searchsorted(keys, keys_kb)
        dk += gk[0, 0][at]
        dv += gv[0, 0][at]
    return dqs, dk, dv
