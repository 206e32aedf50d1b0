"""fp64 reference attention (forward and backward), row-blocked.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Readings taken where the pages are silent (each is listed in the design
notes with its reason):

* scale defaults to 1/sqrt(d) -- the d_k of the attention equation in
  "FlashAttention — フラッシュアテンション" (標準的なアテンションの問題点);
* causal: key j is visible to query i iff j <= i (diagonal included);
* GQA: query head h reads K/V head floor(h / (H / H_kv)) (contiguous groups);
* LSE_i = ln sum_{j visible} exp(S_ij), natural log, scale included -- the
  softmax normalisation statistic that "FlashAttentionとは？…" (section
  逆伝播でL×L行列を保存せず再計算する設計) says the forward keeps for the
  backward;
* the backward is the textbook chain rule through the row softmax (the pages
  give only "recompute P from Q/K blocks with the saved statistics").

Inputs are float64 numpy arrays holding exactly the values a kernel receives
(bf16-rounded or fp8-dequantised upstream).
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 512


def kv_head_of(h: int, H: int, H_kv: int) -> int:
    """Grouped-query head map: H/H_kv consecutive query heads share a K/V head.

    GQA support is listed under FlashAttention-2 in "FlashAttention — フラッシュ
    アテンション" (進化と関連技術); the contiguous grouping is the reading taken.
    """
    if H % H_kv:
        raise ValueError("H must be a multiple of H_kv")
    return h // (H // H_kv)


def scores_rows(q_rows, k, scale, causal, row_ids):
    """S = scale * Q K^T for the given query rows, masked entries set to -inf.

    The attention equation's argument QK^T/sqrt(d_k) ("FlashAttention —
    フラッシュアテンション", 標準的なアテンションの問題点), with the causal mask
    of the FA2 paragraph of "Flash Attention 2 / 3 とは 2026年版" (FA2 の改善):
    query i sees keys 0..i.
    """
    s = scale * (q_rows @ k.T)
    if causal:
        n_k = k.shape[0]
        cols = np.arange(n_k)[None, :]
        rows = np.asarray(row_ids)[:, None]
        s = np.where(cols <= rows, s, -np.inf)
    return s


def softmax_rows(s):
    """Row softmax P = exp(S - m) / sum exp(S - m) and its logsumexp m + ln l.

    Subtracting the row max does not change P (it cancels in the ratio); it is
    the max that the online softmax of "FlashAttentionとは？…" (最大値と正規化項を
    持ち回るオンラインsoftmaxの再スケール) carries, here taken over the whole row
    at once.
    """
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    p = e / l
    lse = (m + np.log(l))[:, 0]
    return p, lse


def forward_rows(q, k, v, scale, causal, rows):
    """O and LSE for selected query rows of one head (q [N,d], k/v [N_k,d])."""
    rows = np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.size, v.shape[1]), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    for r0 in range(0, rows.size, ROW_BLOCK):
        rid = rows[r0:r0 + ROW_BLOCK]
        s = scores_rows(q[rid], k, scale, causal, rid)
        p, lse[r0:r0 + ROW_BLOCK] = softmax_rows(s)
        o[r0:r0 + ROW_BLOCK] = p @ v
    return o, lse


def forward_head(q, k, v, scale, causal):
    """Attention(Q,K,V) = softmax(QK^T * scale) V for every row of one head."""
    return forward_rows(q, k, v, scale, causal, np.arange(q.shape[0]))


def forward(q, k, v, scale=None, causal=True):
    """All heads: q [B,H,N,d], k/v [B,H_kv,N,d] -> O [B,H,N,d], LSE [B,H,N]."""
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty((B, H, N, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kv = kv_head_of(h, H, H_kv)
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, kv], v[b, kv], scale, causal)
    return o, lse


def visible_range(i, n, window, causal):
    """Keys query i sees in a sequence of n valid tokens: [lo, hi] (empty if lo > hi).

    The padding mask keeps keys below n (the 2D padding mask of
    "FlashAttentionとは？…", TransformersのFA2における4Dマスクの非対応); the causal
    mask of scores_rows keeps keys up to i; a sliding window of `window`
    (local attention, named for Mistral-style models in the local-LLM guide
    page) keeps keys from i - window on.
    """
    hi = min(i, n - 1) if causal else n - 1
    lo = max(0, i - window) if window is not None and window >= 0 else 0
    return lo, hi


def forward_masked(q, k, v, seqlens=None, window=None, scale=None, causal=True):
    """Attention with a per-sequence padding mask and an optional causal window.

    q [B,H,N,d], k/v [B,H_kv,N,d]; sequence b is valid in rows 0..seqlens[b]-1
    (all N when seqlens is None).  Query i < len_b sees the keys of
    visible_range; rows at or past len_b are padding and are returned as
    O = 0, LSE = -inf (the value of an empty softmax taken here).
    """
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if window is not None and window >= 0 and not causal:
        raise ValueError("a sliding window is causal")
    lens = [N] * B if seqlens is None else [int(x) for x in seqlens]
    if len(lens) != B or any(not 0 <= n <= N for n in lens):
        raise ValueError("seqlens must hold B values in [0, N]")
    o = np.zeros((B, H, N, v.shape[3]), dtype=np.float64)
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        n = lens[b]
        if n == 0:
            continue
        rows = np.arange(n)
        for h in range(H):
            kv = kv_head_of(h, H, H_kv)
            keys, vals = k[b, kv, :n], v[b, kv, :n]         # the valid tokens
            s = scores_rows(q[b, h, :n], keys, scale, causal, rows)
            if window is not None and window >= 0:
                cols = np.arange(keys.shape[0])[None, :]
                s = np.where(cols >= rows[:, None] - window, s, -np.inf)
            p, lse[b, h, :n] = softmax_rows(s)
            o[b, h, :n] = p @ vals
    return o, lse


def forward_masked_rows(q, k, v, n, window, scale, causal, rows):
    """Selected query rows of one head of forward_masked (q [N,d], k/v [N_k,d]),
    for sequence length n: each row's visible keys of visible_range, taken one
    row at a time."""
    rows = np.asarray(rows, dtype=np.int64)
    o = np.zeros((rows.size, v.shape[1]))
    lse = np.full(rows.size, -np.inf)
    for t, i in enumerate(rows):
        if i >= n:
            continue
        lo, hi = visible_range(int(i), n, window, causal)
        s = scale * (k[lo:hi + 1] @ q[i])
        p, l = softmax_rows(s[None, :])
        o[t] = p[0] @ v[lo:hi + 1]
        lse[t] = l[0]
    return o, lse


def backward_masked(q, k, v, do, seqlens=None, window=None, scale=None, causal=True):
    """Gradients of L = sum(O * dO) for forward_masked.

    Only the valid tokens of each sequence take part: the chain rule of
    backward_head runs on the unpadded sequence with the window applied to its
    scores, and padding rows and keys get zero gradients (padding outputs are
    the constant 0, so their dO does not matter).
    """
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lens = [N] * B if seqlens is None else [int(x) for x in seqlens]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        n = lens[b]
        if n == 0:
            continue
        rows = np.arange(n)
        for h in range(H):
            kv = kv_head_of(h, H, H_kv)
            qs, ks, vs, dos = q[b, h, :n], k[b, kv, :n], v[b, kv, :n], do[b, h, :n]
            s = scores_rows(qs, ks, scale, causal, rows)
            if window is not None and window >= 0:
                s = np.where(np.arange(n)[None, :] >= rows[:, None] - window, s, -np.inf)
            p, _ = softmax_rows(s)
            dp = dos @ vs.T
            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dq[b, h, :n] = scale * (ds @ ks)
            dk[b, kv, :n] += scale * (ds.T @ qs)
            dv[b, kv, :n] += p.T @ dos
    return dq, dk, dv


def block_mask_dense(block_mask, n, block, causal):
    """The [H, n, n] boolean key-visibility matrix of a block mask.

    block_mask [H, nb, nb] (nonzero: query block qb sees key block kb) is
    the block-sparse pattern of "FlashAttentionとは？…" (逆伝播でL×L行列を
    保存せず再計算する設計: block-sparse FlashAttention at 64K); element (i, j)
    is visible iff its block is on, and under the causal mask also j <= i.
    """
    bm = np.asarray(block_mask) != 0
    idx = np.arange(n) // block
    vis = bm[:, idx][:, :, idx]
    if causal:
        vis = vis & (np.arange(n)[None, :] <= np.arange(n)[:, None])[None]
    return vis


def forward_dense_mask(q, k, v, vis, scale=None):
    """Attention with an explicit visibility matrix vis [H, N, N]; a row that
    sees no key is O = 0, LSE = -inf."""
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros((B, H, N, v.shape[3]))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            kv = kv_head_of(h, H, H_kv)
            rows = np.flatnonzero(vis[h].any(axis=1))
            if rows.size == 0:
                continue
            s = np.where(vis[h][rows], scale * (q[b, h, rows] @ k[b, kv].T), -np.inf)
            p, lse[b, h, rows] = softmax_rows(s)
            o[b, h, rows] = p @ v[b, kv]
    return o, lse


def backward_dense_mask(q, k, v, do, vis, scale=None):
    """Gradients of sum(O * dO) for forward_dense_mask (rows that see no key
    contribute nothing)."""
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            kv = kv_head_of(h, H, H_kv)
            rows = np.flatnonzero(vis[h].any(axis=1))
            if rows.size == 0:
                continue
            s = np.where(vis[h][rows], scale * (q[b, h, rows] @ k[b, kv].T), -np.inf)
            p, _ = softmax_rows(s)
            dp = do[b, h, rows] @ v[b, kv].T
            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dq[b, h, rows] = scale * (ds @ k[b, kv])
            dk[b, kv] += scale * (ds.T @ q[b, h, rows])
            dv[b, kv] += p.T @ do[b, h, rows]
    return dq, dk, dv


def forward_blocksparse(q, k, v, block_mask, block=128, scale=None, causal=True):
    """Block-sparse attention: forward_dense_mask of block_mask_dense."""
    return forward_dense_mask(q, k, v, block_mask_dense(block_mask, q.shape[2], block, causal), scale)


def backward_blocksparse(q, k, v, do, block_mask, block=128, scale=None, causal=True):
    return backward_dense_mask(q, k, v, do, block_mask_dense(block_mask, q.shape[2], block, causal), scale)


def forward_blocksparse_rows(q, k, v, block_mask, block, scale, causal, rows):
    """Selected query rows of one head of forward_blocksparse (q [N,d], k/v
    [N,d], block_mask [nb, nb] of that head), one row at a time."""
    bm = np.asarray(block_mask) != 0
    n = k.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    o = np.zeros((rows.size, v.shape[1]))
    lse = np.full(rows.size, -np.inf)
    kblock = np.arange(n) // block
    for t, i in enumerate(rows):
        vis = bm[i // block][kblock]
        if causal:
            vis = vis & (np.arange(n) <= i)
        js = np.flatnonzero(vis)
        if js.size == 0:
            continue
        p, l = softmax_rows((scale * (k[js] @ q[i]))[None, :])
        o[t] = p[0] @ v[js]
        lse[t] = l[0]
    return o, lse


def forward_kvcache(q, k, v, kv_len=None, scale=None, causal=True):
    """Attention of a few new queries against a KV cache.

    q [B,H,N_q,d]; k/v [B,H_kv,N_kv,d] hold the cache, of which batch b uses
    the first kv_len[b] rows (all N_kv when kv_len is None).  The decode case
    of "FlashAttentionとは？…" (短い系列の効果とデコード向け最適化の違い): the
    query side is short (one token per step) and the whole cache is read.
    The N_q queries are taken to be the last N_q positions of the sequence,
    so query i sits at position kv_len - N_q + i and, under the causal mask
    of scores_rows, sees keys 0..kv_len - N_q + i.  A row that sees no key
    (an empty cache, or kv_len < N_q under the mask) has no softmax; its
    output is taken as zero and its LSE as -inf (the log of an empty sum).
    Returns O [B,H,N_q,d_v] and LSE [B,H,N_q].
    """
    B, H, n_q, d = q.shape
    H_kv, n_kv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lens = [n_kv] * B if kv_len is None else [int(x) for x in kv_len]
    if len(lens) != B or any(not 0 <= n <= n_kv for n in lens):
        raise ValueError("kv_len must hold B values in [0, N_kv]")
    o = np.zeros((B, H, n_q, v.shape[3]), dtype=np.float64)
    lse = np.full((B, H, n_q), -np.inf)
    for b in range(B):
        n = lens[b]
        pos = n - n_q + np.arange(n_q)                    # positions of the queries
        n_seen = np.clip(pos + 1, 0, n) if causal else np.full(n_q, n)
        rows = np.flatnonzero(n_seen > 0)
        if rows.size == 0:
            continue
        for h in range(H):
            kv = kv_head_of(h, H, H_kv)
            s = scores_rows(q[b, h, rows], k[b, kv, :n], scale, causal, pos[rows])
            p, lse[b, h, rows] = softmax_rows(s)
            o[b, h, rows] = p @ v[b, kv, :n]
    return o, lse


def backward_head(q, k, v, do, scale, causal):
    """Gradients of L = sum(O * dO) with respect to Q, K, V for one head.

    Recomputes P from Q and K (the backward-by-recompute paragraph of
    "FlashAttentionとは？…", 逆伝播でL×L行列を保存せず再計算する設計) and applies
    the chain rule of O = P V and of the row softmax:
      dV = P^T dO;  dP = dO V^T;  dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik);
      dQ = scale dS K;  dK = scale dS^T Q.
    Returns dq, dk, dv, O, LSE (all float64).
    """
    n_q, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.empty((n_q, v.shape[1]))
    lse = np.empty(n_q)
    for r0 in range(0, n_q, ROW_BLOCK):
        rid = np.arange(r0, min(n_q, r0 + ROW_BLOCK))
        s = scores_rows(q[rid], k, scale, causal, rid)
        p, lse[rid] = softmax_rows(s)
        o[rid] = p @ v
        dp = do[rid] @ v.T
        row_dot = np.sum(p * dp, axis=1, keepdims=True)
        ds = p * (dp - row_dot)
        dq[rid] = scale * (ds @ k)
        dk += scale * (ds.T @ q[rid])
        dv += p.T @ do[rid]
    return dq, dk, dv, o, lse


def backward(q, k, v, do, scale=None, causal=True):
    """All heads; K/V gradients of a GQA group are summed over its query heads."""
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            kv = kv_head_of(h, H, H_kv)
            gq, gk, gv, _, _ = backward_head(q[b, h], k[b, kv], v[b, kv], do[b, h], scale, causal)
            dq[b, h] = gq
            dk[b, kv] += gk
            dv[b, kv] += gv
    return dq, dk, dv
