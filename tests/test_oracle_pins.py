"""CPU tests that pin the fp64 oracle to facts outside itself.

Besides the pins of ``tests/pins.py`` this file cross-checks the oracle with
PyTorch's own CPU attention (a library routine computing the same
definition), compares it with the fp32 rounding level the pages measured for
two exact CPU implementations, and plants mistakes in copies of the oracle to
show that every plausible slip is caught by at least one pin.
"""
import math
import os
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.attention as oa
from tests import pins

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oa)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 4, 4, 33, 16), (1, 8, 2, 70, 32), (1, 2, 1, 129, 64)])
def test_matches_torch_sdpa_fp64(shape, causal):
    """Library cross-check: torch's CPU SDPA (math path) in float64, with autograd."""
    B, H, H_kv, N, d = shape
    g = torch.Generator().manual_seed(sum(shape) + causal)
    q = torch.randn(B, H, N, d, generator=g, dtype=torch.float64, requires_grad=True)
    k = torch.randn(B, H_kv, N, d, generator=g, dtype=torch.float64, requires_grad=True)
    v = torch.randn(B, H_kv, N, d, generator=g, dtype=torch.float64, requires_grad=True)
    do = torch.randn(B, H, N, d, generator=g, dtype=torch.float64)
    rep = H // H_kv
    ref = F.scaled_dot_product_attention(q, k.repeat_interleave(rep, 1), v.repeat_interleave(rep, 1),
                                         is_causal=causal)
    ref.backward(do)
    o, lse = oracle.forward(q.detach().numpy(), k.detach().numpy(), v.detach().numpy(), None, causal)
    assert np.max(np.abs(o - ref.detach().numpy())) < 1e-12
    # logsumexp cross-check against torch.logsumexp of the masked scores
    s = (q @ k.repeat_interleave(rep, 1).transpose(-1, -2)).detach() / math.sqrt(d)
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(s, -1).numpy())) < 1e-12
    dq, dk, dv = oracle.backward(q.detach().numpy(), k.detach().numpy(), v.detach().numpy(),
                                 do.numpy(), None, causal)
    assert np.max(np.abs(dq - q.grad.numpy())) < 1e-11
    assert np.max(np.abs(dk - k.grad.numpy())) < 1e-11
    assert np.max(np.abs(dv - v.grad.numpy())) < 1e-11


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 8, 2, 1, 97, 32), (3, 4, 4, 5, 40, 16), (1, 6, 2, 7, 7, 8)])
def test_kvcache_matches_torch_sdpa_fp64(shape, causal):
    """Library cross-check of the KV-cache forward: torch's CPU SDPA in float64 with a
    boolean mask built here (query i of N_q sees keys j <= len - N_q + i)."""
    B, H, H_kv, n_q, n_kv, d = shape
    g = torch.Generator().manual_seed(sum(shape) + 7 * causal)
    q = torch.randn(B, H, n_q, d, generator=g, dtype=torch.float64)
    k = torch.randn(B, H_kv, n_kv, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, H_kv, n_kv, d, generator=g, dtype=torch.float64)
    lens = torch.randint(n_q, n_kv + 1, (B,), generator=g).tolist()
    lens[0] = n_kv
    o, lse = oracle.forward_kvcache(q.numpy(), k.numpy(), v.numpy(), lens, None, causal)
    rep = H // H_kv
    for b, n in enumerate(lens):
        kk = k[b:b + 1, :, :n].repeat_interleave(rep, 1)
        vv = v[b:b + 1, :, :n].repeat_interleave(rep, 1)
        mask = torch.ones(n_q, n, dtype=torch.bool)
        if causal:
            mask = mask.tril(diagonal=n - n_q)
        ref = F.scaled_dot_product_attention(q[b:b + 1], kk, vv, attn_mask=mask)
        assert np.max(np.abs(o[b] - ref[0].numpy())) < 1e-12
        s = (q[b:b + 1] @ kk.transpose(-1, -2)) / math.sqrt(d)
        s = s.masked_fill(~mask, float("-inf"))
        assert np.max(np.abs(lse[b] - torch.logsumexp(s, -1)[0].numpy())) < 1e-12


@pytest.mark.parametrize("case", [(2, 8, 2, 70, 16, 20, True), (3, 4, 4, 33, 8, None, True),
                                  (2, 4, 2, 50, 32, None, False), (1, 2, 1, 64, 8, 0, True)])
def test_masked_matches_torch_sdpa_fp64(case):
    """Library cross-check of the padded / sliding-window forward: torch's CPU SDPA in
    float64 on each unpadded sequence with a band mask built here."""
    B, H, H_kv, N, d, window, causal = case
    g = torch.Generator().manual_seed(N + d + (window or 0))
    q = torch.randn(B, H, N, d, generator=g, dtype=torch.float64)
    k = torch.randn(B, H_kv, N, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, H_kv, N, d, generator=g, dtype=torch.float64)
    lens = torch.randint(1, N + 1, (B,), generator=g).tolist()
    lens[0] = N
    o, lse = oracle.forward_masked(q.numpy(), k.numpy(), v.numpy(), lens, window, None, causal)
    rep = H // H_kv
    for b, n in enumerate(lens):
        kk = k[b:b + 1, :, :n].repeat_interleave(rep, 1)
        vv = v[b:b + 1, :, :n].repeat_interleave(rep, 1)
        i = torch.arange(n)[:, None]
        j = torch.arange(n)[None, :]
        mask = torch.ones(n, n, dtype=torch.bool)
        if causal:
            mask &= j <= i
        if window is not None:
            mask &= j >= i - window
        ref = F.scaled_dot_product_attention(q[b:b + 1, :, :n], kk, vv, attn_mask=mask)
        assert np.max(np.abs(o[b, :, :n] - ref[0].numpy())) < 1e-12
        assert np.all(o[b, :, n:] == 0) and np.all(lse[b, :, n:] == -np.inf)
        s = (q[b:b + 1, :, :n] @ kk.transpose(-1, -2)) / math.sqrt(d)
        s = s.masked_fill(~mask, float("-inf"))
        assert np.max(np.abs(lse[b, :, :n] - torch.logsumexp(s, -1)[0].numpy())) < 1e-12


@pytest.mark.parametrize("case", [(2, 4, 2, 40, 8, 9, True), (2, 4, 4, 33, 8, None, True),
                                  (2, 2, 1, 30, 16, None, False)])
def test_masked_backward_matches_torch_autograd_fp64(case):
    """Library cross-check of backward_masked: torch autograd through CPU SDPA in
    float64 on each unpadded sequence with the band mask."""
    B, H, H_kv, N, d, window, causal = case
    g = torch.Generator().manual_seed(3 * N + d)
    q = torch.randn(B, H, N, d, generator=g, dtype=torch.float64)
    k = torch.randn(B, H_kv, N, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, H_kv, N, d, generator=g, dtype=torch.float64)
    do = torch.randn(B, H, N, d, generator=g, dtype=torch.float64)
    lens = [N, N // 2 + 1]
    dq, dk, dv = oracle.backward_masked(q.numpy(), k.numpy(), v.numpy(), do.numpy(), lens, window, None, causal)
    rep = H // H_kv
    for b, n in enumerate(lens):
        qq = q[b:b + 1, :, :n].clone().requires_grad_(True)
        kk = k[b:b + 1, :, :n].clone().requires_grad_(True)
        vv = v[b:b + 1, :, :n].clone().requires_grad_(True)
        i, j = torch.arange(n)[:, None], torch.arange(n)[None, :]
        mask = torch.ones(n, n, dtype=torch.bool)
        if causal:
            mask &= j <= i
        if window is not None:
            mask &= j >= i - window
        out = F.scaled_dot_product_attention(qq, kk.repeat_interleave(rep, 1), vv.repeat_interleave(rep, 1),
                                             attn_mask=mask)
        out.backward(do[b:b + 1, :, :n])
        assert np.max(np.abs(dq[b, :, :n] - qq.grad[0].numpy())) < 1e-11
        assert np.max(np.abs(dk[b, :, :n] - kk.grad[0].numpy())) < 1e-11
        assert np.max(np.abs(dv[b, :, :n] - vv.grad[0].numpy())) < 1e-11
        assert np.all(dq[b, :, n:] == 0) and np.all(dk[b, :, n:] == 0) and np.all(dv[b, :, n:] == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_matches_torch_sdpa_fp64(causal):
    """Library cross-check of the block-sparse forward and backward: torch's CPU
    SDPA and autograd in float64 with the block mask expanded here."""
    B, H, H_kv, N, d, blk = 2, 4, 2, 40, 8, 8
    g = torch.Generator().manual_seed(40 + causal)
    q = torch.randn(B, H, N, d, generator=g, dtype=torch.float64, requires_grad=True)
    k = torch.randn(B, H_kv, N, d, generator=g, dtype=torch.float64, requires_grad=True)
    v = torch.randn(B, H_kv, N, d, generator=g, dtype=torch.float64, requires_grad=True)
    do = torch.randn(B, H, N, d, generator=g, dtype=torch.float64)
    nb = N // blk
    bm = torch.randint(0, 2, (H, nb, nb), generator=g)
    bm[:, torch.arange(nb), torch.arange(nb)] = 1          # every row sees its own block
    mask = bm.repeat_interleave(blk, 1).repeat_interleave(blk, 2).bool()
    if causal:
        mask &= torch.ones(N, N, dtype=torch.bool).tril()
    rep = H // H_kv
    ref = F.scaled_dot_product_attention(q, k.repeat_interleave(rep, 1), v.repeat_interleave(rep, 1),
                                         attn_mask=mask[None])
    ref.backward(do)
    o, lse = oracle.forward_blocksparse(q.detach().numpy(), k.detach().numpy(), v.detach().numpy(),
                                        bm.numpy(), blk, None, causal)
    assert np.max(np.abs(o - ref.detach().numpy())) < 1e-12
    s = (q @ k.repeat_interleave(rep, 1).transpose(-1, -2)).detach() / math.sqrt(d)
    assert np.max(np.abs(lse - torch.logsumexp(s.masked_fill(~mask[None], float("-inf")), -1).numpy())) < 1e-12
    dq, dk, dv = oracle.backward_blocksparse(q.detach().numpy(), k.detach().numpy(), v.detach().numpy(),
                                             do.numpy(), bm.numpy(), blk, None, causal)
    assert np.max(np.abs(dq - q.grad.numpy())) < 1e-11
    assert np.max(np.abs(dk - k.grad.numpy())) < 1e-11
    assert np.max(np.abs(dv - v.grad.numpy())) < 1e-11


def _page_fp32_errors():
    path = os.path.join(os.path.dirname(__file__), "golden", "cpu_sdpa_fp32_error.txt")
    out = {}
    with open(path) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                n, e = line.split()
                out[int(n)] = float(e)
    return out


def test_fp32_rounding_level_matches_pages():
    """torch's fused CPU fp32 attention lands within the pages' fp32 error level of the oracle.

    The pages measured ~1e-6 between two exact fp32 CPU paths at B=1, H=8,
    N=1024, d=64, causal.  An fp32 fused implementation must sit at that level
    against the fp64 oracle; an oracle with a wrong term would be far off.
    """
    errs = _page_fp32_errors()
    N = 1024
    g = torch.Generator().manual_seed(1)
    q, k, v = (torch.randn(1, 8, N, 64, generator=g) for _ in range(3))
    got = F.scaled_dot_product_attention(q, k, v, is_causal=True)
    o, _ = oracle.forward(q.double().numpy(), k.double().numpy(), v.double().numpy(), None, True)
    err = np.max(np.abs(got.double().numpy() - o))
    assert err < 10 * errs[N], err


# ------------------------------------------------------------ mutation test ---

MUTANTS = {
    "no_scale": ("s = scale * (q_rows @ k.T)", "s = (q_rows @ k.T)"),
    "mask_excludes_diagonal": ("cols <= rows", "cols < rows"),
    "mask_one_too_many": ("cols <= rows", "cols <= rows + 1"),
    "lse_missing_log_l": ("lse = (m + np.log(l))[:, 0]", "lse = m[:, 0]"),
    "lse_log2": ("lse = (m + np.log(l))[:, 0]", "lse = (m + np.log2(l))[:, 0]"),
    "softmax_no_normalise": ("p = e / l", "p = e"),
    "gqa_modulo_map": ("return h // (H // H_kv)", "return h % H_kv"),
    "pv_uses_k": ("o[r0:r0 + ROW_BLOCK] = p @ v", "o[r0:r0 + ROW_BLOCK] = p @ k[:, :v.shape[1]]"),
    "ds_missing_rowdot": ("ds = p * (dp - row_dot)", "ds = p * dp"),
    "ds_sign": ("ds = p * (dp - row_dot)", "ds = p * (row_dot - dp)"),
    "dq_missing_scale": ("dq[rid] = scale * (ds @ k)", "dq[rid] = (ds @ k)"),
    "dq_uses_v": ("dq[rid] = scale * (ds @ k)", "dq[rid] = scale * (ds @ v)"),
    "dk_missing_scale": ("dk += scale * (ds.T @ q[rid])", "dk += (ds.T @ q[rid])"),
    "dv_uses_ds": ("dv += p.T @ do[rid]", "dv += ds.T @ do[rid]"),
    "gqa_grads_overwrite": ("dk[b, kv] += gk", "dk[b, kv] = gk"),
    "kvcache_top_left": ("pos = n - n_q + np.arange(n_q)", "pos = np.arange(n_q)"),
    "kvcache_off_by_one": ("pos = n - n_q + np.arange(n_q)", "pos = n - n_q + 1 + np.arange(n_q)"),
    "kvcache_whole_cache": ("s = scores_rows(q[b, h, rows], k[b, kv, :n],", "s = scores_rows(q[b, h, rows], k[b, kv],"),
    "kvcache_empty_rows_nan": ("rows = np.flatnonzero(n_seen > 0)", "rows = np.arange(n_q)"),
    "window_off_by_one": ("s = np.where(cols >= rows[:, None] - window, s, -np.inf)",
                          "s = np.where(cols > rows[:, None] - window, s, -np.inf)"),
    "window_ignored": ("s = np.where(cols >= rows[:, None] - window, s, -np.inf)", "s = s"),
    "padding_keys_kept": ("keys, vals = k[b, kv, :n], v[b, kv, :n]", "keys, vals = k[b, kv], v[b, kv]"),
    "masked_bwd_no_window": ("                s = np.where(np.arange(n)[None, :] >= rows[:, None] - window, s, -np.inf)",
                             "                s = s"),
    "masked_bwd_ds_sign": ("            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))",
                           "            ds = p * (np.sum(p * dp, axis=1, keepdims=True) - dp)"),
    "blocksparse_transposed": ("    vis = bm[:, idx][:, :, idx]", "    vis = bm[:, idx][:, :, idx].transpose(0, 2, 1)"),
    "blocksparse_no_causal": ("        vis = vis & (np.arange(n)[None, :] <= np.arange(n)[:, None])[None]", "        vis = vis"),
    "dense_mask_empty_rows_nan": ("            rows = np.flatnonzero(vis[h].any(axis=1))\n            if rows.size == 0:\n                continue\n            s = np.where(vis[h][rows], scale * (q[b, h, rows] @ k[b, kv].T), -np.inf)\n            p, lse[b, h, rows]",
                                  "            rows = np.arange(N)\n            if rows.size == 0:\n                continue\n            s = np.where(vis[h][rows], scale * (q[b, h, rows] @ k[b, kv].T), -np.inf)\n            p, lse[b, h, rows]"),
    "kvcache_v_whole_cache": ("o[b, h, rows] = p @ v[b, kv, :n]", "o[b, h, rows] = p @ v[b, kv, :p.shape[1]][::-1]"),
}


def _mutant_module(old, new):
    src = open(oa.__file__).read()
    assert old in src, f"mutation anchor missing: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    mod = _mutant_module(*MUTANTS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
