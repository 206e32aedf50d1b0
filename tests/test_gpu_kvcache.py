"""GPU parity of the KV-cache forward (decode) against the fp64 oracle.

Small problems are compared in full: ragged cache lengths (including an
empty cache and caches shorter than N_q), one and two 32-row query groups,
every head dim, a long cache split into many chunks.  The decode workloads
(8 sequences, 32 query heads on 8 K/V heads, d = 128, 32K-token caches, with
full and with mixed lengths) are compared on sampled (batch, head) rows.
Tolerances are the bf16 ones: max abs error <= 1e-2 on O and on LSE; rows
that see no key must come back as exactly O = 0, LSE = -inf.
"""
import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_amd as fa
import oracle
import synthetic as syn

pytestmark = pytest.mark.gpu

TOL = 1e-2
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


def _run(x, causal):
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    kv_len = x["kv_len"].to(DEV) if x["kv_len"] is not None else None
    o, lse = fa.fa_fwd_kvcache(q, k, v, kv_len, causal=causal, scale=x["scale"])
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def _compare(o, lse, o_ref, lse_ref, tol_o=TOL, tol_l=TOL, what=""):
    empty = ~np.isfinite(lse_ref)
    assert np.array_equal(~np.isfinite(lse), empty), what
    assert np.all(o[empty] == 0.0), what
    eo = float(np.max(np.abs(o - o_ref)))
    el = float(np.max(np.abs(lse[~empty] - lse_ref[~empty]), initial=0.0))
    assert eo <= tol_o and el <= tol_l, (what, eo, el)


def _inputs(B, H, H_kv, N_q, N_kv, d, lens, seed, amp=1.0):
    q, k, v = syn.draw_kvcache(B, H, H_kv, N_q, N_kv, d, amp, seed)
    x = syn.pack_inputs(q, k, v, None, "bf16")
    x["kv_len"] = None if lens is None else torch.tensor(lens, dtype=torch.int32)
    x["lens"] = [N_kv] * B if lens is None else list(lens)
    return x


CASES = [
    # B, H, H_kv, N_q, N_kv, d, cache lengths (None: all N_kv)
    (2, 8, 2, 1, 1000, 128, None),
    (3, 4, 4, 3, 777, 64, [777, 5, 300]),
    (1, 16, 2, 4, 513, 256, None),          # 32 query rows per group exactly
    (2, 32, 2, 3, 400, 128, [400, 2]),      # 48 rows: two row groups; a cache shorter than N_q
    (2, 8, 8, 1, 1, 64, None),              # a single key
    (3, 8, 4, 2, 300, 128, [0, 1, 300]),    # an empty cache and a one-row cache
    (1, 4, 1, 1, 20000, 128, None),         # one group, a long cache in many chunks
    (2, 8, 1, 5, 129, 64, [129, 33]),       # 40 rows; ragged tail tiles
    (1, 2, 2, 7, 7, 256, None),             # N_q = N_kv: ordinary causal attention
    (300, 4, 4, 1, 40, 64, None),           # more units than resident waves
    (40, 8, 2, 2, 700, 128, "ragged"),      # a seeded mix of lengths, including 0
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(str(v) for v in c[:6]))
def test_kvcache_small(case, causal):
    B, H, H_kv, N_q, N_kv, d, lens = case
    _say(f"kvcache {case} causal={causal}")
    if lens == "ragged":
        g = torch.Generator().manual_seed(B + N_kv)
        lens = torch.randint(0, N_kv + 1, (B,), generator=g).tolist()
        lens[:3] = [0, N_kv, 1]
    x = _inputs(B, H, H_kv, N_q, N_kv, d, lens, seed=sum(case[:6]) + causal)
    o, lse = _run(x, causal)
    o_ref, lse_ref = oracle.forward_kvcache(x["q_64"], x["k_64"], x["v_64"], x["lens"], x["scale"], causal)
    _compare(o, lse, o_ref, lse_ref, what=(case, causal))


def test_kvcache_matches_forward_on_square_problem():
    """N_q = N_kv with full caches is ordinary attention: both entry points agree
    with the oracle, and with each other to within their rounding."""
    w = syn.Workload("sq", 1, 8, 2, 200, 128, "bf16", True, 1.0, 31)
    x = syn.make_inputs(w)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    o1, l1 = fa.fa_fwd(q, k, v, causal=True)
    o2, l2 = fa.fa_fwd_kvcache(q, k, v, None, causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(x["q_64"], x["k_64"], x["v_64"], x["scale"], True)
    for o, l in ((o1, l1), (o2, l2)):
        _compare(o.double().cpu().numpy(), l.double().cpu().numpy(), o_ref, lse_ref)


def test_kvcache_lengths_are_clamped():
    """kv_len values outside [0, N_kv] act as 0 and N_kv."""
    x = _inputs(2, 4, 2, 2, 150, 64, [-5, 100000], seed=3)
    o, lse = _run(x, True)
    o_ref, lse_ref = oracle.forward_kvcache(x["q_64"], x["k_64"], x["v_64"], [0, 150], x["scale"], True)
    _compare(o, lse, o_ref, lse_ref)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_kvcache_running_max_moves(causal):
    """Key blocks of very different norms make the running max move inside a
    chunk and the chunk maxima differ widely, so both the in-chunk rescale and
    the merge of chunks are exercised.  Bounds as for the prefill stress
    test: 3 * 2^-8 * max|V| on O and 2^-8 on LSE (P rounded to bf16)."""
    B, H, H_kv, N_q, N_kv, d = 2, 8, 2, 2, 5000, 128
    q, k, v = syn.draw_kvcache(B, H, H_kv, N_q, N_kv, d, 1.0, 777)
    g = torch.Generator().manual_seed(778)
    f = torch.tensor([0.25, 1.0, 3.0, 0.5, 8.0, 0.1, 5.0, 2.0])
    idx = torch.randint(0, len(f), ((N_kv + 47) // 48,), generator=g)
    k = k * f[idx].repeat_interleave(48)[:N_kv][None, None, :, None]
    x = syn.pack_inputs(q, k, v, None, "bf16")
    x["kv_len"] = torch.tensor([5000, 3001], dtype=torch.int32)
    x["lens"] = [5000, 3001]
    o, lse = _run(x, causal)
    o_ref, lse_ref = oracle.forward_kvcache(x["q_64"], x["k_64"], x["v_64"], x["lens"], x["scale"], causal)
    vmax = float(np.max(np.abs(x["v_64"])))
    _compare(o, lse, o_ref, lse_ref, tol_o=max(TOL, 3 * 2.0 ** -8 * vmax), tol_l=max(TOL, 2.0 ** -8))


@pytest.mark.parametrize("name", sorted(syn.KV_WORKLOADS))
def test_kvcache_full_size_sampled(name):
    """The decode workloads at full size, in the launch the bench times; the
    oracle recomputes sampled (batch, head) pairs one at a time."""
    w = syn.KV_WORKLOADS[name]
    _say(f"kvcache full size {name}")
    x = syn.make_kvcache_inputs(w)
    o, lse = _run(x, w.causal)
    g = w.H // w.H_kv
    pairs = [(0, 0), (w.B - 1, w.H - 1), (3 % w.B, 17 % w.H), (5 % w.B, 6 % w.H), (1 % w.B, 31 % w.H)]
    for b, h in pairs:
        kv = h // g
        o_ref, lse_ref = oracle.forward_kvcache(x["q_64"][b:b + 1, h:h + 1], x["k_64"][b:b + 1, kv:kv + 1],
                                                x["v_64"][b:b + 1, kv:kv + 1], [x["lens"][b]],
                                                x["scale"], w.causal)
        _compare(o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], o_ref, lse_ref, what=(name, b, h))
