"""GPU parity of the block-sparse forward and backward (fa_fwd_blocksparse,
fa_bwd_blocksparse) against the fp64 oracle.

Seeded 128 x 128 block masks of several densities, with some query blocks
switched off entirely (their rows must come back exactly O = 0, LSE = -inf)
and a key block no query sees (zero dK, dV), causal and not, d = 64 and 128,
ragged last blocks, a large grid; all blocks on must give what fa_fwd gives
(bit for bit where the same kernel serves both); the 64K block-sparse workload is checked on sampled rows (forward)
and on sampled key blocks with the query rows that see them (backward).
Tolerances: 1e-2 on O and LSE; 2e-2 plus 2^-8 of the reference magnitude on
gradients (2^-8: the relative rounding of the bf16 result).
"""
import numpy as np
import pytest
import torch

import exact_tiled_attention_amd as fa
import blocksparse_sub as bsub
import oracle
import synthetic as syn
from oracle.tolerance import GRAD_ABS, grad_excess

pytestmark = pytest.mark.gpu

TOL = 1e-2
GRAD_TOL = GRAD_ABS   # per element: 2e-2 + 2^-8 |ref_i| (R18/R10b, oracle.tolerance)
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


def _mask(H, N, density, seed, off_blocks=True):
    nb = (N + 127) // 128
    g = torch.Generator().manual_seed(seed)
    m = (torch.rand(H, nb, nb, generator=g) < density).to(torch.uint8)
    if off_blocks:
        m[0, nb // 2, :] = 0                 # a query block that sees nothing
        m[-1, 0, :] = 0
        m[:, :, nb // 3] = 0                 # a key block no query sees
    return m


def _compare(o, lse, o_ref, lse_ref, what=""):
    empty = ~np.isfinite(lse_ref)
    assert np.array_equal(~np.isfinite(lse), empty), what
    assert np.all(o[empty] == 0.0), what
    eo = float(np.max(np.abs(o - o_ref)))
    el = float(np.max(np.abs(lse[~empty] - lse_ref[~empty]), initial=0.0))
    assert eo <= TOL and el <= TOL, (what, eo, el)


CASES = [
    # B, H, H_kv, N, d, density, causal
    (2, 4, 2, 300, 64, 0.5, True),
    (2, 4, 2, 300, 64, 0.5, False),
    (1, 4, 1, 1000, 64, 0.2, True),
    (2, 4, 2, 700, 128, 0.4, True),
    (2, 4, 4, 513, 128, 0.3, False),
    (2, 132, 4, 300, 128, 0.5, True),        # more items than CUs: the looping grid
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[3]}x{c[4]}-p{c[5]}-{'c' if c[6] else 'nc'}")
def test_blocksparse_forward_small(case):
    B, H, H_kv, N, d, density, causal = case
    _say(f"blocksparse {case}")
    q, k, v, _ = syn.draw(B, H, H_kv, N, d, 1.0, N + d)
    x = syn.pack_inputs(q, k, v, None, "bf16")
    bm = _mask(H, N, density, N + 3 * d)
    o, lse = fa.fa_fwd_blocksparse(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), bm.to(DEV), causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward_blocksparse(x["q_64"], x["k_64"], x["v_64"], bm.numpy(), 128, x["scale"],
                                                causal)
    _compare(o.double().cpu().numpy(), lse.double().cpu().numpy(), o_ref, lse_ref, what=case)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_blocksparse_all_on_matches_fa_fwd(d, causal):
    w = syn.Workload("m", 2, 4, 2, 333, d, "bf16", causal, 1.0, 60 + d)
    x = syn.make_inputs(w)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    o1, l1 = fa.fa_fwd(q, k, v, causal=causal)
    o2, l2 = fa.fa_fwd_blocksparse(q, k, v, torch.ones(4, 3, 3, dtype=torch.uint8, device=DEV), causal=causal)
    torch.cuda.synchronize()
    # another tiling (short causal d=64 grids split each row's keys over two
    # waves in the plain forward): the same values up to rounding
    assert float((o1.float() - o2.float()).abs().max()) <= TOL
    assert float((l1 - l2).abs().max()) <= TOL


BWD_CASES = [
    (2, 4, 2, 300, 64, 0.5, True),
    (2, 4, 2, 300, 128, 0.5, False),
    (1, 4, 4, 400, 128, 0.3, True),
    (2, 8, 2, 257, 64, 0.4, False),
    (1, 8, 2, 3000, 128, 0.3, True),         # a group's mask column spans two 64-bit words
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: f"{c[3]}x{c[4]}-p{c[5]}-{'c' if c[6] else 'nc'}")
def test_blocksparse_backward_small(case):
    B, H, H_kv, N, d, density, causal = case
    _say(f"blocksparse backward {case}")
    q, k, v, do = syn.draw(B, H, H_kv, N, d, 1.0, 5 * N + d, with_do=True)
    x = syn.pack_inputs(q, k, v, do, "bf16")
    bm = _mask(H, N, density, 7 * N + d)
    qd, kd, vd, dod, bmd = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), x["do"].to(DEV), bm.to(DEV)
    o, lse = fa.fa_fwd_blocksparse(qd, kd, vd, bmd, causal=causal)
    dq, dk, dv = fa.fa_bwd_blocksparse(qd, kd, vd, o, lse, dod, bmd, causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward_blocksparse(x["q_64"], x["k_64"], x["v_64"], x["do_64"], bm.numpy(), 128,
                                             x["scale"], causal)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g64 = got.double().cpu().numpy()
        excess = grad_excess(g64, ref)
        assert excess <= GRAD_TOL, (case, name, excess)


@pytest.mark.parametrize("name", sorted(syn.BLOCKSPARSE_WORKLOADS))
def test_blocksparse_full_size_sampled(name):
    """The 64K block-sparse workload in the launch the bench times; the oracle
    recomputes sampled rows one at a time."""
    w = syn.BLOCKSPARSE_WORKLOADS[name]
    _say(f"blocksparse full size {name}")
    x = syn.make_blocksparse_inputs(w)
    bm = x["block_mask"]
    o, lse = fa.fa_fwd_blocksparse(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), bm.to(DEV), causal=w.causal)
    torch.cuda.synchronize()
    o, lse = o.double().cpu().numpy(), lse.double().cpu().numpy()
    g = w.H // w.H_kv
    for b, h in [(0, 0), (0, w.H - 1), (0, 7 % w.H)]:
        rows = syn.rand_rows(w.N, 16, seed=h + 1)
        o_ref, lse_ref = oracle.forward_blocksparse_rows(x["q_64"][b, h], x["k_64"][b, h // g], x["v_64"][b, h // g],
                                                         bm[h].numpy(), 128, x["scale"], w.causal, rows)
        _compare(o[b, h, rows], lse[b, h, rows], o_ref, lse_ref, what=(name, h))



@pytest.mark.parametrize("name", sorted(syn.BLOCKSPARSE_WORKLOADS))
def test_blocksparse_full_size_backward_sampled(name):
    """Backward in the launch the bench times (the 64K shape), with a sparse
    causal mask so that the oracle's work stays small: for sampled key blocks
    of the last K/V group, the oracle solves the sub-problem of the query
    blocks that see the key block and the key blocks those rows see, which
    gives those rows' dQ and the key block's dK, dV exactly."""
    w = syn.BLOCKSPARSE_WORKLOADS[name]
    assert w.causal
    _say(f"blocksparse full-size backward {name}")
    q, k, v, do = syn.draw(w.B, w.H, w.H_kv, w.N, w.d, w.amp, w.seed + 5, with_do=True)
    x = syn.pack_inputs(q, k, v, do, "bf16")
    del q, k, v, do
    nb = (w.N + 127) // 128
    bm = bsub.sparse_causal_mask(w.H, nb, 2, w.seed + 6)
    qd, kd, vd, dod, bmd = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), x["do"].to(DEV), bm.to(DEV)
    o, lse = fa.fa_fwd_blocksparse(qd, kd, vd, bmd, causal=True)
    dq, dk, dv = fa.fa_bwd_blocksparse(qd, kd, vd, o, lse, dod, bmd, causal=True)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    b, kv = w.B - 1, w.H_kv - 1

    def check(what, got, ref):
        excess = grad_excess(got, ref)
        assert excess <= GRAD_TOL, (what, excess)

    for kb in (0, 1, nb // 2, nb - 1):
        _say(f"  key block {kb}")
        dqs, dk_ref, dv_ref = bsub.key_block_grads(x["q_64"][b], x["k_64"][b], x["v_64"][b], x["do_64"][b],
                                                   bm.numpy() != 0, kv, kb, x["scale"])
        for h, rows, gq in dqs:
            check(("dq", kb, h), dq[b, h, rows], gq)
        keys = bsub.span([kb], w.N)
        check(("dk", kb), dk[b, kv, keys], dk_ref)
        check(("dv", kb), dv[b, kv, keys], dv_ref)
