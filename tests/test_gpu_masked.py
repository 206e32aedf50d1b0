"""GPU parity of the forward with a padding mask and/or a causal sliding
window (fa_fwd_masked) against the fp64 oracle.

Small problems are compared in full for every bf16 head dim, causal and not,
with windows from 0 keys to wider than the sequence, ragged valid lengths
(including 0 and 1) and grids large enough for the looping (persistent)
kernel; the two masked prefill workloads are compared at full size on
sampled rows.  Padding rows must come back exactly as O = 0, LSE = -inf.
Tolerance: the bf16 one, max abs error <= 1e-2 on O and LSE.
"""
import numpy as np
import pytest
import torch

import exact_tiled_attention_amd as fa
import oracle
import synthetic as syn
from oracle.tolerance import GRAD_ABS, grad_excess

pytestmark = pytest.mark.gpu

TOL = 1e-2
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


def _run(x, window, causal):
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    sl = x["seqlens"].to(DEV) if x["seqlens"] is not None else None
    o, lse = fa.fa_fwd_masked(q, k, v, sl, window, causal=causal, scale=x["scale"])
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def _compare(o, lse, o_ref, lse_ref, what="", tol_o=TOL):
    empty = ~np.isfinite(lse_ref)
    assert np.array_equal(~np.isfinite(lse), empty), what
    assert np.all(o[empty] == 0.0), what
    eo = float(np.max(np.abs(o - o_ref)))
    el = float(np.max(np.abs(lse[~empty] - lse_ref[~empty]), initial=0.0))
    assert eo <= tol_o and el <= TOL, (what, eo, el)


def _tol_o(window, v64):
    """The stated 1e-2 assumes rows that see many keys, where the bf16 rounding
    of P averages out.  When every row sees few keys (a window under 64) the
    bound follows from the arithmetic instead: with P rounded to bf16
    (u = 2^-8), |O~ - O| <= 3 u max|V| (the same bound as the stress tests)."""
    if window is not None and window < 64:
        return max(TOL, 3 * 2.0 ** -8 * float(np.max(np.abs(v64))))
    return TOL


def _inputs(B, H, H_kv, N, d, lens, seed):
    q, k, v, _ = syn.draw(B, H, H_kv, N, d, 1.0, seed)
    x = syn.pack_inputs(q, k, v, None, "bf16")
    x["seqlens"] = None if lens is None else torch.tensor(lens, dtype=torch.int32)
    x["lens"] = [N] * B if lens is None else list(lens)
    return x


CASES = [
    # B, H, H_kv, N, d, valid lengths (None: all N), window (None: none), causal
    (2, 4, 2, 200, 64, None, 31, True),
    (2, 4, 2, 200, 64, [200, 77], None, True),
    (2, 4, 2, 300, 64, [300, 1], None, False),
    (1, 4, 2, 1000, 64, None, 1000, True),       # window wider than the sequence
    (2, 4, 2, 700, 128, [700, 333], 100, True),
    (1, 8, 2, 513, 128, None, 0, True),          # each row sees only itself
    (2, 4, 4, 600, 128, [0, 600], 257, True),    # an empty sequence
    (2, 4, 2, 400, 128, [400, 150], None, False),
    (2, 4, 4, 300, 256, [300, 129], 64, True),
    (1, 4, 4, 257, 256, None, 1, True),
    (2, 4, 4, 300, 256, [300, 3], None, False),
    (2, 132, 4, 300, 128, [300, 211], 50, True),  # more items than CUs: the looping grid
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[3]}x{c[4]}-w{c[6]}-{'c' if c[7] else 'nc'}")
def test_masked_small(case):
    B, H, H_kv, N, d, lens, window, causal = case
    _say(f"masked {case}")
    x = _inputs(B, H, H_kv, N, d, lens, seed=N + d + (window or 0))
    o, lse = _run(x, window, causal)
    o_ref, lse_ref = oracle.forward_masked(x["q_64"], x["k_64"], x["v_64"], x["lens"], window, x["scale"], causal)
    _compare(o, lse, o_ref, lse_ref, what=case, tol_o=_tol_o(window, x["v_64"]))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_masked_without_mask_matches_fa_fwd(d, causal):
    """Full-length sequences and no window through the masked kernels give
    what the plain forward gives: bit for bit where both run the same
    schedule.  For short causal d=64 grids the plain forward splits each
    row's keys over two waves and merges the halves (another tiling, whose
    waves round P to bf16 against their own running maxima), so there the two
    agree up to rounding, within the stated tolerance."""
    w = syn.Workload("m", 2, 4, 2, 333, d, "bf16", causal, 1.0, 40 + d)
    x = syn.make_inputs(w)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    o1, l1 = fa.fa_fwd(q, k, v, causal=causal)
    o2, l2 = fa.fa_fwd_masked(q, k, v, torch.full((2,), 333, dtype=torch.int32, device=DEV), None, causal=causal)
    torch.cuda.synchronize()
    if d == 64 and causal:
        assert float((o1.float() - o2.float()).abs().max()) <= TOL
        assert float((l1 - l2).abs().max()) <= TOL
    else:
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_masked_unsupported_dtypes_raise():
    for dt, d in ((torch.float32, 64), (torch.float8_e4m3fn, 128)):
        q = torch.zeros(1, 1, 16, d, device=DEV).to(dt)
        with pytest.raises(fa.FaError):
            fa.fa_fwd_masked(q, q, q, None, 4)
    q = torch.zeros(1, 1, 16, 64, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(fa.FaError):
        fa.fa_fwd_masked(q, q, q, None, 4, causal=False)   # a window is causal


@pytest.mark.parametrize("name", sorted(syn.MASKED_WORKLOADS))
def test_masked_full_size_sampled(name):
    """The masked prefill workloads at full size, in the launch the bench
    times; the oracle recomputes sampled rows one at a time."""
    w = syn.MASKED_WORKLOADS[name]
    _say(f"masked full size {name}")
    x = syn.make_masked_inputs(w)
    o, lse = _run(x, w.window, w.causal)
    g = w.H // w.H_kv
    for b, h in [(0, 0), (w.B - 1, w.H - 1), (2 % w.B, 13 % w.H), (5 % w.B, 30 % w.H)]:
        kv = h // g
        n = x["lens"][b]
        rows = syn.rand_rows(w.N, 24, seed=b * 100 + h)
        rows = sorted(set(rows + [max(0, n - 1), min(w.N - 1, n)]))
        o_ref, lse_ref = oracle.forward_masked_rows(x["q_64"][b, h], x["k_64"][b, kv], x["v_64"][b, kv], n,
                                                    w.window, x["scale"], w.causal, rows)
        _compare(o[b, h, rows], lse[b, h, rows], o_ref, lse_ref, what=(name, b, h))


GRAD_TOL = GRAD_ABS

BWD_CASES = [
    # B, H, H_kv, N, d, valid lengths, window, causal
    (2, 4, 2, 300, 64, [300, 129], None, True),
    (2, 4, 2, 300, 64, [300, 77], 100, True),
    (2, 4, 4, 200, 64, [200, 31], None, False),
    (2, 4, 2, 333, 128, [0, 333], 64, True),
    (2, 8, 2, 300, 128, [300, 170], None, False),
    (1, 4, 4, 400, 128, None, 200, True),
    (2, 4, 2, 300, 256, [300, 111], 70, True),
    (2, 4, 4, 200, 256, [200, 57], None, False),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: f"{c[3]}x{c[4]}-w{c[6]}-{'c' if c[7] else 'nc'}")
def test_masked_backward_small(case):
    """Gradients through the masked kernels against the oracle's masked
    backward; padding gradient rows must be exactly zero.  The bound is the
    per-element one of R18/R10b (oracle.tolerance): every element i within
    2e-2 + 2^-8 |ref_i|, as for the plain and block-sparse backward."""
    B, H, H_kv, N, d, lens, window, causal = case
    _say(f"masked backward {case}")
    q, k, v, do = syn.draw(B, H, H_kv, N, d, 1.0, N + 7 * d + (window or 0), with_do=True)
    x = syn.pack_inputs(q, k, v, do, "bf16")
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    qd, kd, vd, dod = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd_masked(qd, kd, vd, sl, window, causal=causal)
    dq, dk, dv = fa.fa_bwd_masked(qd, kd, vd, o, lse, dod, sl, window, causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward_masked(x["q_64"], x["k_64"], x["v_64"], x["do_64"], lens, window, x["scale"],
                                        causal)
    lens_ = [N] * B if lens is None else lens
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g64 = got.double().cpu().numpy()
        excess = grad_excess(g64, ref)
        assert excess <= GRAD_TOL, (case, name, excess)
        for b, n in enumerate(lens_):
            assert np.all(g64[b, :, n:] == 0.0), (case, name, b)
