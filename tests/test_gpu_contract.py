"""GPU checks of the library's contract beyond parity: bitwise repeatability
of the backward, no device allocation at run time (no N x N buffer), fp8
block scales of zero, the binding's rejection of wrong tensors, and the
autograd entry point.
"""
import numpy as np
import pytest
import torch

import exact_tiled_attention_amd as fa
import oracle
import synthetic as syn
from oracle.tolerance import TOL, max_abs_err

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("d,H,H_kv,causal", [(64, 4, 4, True), (128, 8, 2, True), (128, 4, 4, False),
                                            (256, 2, 2, True)])
def test_backward_is_deterministic(d, H, H_kv, causal):
    """The backward uses no atomics (dK/dV and dQ each have one owner), so two
    calls on the same inputs give bitwise-equal gradients."""
    _say(f"bwd determinism d={d} H={H}/{H_kv} causal={causal}")
    w = syn.Workload("det_b", 2, H, H_kv, 777, d, "bf16", causal, 1.0, 60 + d, backward=True)
    x = syn.make_inputs(w)
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd(q, k, v, causal=causal)
    g1 = fa.fa_bwd(q, k, v, o, lse, do, causal=causal)
    g2 = fa.fa_bwd(q, k, v, o, lse, do, causal=causal)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_no_device_memory_at_run_time():
    """The pages measure the memory FlashAttention saves by the growth of the
    peak footprint, which stays flat where the plain path grows with N^2.  Here:
    with outputs and workspace allocated by the caller, forward and backward at
    the training shape (B=2, H=16, N=16384, d=64: an fp32 score matrix per head
    would be 1 GiB, 32 GiB for all heads) leave the device's free memory and
    torch's allocator untouched."""
    w = syn.WORKLOADS["C4"]
    x = syn.make_inputs(w)
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, device=DEV, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.H_kv, w.N, w.d), device=DEV, dtype=torch.uint8)

    def run():
        fa.fa_fwd(q, k, v, causal=True, out=o, lse=lse)
        fa.fa_bwd(q, k, v, o, lse, do, causal=True, workspace=ws, dq=dq, dk=dk, dv=dv)

    run()                           # first use loads the code objects
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    peak = torch.cuda.max_memory_allocated()
    n2_bytes = w.B * w.H * w.N * w.N * 4
    _say(f"free memory {free0 / 2**20:.0f} -> {free1 / 2**20:.0f} MiB; torch peak delta "
         f"{(peak - alloc0) / 2**20:.1f} MiB; one fp32 N x N matrix per head would be "
         f"{n2_bytes / 2**30:.0f} GiB")
    assert peak == alloc0
    assert free1 >= free0 - (4 << 20)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_fp8_zero_block_scales(causal):
    """A block scale of 0 means the block's values are all 0 whatever its codes
    (as an amax/448 quantiser gives an all-zero block): a zero V block adds
    nothing to O but its keys still count in the softmax sum; a zero Q or K
    block gives scores of 0.  Checked against the oracle on the dequantised
    values (codes times scales)."""
    N, d = 600, 128
    q, k, v, _ = syn.draw(1, 2, 2, N, d, 1.0, 4711)
    x = syn.pack_inputs(q, k, v, None, "fp8")
    qs, ks, vs = x["q_scale"].clone(), x["k_scale"].clone(), x["v_scale"].clone()
    vs[:, :, 1] = 0.0        # V rows 128..255: zero, codes left as they are
    qs[:, 0, 2] = 0.0        # Q rows 256..383 of head 0
    ks[:, 1, 3] = 0.0        # K rows 384..511 of head 1
    deq = syn.dequantize_fp8_blocks_torch
    q64, k64, v64 = (deq(c, s_).numpy() for c, s_ in ((x["q"], qs), (x["k"], ks), (x["v"], vs)))
    assert np.all(v64[:, :, 128:256] == 0) and np.any(x["v"][:, :, 128:256].float().numpy() != 0)
    o, lse = fa.fa_fwd(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), causal=causal, scale=x["scale"],
                       q_descale=qs.to(DEV), k_descale=ks.to(DEV), v_descale=vs.to(DEV))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(q64, k64, v64, x["scale"], causal)
    eo, el = max_abs_err(o, o_ref), max_abs_err(lse, lse_ref)
    _say(f"fp8 zero scales causal={causal}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    assert eo <= TOL["fp8"] and el <= TOL["fp8"], (eo, el)


def test_binding_rejects_wrong_tensors():
    """The C ABI sees only pointers; the binding checks every tensor it passes
    (shape, dtype, device, contiguity, workspace bytes) and raises ValueError
    instead of letting a kernel read or write out of bounds."""
    B, H, N, d = 1, 2, 256, 64
    g = torch.Generator().manual_seed(3)
    q, k, v, do = (torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(DEV) for _ in range(4))
    o, lse = fa.fa_fwd(q, k, v)
    bad_fwd = [
        dict(out=torch.empty(B, H, N - 1, d, device=DEV, dtype=torch.bfloat16)),      # undersized
        dict(out=torch.empty(B, H, N, d, device=DEV, dtype=torch.float32)),           # wrong dtype
        dict(out=torch.empty(B, H, d, N, device=DEV, dtype=torch.bfloat16).transpose(2, 3)),
        dict(lse=torch.empty(B, H, N - 1, device=DEV)),
        dict(lse=torch.empty(B, H, N, device="cpu")),
    ]
    for kw in bad_fwd:
        with pytest.raises(ValueError):
            fa.fa_fwd(q, k, v, **kw)
    bad_bwd = [
        dict(do=do.transpose(2, 3).contiguous().transpose(2, 3)),                       # transposed view
        dict(do=do.float()),                                                            # fp32 dO
        dict(o=o[:, :, : N // 2]),
        dict(lse=lse.double()),
        dict(dq=torch.empty(B, H, N, d // 2, device=DEV, dtype=torch.bfloat16)),
        dict(workspace=torch.empty(16, device=DEV, dtype=torch.uint8)),
    ]
    for kw in bad_bwd:
        args = dict(o=o, lse=lse, do=do)
        args.update({kk: vv for kk, vv in kw.items() if kk in args})
        rest = {kk: vv for kk, vv in kw.items() if kk not in args}
        with pytest.raises(ValueError):
            fa.fa_bwd(q, k, v, args["o"], args["lse"], args["do"], **rest)
    # fp8: descales of the wrong shape
    y = torch.zeros(1, 1, 200, 128, device=DEV, dtype=torch.float8_e4m3fn)
    s_ok = torch.ones(1, 1, 2, device=DEV)
    with pytest.raises(ValueError):
        fa.fa_fwd(y, y, y, q_descale=torch.ones(1, 1, 1, device=DEV), k_descale=s_ok, v_descale=s_ok)
    # a workspace counted in bytes, whatever its dtype
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, H, N, d) // 4, device=DEV, dtype=torch.float32)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, lse, do, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all()


@pytest.mark.parametrize("H,H_kv,causal", [(4, 2, True), (2, 2, False)])
def test_attention_autograd_is_the_entry_points(H, H_kv, causal):
    """fa.attention under autograd gives exactly fa_fwd's O and, for a strided
    upstream gradient, exactly fa_bwd's dQ, dK, dV (per K/V head)."""
    _say(f"autograd H={H}/{H_kv} causal={causal}")
    w = syn.Workload("autograd", 2, H, H_kv, 333, 128, "bf16", causal, 1.0, 71, backward=True)
    x = syn.make_inputs(w)
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = fa.attention(qa, ka, va, causal=causal)
    do_strided = do.transpose(2, 3).contiguous().transpose(2, 3)
    assert not do_strided.is_contiguous()
    (o * do_strided).sum().backward()
    o_ref, lse = fa.fa_fwd(q, k, v, causal=causal)
    grads = fa.fa_bwd(q, k, v, o_ref, lse, do, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    for got, ref in zip((qa.grad, ka.grad, va.grad), grads):
        assert got.shape == ref.shape and torch.equal(got, ref)


def test_attention_autograd_masks_are_the_entry_points():
    """fa.attention with seqlens and a window, or with a block mask, gives
    exactly the masked and block-sparse entry points' outputs and gradients."""
    _say("autograd masked / block-sparse")
    B, H, N, d = 2, 2, 384, 128
    w = syn.Workload("autograd_m", B, H, H, N, d, "bf16", True, 1.0, 73, backward=True)
    x = syn.make_inputs(w)
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    seqlens = torch.tensor([300, 384], device=DEV, dtype=torch.int32)
    nb = (N + 127) // 128
    bm = (torch.rand(H, nb, nb, generator=torch.Generator().manual_seed(5)) < 0.6).to(torch.uint8)
    bm[:, torch.arange(nb), torch.arange(nb)] = 1
    bm = bm.to(DEV)
    cases = [(dict(seqlens=seqlens, window=100),
              lambda: fa.fa_fwd_masked(q, k, v, seqlens=seqlens, window=100, causal=True),
              lambda o, lse: fa.fa_bwd_masked(q, k, v, o, lse, do, seqlens=seqlens, window=100, causal=True)),
             (dict(block_mask=bm),
              lambda: fa.fa_fwd_blocksparse(q, k, v, bm, causal=True),
              lambda o, lse: fa.fa_bwd_blocksparse(q, k, v, o, lse, do, bm, causal=True))]
    for kw, f_ref, b_ref in cases:
        qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
        o = fa.attention(qa, ka, va, causal=True, **kw)
        (o * do).sum().backward()
        o_ref, lse = f_ref()
        grads = b_ref(o_ref, lse)
        torch.cuda.synchronize()
        assert torch.equal(o.detach(), o_ref)
        for got, ref in zip((qa.grad, ka.grad, va.grad), grads):
            assert torch.equal(got, ref)
    with pytest.raises(ValueError):
        fa.attention(q, k, v, seqlens=seqlens, block_mask=bm)
