"""CPU tests of the seeded input generator and the fp8 block encoder."""
import math

import numpy as np
import torch

import synthetic as syn


def test_draws_are_seeded_and_ordered():
    a = syn.draw(1, 2, 1, 10, 4, seed=3, with_do=True)
    b = syn.draw(1, 2, 1, 10, 4, seed=3, with_do=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    g = torch.Generator().manual_seed(3)
    q = torch.randn(1, 2, 10, 4, generator=g)
    k = torch.randn(1, 1, 10, 4, generator=g)
    assert torch.equal(a[0], q) and torch.equal(a[1], k)


def test_bf16_inputs_are_rne_of_draws():
    w = syn.Workload("t", 1, 2, 2, 33, 16, "bf16", True, 0.5, 9)
    x = syn.make_inputs(w)
    q32 = syn.draw(1, 2, 2, 33, 16, 0.5, 9)[0]
    assert x["q"].dtype == torch.bfloat16
    assert torch.equal(x["q"], q32.to(torch.bfloat16))
    assert np.array_equal(x["q_64"], x["q"].double().numpy())


def _e4m3_values():
    """Every finite non-negative OCP e4m3 value, from its bit layout."""
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue  # NaN encoding
            vals.append((m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(sorted(set(vals)))


def test_fp8_block_encoding():
    g = torch.Generator().manual_seed(5)
    x = torch.randn(2, 3, 300, 8, generator=g) * 3
    x[1, 2, 128:256] = 0.0                       # an all-zero block keeps scale 1
    codes, scales = syn.quantize_fp8_blocks(x)
    assert codes.dtype == torch.float8_e4m3fn
    assert scales.shape == (2, 3, 3)              # ceil(300/128) blocks, last one partial
    assert scales[1, 2, 1] == 1.0
    grid = _e4m3_values()
    assert grid.max() == 448.0
    c = codes.to(torch.float64).numpy()
    assert np.all(np.isin(np.abs(c), grid))       # every code is a finite e4m3 value
    xs = x.double().numpy()
    s = scales.double().numpy()
    for b in range(2):
        for h in range(3):
            for blk in range(3):
                sl = slice(blk * 128, min(300, (blk + 1) * 128))
                cb = c[b, h, sl]
                xb = xs[b, h, sl]
                if np.abs(xb).max() == 0:
                    assert np.all(cb == 0)
                    continue
                # the block amax lands on +-448 (up to the fp32 rounding of the scale)
                assert abs(np.abs(cb).max() - 448.0) <= 16.0
                # nearest-value rounding: |x/s - code| <= half the gap to the next value
                y = np.clip(xb / s[b, h, blk], -448, 448)
                idx = np.searchsorted(grid, np.abs(y))
                hi = grid[np.minimum(idx, grid.size - 1)]
                lo = grid[np.maximum(idx - 1, 0)]
                half_gap = np.maximum(hi - lo, 2.0 ** -9) / 2
                assert np.all(np.abs(np.abs(cb) - np.abs(y)) <= half_gap + 1e-12)
    # the value the consumer sees is code * scale, exact in float64
    deq = syn.dequantize_fp8_blocks_torch(codes, scales).numpy()
    rep = np.repeat(s, 128, axis=2)[:, :, :300, None]
    assert np.array_equal(deq, c * rep)


def test_fp8_workload_inputs():
    w = syn.Workload("t", 1, 2, 2, 200, 128, "fp8", True, 1.0, 6)
    x = syn.make_inputs(w)
    assert x["k_scale"].shape == (1, 2, 2)
    err = np.abs(x["q_64"] - syn.draw(1, 2, 2, 200, 128, 1.0, 6)[0].double().numpy())
    # e4m3 keeps 3 fraction bits: relative error <= 2^-4, absolute <= 2^-4 * amax
    assert err.max() <= 2.0 ** -4 * 5.0


def test_flop_formula():
    w = syn.WORKLOADS["C1"]
    assert w.flops_fwd() == 4 * 1 * 8 * 1024 ** 2 * 64 / 2
    assert w.flops_bwd() == 2.5 * w.flops_fwd()
    assert syn.WORKLOADS["C2a_nc"].flops_fwd() == 4 * 8 * 8192 ** 2 * 64


def test_scale_is_inverse_sqrt_d():
    x = syn.make_inputs(syn.Workload("t", 1, 1, 1, 4, 64, "f32", True))
    assert x["scale"] == 1.0 / math.sqrt(64)
