"""Kernel resources read back from the built gfx950 code objects (CPU only).

A kernel that spills to scratch memory or outgrows the LDS of a CU still
computes the right answer, so no parity test would notice; these checks
catch such regressions at build time instead.
"""
import glob
import os

import pytest

from exact_tiled_attention_amd import build as fa_build

OBJS = sorted(glob.glob(os.path.join(fa_build.BUILD, "*.hip.o")))
pytestmark = pytest.mark.skipif(not OBJS, reason="library not built (run __graft_entry__.build())")

LDS_BYTES_PER_CU = 160 * 1024


def _kernels():
    ks = [k for o in OBJS for k in fa_build.kernel_resources(o)]
    if not ks:
        pytest.skip("LLVM tools to read the code objects are not installed")
    return ks


def test_every_kernel_reports_its_resources():
    names = [k["name"] for k in _kernels()]
    for want in ("fwd_bf16_pp_kernel", "fwd_bf16_pairs_kernel", "fwd_bf16_kernel", "fwd_bf16_sp_kernel",
                 "fwd_fp8_pp_kernel", "fwd_f32_kernel", "bwd_prep_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel",
                 "kv_split_kernel", "kv_combine_kernel"):
        assert any(want in n for n in names), want


def test_no_scratch_outside_the_allowed_list():
    for k in _kernels():
        if any(a in k["name"] for a in fa_build.SCRATCH_ALLOWED):
            continue
        assert k["scratch"] == 0 and k["vgpr_spill"] == 0, k


def test_lds_fits_a_compute_unit():
    for k in _kernels():
        assert k["lds"] is not None and k["lds"] <= LDS_BYTES_PER_CU, k


def test_forward_kernels_keep_two_waves_a_simd():
    # 512 registers a lane per SIMD: two waves need at most 256 each
    for k in _kernels():
        if any(n in k["name"] for n in ("fwd_bf16_pp_kernel", "fwd_bf16_pairs_kernel", "fwd_fp8_pp_kernel")):
            assert k["vgpr"] <= 256, k
