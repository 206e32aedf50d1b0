"""CPU tests of the C ABI: the library loads, exports every declared entry
point, imports no allocator, and rejects every invalid argument before it
touches the HIP runtime (so no GPU is needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import exact_tiled_attention_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        from exact_tiled_attention_amd import build
        build.build(verbose=False)
    return fa.load_library()


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:fa_status|size_t|int|const char\*)\s+(fa_\w+)\s*\(", src, re.M)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(fa.EXPORTED)


def test_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, re.M))
    for name in _declared():
        assert name in exported, name
        getattr(lib, name)


def test_library_never_allocates_device_memory():
    out = subprocess.run(["nm", "-D", "--undefined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    for bad in ("hipMalloc", "hipFree", "hipMallocAsync", "hipHostMalloc", "hipMallocManaged"):
        assert not re.search(rf"\b{bad}\b", out), bad


def test_status_strings(lib):
    for code in range(7):
        s = fa.fa_status_string(code)
        assert s.startswith(fa.STATUS_NAMES[code])
    assert fa.fa_status_string(99) == "unknown fa_status"


def test_supported_table(lib):
    assert fa.fa_supported(0, 64, False)
    for d in (64, 128, 256):
        assert fa.fa_supported(1, d, False)
    assert fa.fa_supported(2, 128, False)
    assert fa.fa_supported(1, 64, True) and fa.fa_supported(1, 128, True) and fa.fa_supported(1, 256, True)
    for dt, d, bwd in [(1, 96, False), (1, 192, False), (0, 128, False), (2, 64, False), (2, 128, True),
                       (0, 64, True), (1, 96, True), (7, 64, False)]:
        assert not fa.fa_supported(dt, d, bwd), (dt, d, bwd)


P = 1 << 20  # a fake, 16-byte aligned address: validation rejects before any use


def fwd(lib, q=P, k=2 * P, v=3 * P, o=4 * P, lse=5 * P, qs=None, ks=None, vs=None,
        B=1, H=2, Hkv=2, N=16, d=64, scale=0.125, causal=1, dtype=1):
    return lib.fa_fwd(q, k, v, o, lse, qs, ks, vs, B, H, Hkv, N, d, scale, causal, dtype, None)


def bwd(lib, ws=64 * P, ws_bytes=1 << 21, d=64, dtype=1, N=16, H=2, Hkv=2, B=1, scale=0.125,
        ptrs=None):
    p = ptrs or [P * (i + 1) for i in range(9)]
    return lib.fa_bwd(*p, ws, ws_bytes, B, H, Hkv, N, d, scale, 1, dtype, None)


def test_fwd_validation(lib):
    assert fwd(lib, q=None) == 1
    assert fwd(lib, o=None) == 1
    assert fwd(lib, dtype=2) == 1                    # fp8 without descales
    assert fwd(lib, N=0) == 2
    assert fwd(lib, B=-1) == 2
    assert fwd(lib, H=6, Hkv=4) == 2                 # H % H_kv != 0
    assert fwd(lib, N=1 << 29) == 2
    assert fwd(lib, d=96) == 3                       # unsupported head dim
    assert fwd(lib, d=128, dtype=0) == 3
    assert fwd(lib, dtype=9) == 3
    assert fwd(lib, scale=float("nan")) == 4
    assert fwd(lib, scale=float("inf")) == 4
    assert fwd(lib, scale=0.0) == 4                  # a masked -inf score times 0 is NaN
    assert fwd(lib, scale=-0.125) == 4               # would turn masked scores into +inf
    assert fwd(lib, qs=7 * P) == 4                   # descale on a non-fp8 call
    assert fwd(lib, q=P + 8) == 4                    # misaligned
    assert fwd(lib, lse=P + 4) == 4
    assert fwd(lib, o=P) == 4                        # O aliases Q
    assert fwd(lib, lse=4 * P + 64) == 4             # LSE inside O


def test_bwd_validation(lib):
    assert bwd(lib, ptrs=[None] + [P * (i + 2) for i in range(8)]) == 1
    assert bwd(lib, dtype=2, d=128) == 3             # FP8 has no backward
    assert bwd(lib, d=96) == 3
    assert bwd(lib, N=0) == 2
    assert bwd(lib, scale=float("nan")) == 4
    assert bwd(lib, scale=-1.0) == 4
    assert bwd(lib, ws=None) == 5
    assert bwd(lib, ws_bytes=16) == 5
    assert bwd(lib, ws=64 * P + 128) == 5            # not 256-byte aligned
    assert bwd(lib, ptrs=[P * (i + 1) for i in range(8)] + [P]) == 4   # dV aliases Q


def fwdm(lib, q=P, k=2 * P, v=3 * P, o=4 * P, lse=5 * P, seqlens=None, window=-1, B=2, H=2, Hkv=2, N=16,
         d=64, scale=0.125, causal=1, dtype=1):
    return lib.fa_fwd_masked(q, k, v, o, lse, seqlens, window, B, H, Hkv, N, d, scale, causal, dtype, None)


def test_masked_validation(lib):
    assert fwdm(lib, q=None) == 1
    assert fwdm(lib, N=0) == 2
    assert fwdm(lib, dtype=0) == 3                   # bf16 only
    assert fwdm(lib, dtype=2, d=128) == 3
    assert fwdm(lib, d=96) == 3
    assert fwdm(lib, scale=0.0) == 4
    assert fwdm(lib, window=8, causal=0) == 4        # a window is causal
    assert fwdm(lib, seqlens=6 * P + 2) == 4         # not 4-byte aligned
    assert fwdm(lib, seqlens=4 * P + 8) == 4         # inside O
    assert fwdm(lib, lse=4 * P + 64) == 4            # LSE inside O


def test_masked_backward_validation(lib):
    ptrs = [P * (i + 2) for i in range(9)]
    def bwdm(seqlens=None, window=-1, d=64, dtype=1, causal=1):
        return lib.fa_bwd_masked(*ptrs, 64 * P, 1 << 21, seqlens, window, 1, 2, 2, 16, d, 0.125, causal, dtype,
                                 None)
    assert bwdm(d=96) == 3
    assert bwdm(dtype=0) == 3
    assert bwdm(window=4, causal=0) == 4
    assert bwdm(seqlens=70 * P + 1) == 4           # not 4-byte aligned
    assert bwdm(seqlens=8 * P) == 4                # inside dQ


def test_blocksparse_validation(lib):
    f = lambda bm=9 * P, d=64, dtype=1, o=4 * P, N=16: lib.fa_fwd_blocksparse(
        P, 2 * P, 3 * P, o, 5 * P, bm, 1, 2, 2, N, d, 0.125, 1, dtype, None)
    assert f(bm=None) == 1
    assert f(d=256) == 3                             # no d = 256 block-sparse kernel
    assert f(dtype=0) == 3
    assert f(bm=4 * P + 64) == 4                     # mask inside O
    assert f(N=131073) == 2                          # a mask row is at most 1024 blocks
    ptrs = [P * (i + 2) for i in range(9)]
    g = lambda bm=70 * P, d=64, H=2, Hkv=2, N=16: lib.fa_bwd_blocksparse(
        *ptrs, 64 * P, 1 << 40, bm, 1, H, Hkv, N, d, 0.125, 1, 1, None)
    assert g(bm=None) == 1
    assert g(d=256) == 3
    assert g(bm=8 * P) == 4                          # mask inside dQ
    assert g(N=131073) == 2
    assert g(H=32, Hkv=1, N=65536 + 1) == 2          # a GQA group's key-block column over 16384 flags


def kvc(lib, q=P, k=2 * P, v=3 * P, kv_len=None, o=4 * P, lse=5 * P, ws=64 * P, ws_bytes=1 << 30,
        B=2, H=8, Hkv=2, Nq=1, Nkv=300, d=128, scale=0.08, causal=1, dtype=1):
    return lib.fa_fwd_kvcache(q, k, v, kv_len, o, lse, ws, ws_bytes, B, H, Hkv, Nq, Nkv, d, scale,
                              causal, dtype, None)


def test_kvcache_validation(lib):
    assert kvc(lib, q=None) == 1
    assert kvc(lib, o=None) == 1
    assert kvc(lib, Nq=0) == 2
    assert kvc(lib, Nkv=0) == 2
    assert kvc(lib, Hkv=3) == 2                      # H not a multiple of H_kv
    assert kvc(lib, d=96) == 3
    assert kvc(lib, dtype=0, d=64) == 3              # no fp32 decode kernel
    assert kvc(lib, dtype=2) == 3
    assert kvc(lib, scale=0.0) == 4
    assert kvc(lib, scale=float("inf")) == 4
    assert kvc(lib, kv_len=6 * P + 2) == 4           # kv_len not 4-byte aligned
    assert kvc(lib, o=P + 16) == 4                   # O overlaps Q
    assert kvc(lib, kv_len=4 * P) == 4               # O overlaps kv_len
    assert kvc(lib, ws=None) == 5
    assert kvc(lib, ws_bytes=1024) == 5
    assert kvc(lib, ws=64 * P + 16) == 5             # workspace not 256-byte aligned
    assert kvc(lib, ws=4 * P) == 4                   # workspace overlaps O


def test_kvcache_workspace_bytes(lib):
    for d in (64, 128, 256):
        assert fa.fa_kvcache_supported(1, d)
    assert not fa.fa_kvcache_supported(1, 96) and not fa.fa_kvcache_supported(0, 64)
    assert fa.fa_fwd_kvcache_workspace_bytes(1, 8, 2, 1, 300, 96) == 0
    assert fa.fa_fwd_kvcache_workspace_bytes(1, 8, 3, 1, 300, 128) == 0
    # one partial (query rows x (d outputs + 1 logsumexp), fp32) per wave of
    # the split grid: 256 CUs x 4 resident waves at d = 128
    ws = fa.fa_fwd_kvcache_workspace_bytes(1, 8, 2, 1, 300, 128)
    rows = 1024 * 4                                  # waves * (G * N_q) rows
    assert ws == ((rows * 4 + 255) // 256) * 256 + rows * 128 * 4
    # it does not grow with the cache
    assert fa.fa_fwd_kvcache_workspace_bytes(8, 32, 8, 1, 32768, 128) == ws
    # at least one wave per (batch, K/V head, 32-row query group)
    many = fa.fa_fwd_kvcache_workspace_bytes(2048, 8, 8, 1, 64, 128)
    assert many == ((2048 * 8 * 4 + 255) // 256) * 256 + 2048 * 8 * 128 * 4


def test_workspace_bytes(lib):
    assert fa.fa_bwd_workspace_bytes(2, 16, 16, 16384, 64) == 2 * (2 * 16 * 16384 * 4)
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 3, 64) == 512
    assert fa.fa_bwd_workspace_bytes(0, 1, 1, 3, 64) == 0
