"""Python binding of libfa.so, the gfx950 exact tiled attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/fa.h``.  There is no fallback:
if ``libfa.so`` is missing or a call is unsupported, an exception is raised.

The functions carry the C entry points' names.  ``fa_fwd`` and ``fa_bwd``
take torch tensors on the current HIP device, allocate the outputs (and the
backward workspace) with torch's allocator and enqueue the kernels on
``torch.cuda.current_stream()``.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["fa_fwd", "fa_fwd_masked", "fa_fwd_blocksparse", "fa_bwd", "fa_bwd_masked", "fa_bwd_blocksparse", "fa_bwd_workspace_bytes", "fa_fwd_kvcache",
           "fa_fwd_kvcache_workspace_bytes", "fa_supported", "fa_kvcache_supported",
           "fa_status_string", "FaError", "load_library", "LIB_PATH", "DTYPE_CODES"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_DTYPE_F32, FA_DTYPE_BF16, FA_DTYPE_FP8_E4M3 = 0, 1, 2
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_NULL_POINTER", 2: "FA_ERR_INVALID_SHAPE",
                3: "FA_ERR_UNSUPPORTED", 4: "FA_ERR_INVALID_VALUE", 5: "FA_ERR_WORKSPACE",
                6: "FA_ERR_HIP"}
EXPORTED = ("fa_fwd", "fa_fwd_masked", "fa_fwd_blocksparse", "fa_bwd", "fa_bwd_masked", "fa_bwd_blocksparse", "fa_bwd_workspace_bytes", "fa_fwd_kvcache",
            "fa_fwd_kvcache_workspace_bytes", "fa_supported", "fa_kvcache_supported",
            "fa_status_string")

_lib = None


class FaError(RuntimeError):
    """A non-OK status from libfa.so."""

    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code
        self.name = STATUS_NAMES.get(code, str(code))


def load_library(path: str = LIB_PATH):
    """Load libfa.so and declare its C signatures (raises if it is not built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() "
                          "(or python exact_tiled_attention_amd/build.py)")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_masked.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_masked.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_masked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_bwd_masked.restype = i
    lib.fa_fwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_blocksparse.restype = i
    lib.fa_bwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, i, i, i, i, i, f, i, i, vp]
    lib.fa_bwd_blocksparse.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_supported.argtypes = [i, i, i]
    lib.fa_supported.restype = i
    lib.fa_fwd_kvcache.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_kvcache.restype = i
    lib.fa_fwd_kvcache_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.fa_fwd_kvcache_workspace_bytes.restype = sz
    lib.fa_kvcache_supported.argtypes = [i, i]
    lib.fa_kvcache_supported.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def fa_status_string(code: int) -> str:
    return load_library().fa_status_string(int(code)).decode()


def fa_supported(dtype: int, d: int, backward: bool) -> bool:
    return bool(load_library().fa_supported(int(dtype), int(d), int(bool(backward))))


def fa_kvcache_supported(dtype: int, d: int) -> bool:
    return bool(load_library().fa_kvcache_supported(int(dtype), int(d)))


def fa_fwd_kvcache_workspace_bytes(B, H, H_kv, N_q, N_kv, d, dtype=FA_DTYPE_BF16) -> int:
    return int(load_library().fa_fwd_kvcache_workspace_bytes(B, H, H_kv, N_q, N_kv, d, int(dtype)))


def fa_bwd_workspace_bytes(B, H, H_kv, N, d, dtype=FA_DTYPE_BF16) -> int:
    return int(load_library().fa_bwd_workspace_bytes(B, H, H_kv, N, d, int(dtype)))


def _check(code: int):
    if code != 0:
        raise FaError(code, fa_status_string(code))


def _torch():
    import torch
    return torch


def DTYPE_CODES():
    torch = _torch()
    return {torch.float32: FA_DTYPE_F32, torch.bfloat16: FA_DTYPE_BF16,
            torch.float8_e4m3fn: FA_DTYPE_FP8_E4M3}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _shape(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d] / [B, H_kv, N, d]")
    B, H, N, d = q.shape
    if tuple(k.shape) != tuple(v.shape) or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share one dtype")
    return B, H, k.shape[1], N, d


def fa_fwd(q, k, v, causal: bool = True, scale: float | None = None,
           q_descale=None, k_descale=None, v_descale=None, out=None, lse=None,
           want_lse: bool = True):
    """O, LSE = attention(q, k, v).  Returns (o, lse); lse is None if not wanted."""
    torch = _torch()
    lib = load_library()
    B, H, H_kv, N, d = _shape(q, k, v)
    codes = DTYPE_CODES()
    if q.dtype not in codes:
        raise FaError(3, f"unsupported dtype {q.dtype}")
    dt = codes[q.dtype]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out_dtype = torch.float32 if dt == FA_DTYPE_F32 else torch.bfloat16
    if out is None:
        out = torch.empty(B, H, N, d, device=q.device, dtype=out_dtype)
    if lse is None and want_lse:
        lse = torch.empty(B, H, N, device=q.device, dtype=torch.float32)
    for t in (q_descale, k_descale, v_descale):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("descale tensors must be contiguous float32")
    code = lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                      _ptr(q_descale), _ptr(k_descale), _ptr(v_descale),
                      B, H, H_kv, N, d, float(scale), int(bool(causal)), dt, _stream())
    _check(code)
    return out, lse


def fa_fwd_masked(q, k, v, seqlens=None, window: int | None = None, causal: bool = True,
                  scale: float | None = None, out=None, lse=None, want_lse: bool = True):
    """O, LSE with a padding mask (seqlens: int32 device tensor [B] of valid rows,
    or None) and/or a causal sliding window (query i sees keys i - window .. i)."""
    torch = _torch()
    lib = load_library()
    B, H, H_kv, N, d = _shape(q, k, v)
    codes = DTYPE_CODES()
    if q.dtype not in codes:
        raise FaError(3, f"unsupported dtype {q.dtype}")
    dt = codes[q.dtype]
    if seqlens is not None and (seqlens.dtype != torch.int32 or not seqlens.is_cuda
                                or not seqlens.is_contiguous() or tuple(seqlens.shape) != (B,)):
        raise ValueError("seqlens must be a contiguous int32 device tensor of shape [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(B, H, N, d, device=q.device, dtype=torch.bfloat16)
    if lse is None and want_lse:
        lse = torch.empty(B, H, N, device=q.device, dtype=torch.float32)
    code = lib.fa_fwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(seqlens),
                             -1 if window is None else int(window), B, H, H_kv, N, d, float(scale),
                             int(bool(causal)), dt, _stream())
    _check(code)
    return out, lse


def fa_bwd(q, k, v, o, lse, do, causal: bool = True, scale: float | None = None,
           workspace=None, dq=None, dk=None, dv=None):
    """dQ, dK, dV of L = sum(O * dO), recomputing P from q, k and the forward's lse."""
    torch = _torch()
    lib = load_library()
    B, H, H_kv, N, d = _shape(q, k, v)
    codes = DTYPE_CODES()
    if q.dtype not in codes:
        raise FaError(3, f"unsupported dtype {q.dtype}")
    dt = codes[q.dtype]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = int(lib.fa_bwd_workspace_bytes(B, H, H_kv, N, d, dt))
    if workspace is None:
        workspace = torch.empty(max(need, 256), device=q.device, dtype=torch.uint8)
    code = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                      B, H, H_kv, N, d, float(scale), int(bool(causal)), dt, _stream())
    _check(code)
    return dq, dk, dv


def fa_fwd_kvcache(q, k_cache, v_cache, kv_len=None, causal: bool = True, scale: float | None = None,
                   out=None, lse=None, want_lse: bool = True, workspace=None):
    """O, LSE of N_q new queries against a KV cache (decode).

    q [B, H, N_q, d]; k_cache, v_cache [B, H_kv, N_kv, d] (capacity N_kv);
    kv_len: int32 device tensor [B] of cache rows in use, or None for N_kv.
    Returns (o, lse); lse is None if not wanted.
    """
    torch = _torch()
    lib = load_library()
    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("q must be [B, H, N_q, d], the caches [B, H_kv, N_kv, d]")
    B, H, N_q, d = q.shape
    _, H_kv, N_kv, dk = k_cache.shape
    if tuple(k_cache.shape) != tuple(v_cache.shape) or k_cache.shape[0] != B or dk != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k_cache.shape)} "
                         f"v {tuple(v_cache.shape)}")
    for t in (q, k_cache, v_cache):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q and the caches must be contiguous device tensors")
    if q.dtype != k_cache.dtype or q.dtype != v_cache.dtype:
        raise ValueError("q and the caches must share one dtype")
    if kv_len is not None and (kv_len.dtype != torch.int32 or not kv_len.is_cuda
                               or not kv_len.is_contiguous() or tuple(kv_len.shape) != (B,)):
        raise ValueError("kv_len must be a contiguous int32 device tensor of shape [B]")
    codes = DTYPE_CODES()
    if q.dtype not in codes:
        raise FaError(3, f"unsupported dtype {q.dtype}")
    dt = codes[q.dtype]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(B, H, N_q, d, device=q.device, dtype=torch.bfloat16)
    if lse is None and want_lse:
        lse = torch.empty(B, H, N_q, device=q.device, dtype=torch.float32)
    need = int(lib.fa_fwd_kvcache_workspace_bytes(B, H, H_kv, N_q, N_kv, d, dt))
    if workspace is None:
        workspace = torch.empty(max(need, 256), device=q.device, dtype=torch.uint8)
    code = lib.fa_fwd_kvcache(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_len), _ptr(out),
                              _ptr(lse), _ptr(workspace), workspace.numel(), B, H, H_kv, N_q, N_kv,
                              d, float(scale), int(bool(causal)), dt, _stream())
    _check(code)
    return out, lse


def fa_bwd_masked(q, k, v, o, lse, do, seqlens=None, window: int | None = None, causal: bool = True,
                  scale: float | None = None, workspace=None, dq=None, dk=None, dv=None):
    """dQ, dK, dV for fa_fwd_masked with the same seqlens and window."""
    torch = _torch()
    lib = load_library()
    B, H, H_kv, N, d = _shape(q, k, v)
    codes = DTYPE_CODES()
    if q.dtype not in codes:
        raise FaError(3, f"unsupported dtype {q.dtype}")
    dt = codes[q.dtype]
    if seqlens is not None and (seqlens.dtype != torch.int32 or not seqlens.is_cuda
                                or not seqlens.is_contiguous() or tuple(seqlens.shape) != (B,)):
        raise ValueError("seqlens must be a contiguous int32 device tensor of shape [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = int(lib.fa_bwd_workspace_bytes(B, H, H_kv, N, d, dt))
    if workspace is None:
        workspace = torch.empty(max(need, 256), device=q.device, dtype=torch.uint8)
    code = lib.fa_bwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), _ptr(seqlens),
                             -1 if window is None else int(window), B, H, H_kv, N, d, float(scale),
                             int(bool(causal)), dt, _stream())
    _check(code)
    return dq, dk, dv


def _block_mask_arg(block_mask, H, N):
    torch = _torch()
    nb = (N + 127) // 128
    if (block_mask.dtype != torch.uint8 or not block_mask.is_cuda or not block_mask.is_contiguous()
            or tuple(block_mask.shape) != (H, nb, nb)):
        raise ValueError(f"block_mask must be a contiguous uint8 device tensor of shape [{H}, {nb}, {nb}]")
    return _ptr(block_mask)


def fa_fwd_blocksparse(q, k, v, block_mask, causal: bool = True, scale: float | None = None,
                       out=None, lse=None, want_lse: bool = True):
    """O, LSE with a 128 x 128 block mask (uint8 device tensor [H, nb, nb])."""
    torch = _torch()
    lib = load_library()
    B, H, H_kv, N, d = _shape(q, k, v)
    codes = DTYPE_CODES()
    if q.dtype not in codes:
        raise FaError(3, f"unsupported dtype {q.dtype}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    bm = _block_mask_arg(block_mask, H, N)
    if out is None:
        out = torch.empty(B, H, N, d, device=q.device, dtype=torch.bfloat16)
    if lse is None and want_lse:
        lse = torch.empty(B, H, N, device=q.device, dtype=torch.float32)
    code = lib.fa_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), bm, B, H, H_kv, N, d,
                                  float(scale), int(bool(causal)), codes[q.dtype], _stream())
    _check(code)
    return out, lse


def fa_bwd_blocksparse(q, k, v, o, lse, do, block_mask, causal: bool = True, scale: float | None = None,
                       workspace=None, dq=None, dk=None, dv=None):
    """dQ, dK, dV for fa_fwd_blocksparse with the same block mask."""
    torch = _torch()
    lib = load_library()
    B, H, H_kv, N, d = _shape(q, k, v)
    codes = DTYPE_CODES()
    if q.dtype not in codes:
        raise FaError(3, f"unsupported dtype {q.dtype}")
    dt = codes[q.dtype]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    bm = _block_mask_arg(block_mask, H, N)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = int(lib.fa_bwd_workspace_bytes(B, H, H_kv, N, d, dt))
    if workspace is None:
        workspace = torch.empty(max(need, 256), device=q.device, dtype=torch.uint8)
    code = lib.fa_bwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                  _ptr(dv), _ptr(workspace), workspace.numel(), bm, B, H, H_kv, N, d,
                                  float(scale), int(bool(causal)), dt, _stream())
    _check(code)
    return dq, dk, dv
