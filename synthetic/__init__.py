"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module only draws and encodes inputs; it holds none of the attention
arithmetic.  Every tensor is produced on the CPU from a seeded
``torch.Generator`` in the order Q, K, V, dO, scaled by an amplitude and then
encoded in the dtype the kernel consumes:

* ``f32``  -- the draws as they are;
* ``bf16`` -- round-to-nearest-even to bfloat16 (``Tensor.to``);
* ``fp8``  -- OCP e4m3 (``float8_e4m3fn``, largest finite 448) with one fp32
  scale per block of 128 consecutive rows of one head (all d columns).  The
  scale is ``amax / 448`` (1 where the block is all zero); the code is
  ``RNE(x / scale)`` clamped to +-448.  This is the block-wise quantisation
  with per-tile rescaling that the FP8 paragraph of "Flash Attention 2 / 3
  とは 2026年版" (section "FA3 の飛躍") names; the pages leave its details
  open, so the block size and the amax/448 rule follow the FP8 workload
  statement (one fp32 scale per 128-row block).

Layouts are contiguous ``[B][H][N][d]`` for Q, O, dO and ``[B][H_kv][N][d]``
for K and V, the (batch, head, seq, dim) order of the pages' SDPA example.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

FP8_MAX = 448.0          # largest finite OCP e4m3 value
FP8_BLOCK = 128          # rows per fp8 scale block


@dataclass(frozen=True)
class Workload:
    """One attention problem: shape, dtype, mask and the recipe of its inputs."""

    name: str
    B: int
    H: int
    H_kv: int
    N: int
    d: int
    dtype: str            # "f32" | "bf16" | "fp8"
    causal: bool
    amp: float = 1.0
    seed: int = 0
    backward: bool = False
    note: str = field(default="", compare=False)

    def flops_fwd(self) -> float:
        """4*B*H*N^2*d, halved exactly when causal (H counts query heads)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if self.causal else f

    def flops_bwd(self) -> float:
        """Backward is credited as 2.5x the forward count."""
        return 2.5 * self.flops_fwd()


# The five problem statements plus the headline-size stand-ins (causal bf16,
# N >= 8192, d = 128).  Seeds: 1..6 for the five, 7..9 for the stand-ins.
WORKLOADS = {
    "C1": Workload("C1", 1, 8, 8, 1024, 64, "f32", True, 1.0, 1,
                   note="fp32 forward, the shape of the pages' CPU SDPA measurement"),
    "C2a": Workload("C2a", 1, 8, 8, 8192, 64, "bf16", True, 1.0, 2),
    "C2a_nc": Workload("C2a_nc", 1, 8, 8, 8192, 64, "bf16", False, 1.0, 2),
    "C2b": Workload("C2b", 8, 16, 16, 2048, 256, "bf16", True, 1.0, 3),
    "C3": Workload("C3", 4, 32, 8, 4096, 128, "bf16", True, 0.5, 4,
                   note="GQA prefill: 4 query heads share one K/V head"),
    "C4": Workload("C4", 2, 16, 16, 16384, 64, "bf16", True, 1.0, 5, backward=True),
    "C5": Workload("C5", 1, 32, 32, 32768, 128, "fp8", True, 1.0, 6),
    "Ta": Workload("Ta", 4, 32, 32, 8192, 128, "bf16", True, 1.0, 7),
    "Ta_gqa": Workload("Ta_gqa", 4, 32, 8, 8192, 128, "bf16", True, 1.0, 7),
    "Tb": Workload("Tb", 2, 32, 32, 16384, 128, "bf16", True, 1.0, 8),
    "Tc": Workload("Tc", 1, 32, 32, 32768, 128, "bf16", True, 1.0, 9),
}


def draw(B, H, H_kv, N, d, amp=1.0, seed=0, with_do=False):
    """fp32 N(0, amp^2) draws in the fixed order Q, K, V, dO."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    k = torch.randn(B, H_kv, N, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, H_kv, N, d, generator=g, dtype=torch.float32)
    do = torch.randn(B, H, N, d, generator=g, dtype=torch.float32) if with_do else None
    if amp != 1.0:
        q.mul_(amp)
        k.mul_(amp)
        v.mul_(amp)
        if do is not None:
            do.mul_(amp)
    return q, k, v, do


def quantize_fp8_blocks(x: torch.Tensor, block: int = FP8_BLOCK):
    """Encode fp32 ``x`` [B][H][N][d] as e4m3 codes plus per-block fp32 scales.

    Returns ``(codes, scales)``: ``codes`` is ``float8_e4m3fn`` of x's shape,
    ``scales`` is fp32 ``[B][H][ceil(N/block)]``.  The value a consumer must
    use for element (b,h,n,:) is ``float(codes) * scales[b,h,n // block]``.
    """
    B, H, N, d = x.shape
    nb = (N + block - 1) // block
    pad = nb * block - N
    xp = torch.nn.functional.pad(x, (0, 0, 0, pad)) if pad else x
    xb = xp.reshape(B, H, nb, block * d)
    amax = xb.abs().amax(dim=-1)                          # [B,H,nb] fp32
    scales = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    y = (xb / scales.unsqueeze(-1)).clamp_(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).reshape(B, H, nb * block, d)[:, :, :N, :]
    return codes.contiguous(), scales.contiguous()


def dequantize_fp8_blocks_torch(codes: torch.Tensor, scales: torch.Tensor,
                                block: int = FP8_BLOCK) -> torch.Tensor:
    """The exact real value of every fp8 element, in float64."""
    N = codes.shape[2]
    s = scales.to(torch.float64).repeat_interleave(block, dim=2)[:, :, :N]
    return codes.to(torch.float64) * s.unsqueeze(-1)


def make_inputs(w: Workload, with_do: bool | None = None):
    """Build the device-ready (CPU) tensors of a workload.

    Returns a dict with ``q, k, v`` in the kernel dtype (float32, bfloat16 or
    float8_e4m3fn), ``q_scale, k_scale, v_scale`` (fp8 only, else None),
    ``do`` (bfloat16/float32, when requested) and ``*_64``: float64 numpy
    views of exactly the values the kernel sees, for the oracle.
    """
    if with_do is None:
        with_do = w.backward
    q, k, v, do = draw(w.B, w.H, w.H_kv, w.N, w.d, w.amp, w.seed, with_do)
    return pack_inputs(q, k, v, do, w.dtype)


def pack_inputs(q, k, v, do, dtype: str):
    """Cast fp32 CPU tensors ``q, k, v`` (and ``do`` or None) to a kernel dtype.

    Returns the dict described under make_inputs; the softmax scale is
    1/sqrt(d) for the head dim of ``q``.
    """
    out = {"q_scale": None, "k_scale": None, "v_scale": None, "do": None, "do_64": None}
    if dtype == "f32":
        out.update(q=q, k=k, v=v)
        if do is not None:
            out["do"] = do
        exact = (q.double(), k.double(), v.double(), do.double() if do is not None else None)
    elif dtype == "bf16":
        qb, kb, vb = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
        out.update(q=qb, k=kb, v=vb)
        if do is not None:
            out["do"] = do.to(torch.bfloat16)
        exact = (qb.double(), kb.double(), vb.double(),
                 out["do"].double() if do is not None else None)
    elif dtype == "fp8":
        (qc, qs), (kc, ks), (vc, vs) = (quantize_fp8_blocks(t) for t in (q, k, v))
        out.update(q=qc, k=kc, v=vc, q_scale=qs, k_scale=ks, v_scale=vs)
        exact = (dequantize_fp8_blocks_torch(qc, qs), dequantize_fp8_blocks_torch(kc, ks),
                 dequantize_fp8_blocks_torch(vc, vs), None)
        if do is not None:
            out["do"] = do.to(torch.bfloat16)
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    out["q_64"], out["k_64"], out["v_64"] = (t.numpy() for t in exact[:3])
    if exact[3] is not None:
        out["do_64"] = exact[3].numpy()
    out["scale"] = 1.0 / math.sqrt(q.shape[-1])
    return out


def rand_rows(n_total: int, count: int, seed: int):
    """A seeded sorted sample of distinct row indices (always includes 0 and n-1)."""
    g = torch.Generator("cpu").manual_seed(seed)
    count = min(count, n_total)
    idx = torch.randperm(n_total, generator=g)[:count]
    idx = torch.unique(torch.cat([idx, torch.tensor([0, n_total - 1])]))
    return idx.tolist()


# ------------------------------------------------------- KV-cache (decode) ---

@dataclass(frozen=True)
class KvCacheWorkload:
    """N_q new queries per head against a KV cache of capacity N_kv.

    ``ragged``: the cache lengths of the batch are drawn (seeded) in
    [1, N_kv] instead of all being N_kv.
    """

    name: str
    B: int
    H: int
    H_kv: int
    N_q: int
    N_kv: int
    d: int
    dtype: str = "bf16"
    causal: bool = True
    amp: float = 1.0
    seed: int = 0
    ragged: bool = False
    note: str = field(default="", compare=False)

    def cache_bytes(self, lens) -> int:
        """Bytes of K and V a call reads: every used cache row once."""
        elem = {"f32": 4, "bf16": 2, "fp8": 1}[self.dtype]
        return 2 * self.H_kv * self.d * elem * int(sum(lens))

    def flops(self, lens) -> float:
        """4 * d flops per (query, visible key) pair (QK^T and PV)."""
        tot = 0
        for n in lens:
            for i in range(self.N_q):
                tot += max(0, min(n, n - self.N_q + i + 1)) if self.causal else n
        return 4.0 * self.H * self.d * tot


# One new token per sequence with the GQA head layout of the prefill shape
# (32 query heads on 8 K/V heads, d = 128) and a 32K-token cache; seeds 10+.
KV_WORKLOADS = {
    "D1": KvCacheWorkload("D1", 8, 32, 8, 1, 32768, 128, seed=10,
                          note="decode, one new token per sequence, full 32K caches"),
    "D1_ragged": KvCacheWorkload("D1_ragged", 8, 32, 8, 1, 32768, 128, seed=11, ragged=True,
                                 note="decode with a seeded mix of cache lengths in [1, 32768]"),
}


def draw_kvcache(B, H, H_kv, N_q, N_kv, d, amp=1.0, seed=0):
    """fp32 N(0, amp^2) draws in the fixed order Q [B,H,N_q,d], K, V [B,H_kv,N_kv,d]."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, H, N_q, d, generator=g, dtype=torch.float32)
    k = torch.randn(B, H_kv, N_kv, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, H_kv, N_kv, d, generator=g, dtype=torch.float32)
    if amp != 1.0:
        q.mul_(amp)
        k.mul_(amp)
        v.mul_(amp)
    return q, k, v


def cache_lengths(B, N_kv, seed):
    """Seeded cache lengths, uniform in [1, N_kv], as a CPU int32 tensor [B]."""
    g = torch.Generator("cpu").manual_seed(seed + 7919)
    return torch.randint(1, N_kv + 1, (B,), generator=g, dtype=torch.int32)


def make_kvcache_inputs(w: KvCacheWorkload):
    """pack_inputs of the workload's draws plus ``kv_len`` (int32 CPU tensor or
    None) and ``lens`` (the lengths as a list, N_kv each when not ragged)."""
    q, k, v = draw_kvcache(w.B, w.H, w.H_kv, w.N_q, w.N_kv, w.d, w.amp, w.seed)
    out = pack_inputs(q, k, v, None, w.dtype)
    out["kv_len"] = cache_lengths(w.B, w.N_kv, w.seed) if w.ragged else None
    out["lens"] = out["kv_len"].tolist() if w.ragged else [w.N_kv] * w.B
    return out


# ------------------------------------------- padding mask / sliding window ---

@dataclass(frozen=True)
class MaskedWorkload:
    """A forward with a per-sequence padding mask (``ragged``: seeded valid
    lengths in [1, N]) and/or a causal sliding window (query i sees keys
    i - window .. i)."""

    name: str
    B: int
    H: int
    H_kv: int
    N: int
    d: int
    dtype: str = "bf16"
    causal: bool = True
    amp: float = 1.0
    seed: int = 0
    window: int | None = None
    ragged: bool = False
    note: str = field(default="", compare=False)

    def visible_pairs(self, lens) -> int:
        """(query, key) pairs the mask leaves, summed over sequences (per head)."""
        tot = 0
        for n in lens:
            i = torch.arange(int(n), dtype=torch.int64)
            hi = i if self.causal else torch.full_like(i, int(n) - 1)
            lo = (i - self.window).clamp(min=0) if self.window is not None else torch.zeros_like(i)
            tot += int((hi - lo + 1).clamp(min=0).sum())
        return tot

    def flops_fwd(self, lens) -> float:
        """4 * d flops per visible pair and query head."""
        return 4.0 * self.H * self.d * self.visible_pairs(lens)


# Prefill with the GQA head layout of the stated prefill shape: a 4096-key
# sliding window (each query sees itself and 4095 earlier keys) at N = 8192,
# and a right-padded batch of seeded lengths at N = 4096.  Seeds 12+.
MASKED_WORKLOADS = {
    "W1": MaskedWorkload("W1", 4, 32, 8, 8192, 128, seed=12, window=4095,
                         note="causal sliding window of 4096 keys"),
    "P1": MaskedWorkload("P1", 8, 32, 8, 4096, 128, seed=13, ragged=True,
                         note="right-padded batch, seeded valid lengths in [1, 4096]"),
}


def make_masked_inputs(w: MaskedWorkload):
    """pack_inputs of the workload's draws plus ``seqlens`` (int32 CPU tensor
    or None) and ``lens`` (the lengths as a list, N each when not ragged)."""
    q, k, v, _ = draw(w.B, w.H, w.H_kv, w.N, w.d, w.amp, w.seed)
    out = pack_inputs(q, k, v, None, w.dtype)
    out["seqlens"] = cache_lengths(w.B, w.N, w.seed) if w.ragged else None
    out["lens"] = out["seqlens"].tolist() if w.ragged else [w.N] * w.B
    return out


# ------------------------------------------------------------- block-sparse ---

@dataclass(frozen=True)
class BlockSparseWorkload:
    """A forward with a 128 x 128 block mask per head: each block is on with
    probability ``density`` (seeded), and the diagonal blocks are always on
    so that every query sees at least itself."""

    name: str
    B: int
    H: int
    H_kv: int
    N: int
    d: int
    density: float
    dtype: str = "bf16"
    causal: bool = True
    amp: float = 1.0
    seed: int = 0
    note: str = field(default="", compare=False)

    def visible_pairs(self, block_mask) -> int:
        """(query, key) pairs the mask leaves, summed over heads (per sequence)."""
        nb = block_mask.shape[1]
        bm = block_mask.to(torch.int64)
        if not self.causal:
            return int(bm.sum()) * 128 * 128 if self.N % 128 == 0 else _pairs_exact(bm, self.N, False)
        return _pairs_exact(bm, self.N, True)

    def flops_fwd(self, block_mask) -> float:
        return 4.0 * self.B * self.d * self.visible_pairs(block_mask)


def _pairs_exact(bm, n, causal):
    """Visible pairs of a block mask over n tokens, summed over heads."""
    nb = bm.shape[1]
    size = torch.full((nb,), 128, dtype=torch.int64)
    size[-1] = n - 128 * (nb - 1)
    full = size[:, None] * size[None, :]                   # pairs per block
    if causal:
        strict = torch.ones(nb, nb, dtype=torch.bool).tril(-1)
        diag = size * (size + 1) // 2                       # a diagonal block's lower triangle
        per = torch.where(strict, full, torch.zeros_like(full))
        per = per + torch.diag(diag)
    else:
        per = full
    return int((bm * per[None]).sum())


def block_mask(w: BlockSparseWorkload):
    """Seeded uint8 CPU tensor [H, nb, nb] of the workload's block mask."""
    nb = (w.N + 127) // 128
    g = torch.Generator("cpu").manual_seed(w.seed + 31337)
    m = (torch.rand(w.H, nb, nb, generator=g) < w.density).to(torch.uint8)
    idx = torch.arange(nb)
    m[:, idx, idx] = 1
    return m


# The block-sparse setting of the pages' 64K experiment, at the head layout of
# the GQA prefill shape with d = 128; seed 14.
BLOCKSPARSE_WORKLOADS = {
    "S1": BlockSparseWorkload("S1", 1, 16, 4, 65536, 128, 0.25, seed=14,
                              note="causal, 25% of the 128x128 blocks on (diagonal always on)"),
}


def make_blocksparse_inputs(w: BlockSparseWorkload):
    q, k, v, _ = draw(w.B, w.H, w.H_kv, w.N, w.d, w.amp, w.seed)
    out = pack_inputs(q, k, v, None, w.dtype)
    out["block_mask"] = block_mask(w)
    return out
