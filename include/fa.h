/*
 * fa.h -- C ABI of the exact tiled attention library (libfa.so), gfx950.
 *
 * The library computes exact scaled dot-product attention
 *     O = softmax(scale * Q K^T) V
 * (the equation of "FlashAttention — フラッシュアテンション", section
 * 標準的なアテンションの問題点) as fused, tiled kernels that never write the
 * N x N score matrix to memory: K/V tiles stream through on-chip memory and a
 * running row max and row sum of exponentials rescale the partial output
 * whenever the max grows ("FlashAttentionとは？仕組みとFA2・FA3・FA4の違い…",
 * section タイリング・オンラインsoftmax・再計算という3つの仕組み).  The forward
 * saves one logsumexp per query row; the backward recomputes the probabilities
 * from Q/K tiles with it instead of storing them (same page, subsection
 * 逆伝播でL×L行列を保存せず再計算する設計).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory   All tensor pointers are DEVICE pointers owned by the caller.  The
 *          library allocates and frees nothing, keeps no pointer after a call
 *          returns and holds no mutable global state.
 * Layout   Contiguous row-major, d innermost:
 *            Q, O, dO, dQ    [B][H][N][d]
 *            K, V, dK, dV    [B][H_kv][N][d]
 *            LSE, D          [B][H][N]            (fp32)
 *          Every base pointer must be 16-byte aligned.
 * GQA      H must be a multiple of H_kv; query head h reads K/V head
 *          h / (H / H_kv) (contiguous groups), as grouped-query attention is
 *          described under FlashAttention-2 in "FlashAttention — フラッシュ
 *          アテンション" (進化と関連技術).
 * Causal   causal != 0 lets query i see keys 0..i (diagonal included).
 * LSE      LSE[i] = ln sum_{j visible} exp(scale * q_i . k_j)  (natural log).
 * Scale    finite and > 0 (FA_ERR_INVALID_VALUE otherwise); callers normally
 *          pass 1/sqrt(d).
 * Streams  Work is enqueued on `stream` and runs asynchronously; device-side
 *          faults surface at the caller's next synchronisation.
 * Errors   Every entry point validates all arguments on the host before it
 *          touches the HIP runtime and returns a status code; it never aborts
 *          and never silently falls back to another implementation: an
 *          unsupported (dtype, d, direction) combination is an error, as a
 *          forced FLASH backend raises instead of falling back in the pages'
 *          CPU SDPA experiment ("FlashAttentionとは？…", section CPUの
 *          PyTorch SDPAで測った一致度とメモリ削減の実測値).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_DTYPE_F32 = 0,      /* fp32 in, fp32 out                                  */
  FA_DTYPE_BF16 = 1,     /* bf16 in, bf16 out, fp32 accumulation               */
  FA_DTYPE_FP8_E4M3 = 2  /* OCP e4m3 (max 448) Q/K/V + per-128-row fp32 scales,
                            bf16 out                                           */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL_POINTER = 1,  /* a required pointer is NULL                       */
  FA_ERR_INVALID_SHAPE = 2, /* B,H,H_kv,N,d <= 0; H % H_kv != 0; size overflow  */
  FA_ERR_UNSUPPORTED = 3,   /* (dtype, d, direction) has no kernel              */
  FA_ERR_INVALID_VALUE = 4, /* scale not finite and > 0, misaligned pointer,
                               an output aliasing an input, descale for non-fp8 */
  FA_ERR_WORKSPACE = 5,     /* workspace NULL or smaller than required          */
  FA_ERR_HIP = 6            /* the HIP runtime reported an error at launch      */
} fa_status;

/*
 * Forward pass.
 *   Q [B][H][N][d], K/V [B][H_kv][N][d] in `dtype` (fp8: one byte per element).
 *   O [B][H][N][d]: fp32 for F32, bf16 for BF16 and FP8_E4M3.
 *   LSE [B][H][N] fp32, or NULL to skip it.
 *   q_descale [B][H][ceil(N/128)], k_descale and v_descale [B][H_kv][ceil(N/128)]:
 *     fp32 block scales, required for FP8_E4M3 and NULL otherwise; element
 *     (b,h,n,:) of a tensor stands for code * descale[b][h][n/128].  This is
 *     the block-wise quantisation with per-tile rescaling that "Flash
 *     Attention 2 / 3 とは 2026年版" names for FP8 attention (section FA3 の
 *     飛躍); the 128-row block is this library's choice.  Every descale must
 *     be finite and >= 0; 0 stands for a block whose values are all zero (as
 *     an amax/448 quantiser gives an all-zero block), whatever its codes: a
 *     zero Q or K block gives scores of 0, a zero V block adds nothing to O
 *     while its keys still count in the softmax sum.  Descales live on the
 *     device and are not checked: a negative or non-finite one gives
 *     undefined (typically non-finite) results.
 * Supported: F32 d=64; BF16 d=64,128,256; FP8_E4M3 d=128.  Any N >= 1.
 */
fa_status fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                 const float* q_descale, const float* k_descale, const float* v_descale,
                 int B, int H, int H_kv, int N, int d, float scale, int causal,
                 fa_dtype dtype, hipStream_t stream);

/*
 * Forward pass with a padding mask and/or a causal sliding window (local
 * attention).  Transformers' FA2 takes a 2D padding mask ("FlashAttentionとは？
 * …", section TransformersのFA2における4Dマスクの非対応); models that use
 * sliding-window attention are named in the local-LLM guide page (section on
 * models with non-standard sliding-window attention).  Arguments as in fa_fwd
 * (no fp8 descales), plus:
 *   seqlens: DEVICE int32 [B], or NULL.  Sequence b holds valid tokens in rows
 *     0 .. seqlens[b] - 1 of Q, K and V (right padding); keys past it are
 *     never seen, and its query rows past it are written as O = 0,
 *     LSE = -inf.  Values are clamped to [0, N] on the device.
 *   window: < 0 for none; >= 0 (causal only) lets query i see keys
 *     i - window .. i, i.e. window + 1 keys.
 * So query i of sequence b (i < len_b) sees keys max(0, i - window) ..
 * min(i, len_b - 1) when causal, 0 .. len_b - 1 otherwise.
 * Supported: BF16 with d = 64, 128, 256; FA_ERR_UNSUPPORTED otherwise.
 * FA_ERR_INVALID_VALUE for window >= 0 without causal, or a seqlens pointer
 * that is not 4-byte aligned or overlaps an output.
 */
fa_status fa_fwd_masked(const void* Q, const void* K, const void* V, void* O, float* LSE,
                        const int* seqlens, int window, int B, int H, int H_kv, int N, int d,
                        float scale, int causal, fa_dtype dtype, hipStream_t stream);

/*
 * Block-sparse forward: a 128 x 128 block mask decides which (query block,
 * key block) pairs are computed -- the block-sparse variant of FlashAttention
 * that "FlashAttentionとは？…" reports for 64K sequences (subsection
 * 逆伝播でL×L行列を保存せず再計算する設計).  Arguments as in fa_fwd (bf16, no
 * descales), plus:
 *   block_mask: DEVICE uint8 [H][nb][nb], nb = ceil(N / 128), shared by every
 *     sequence of the batch; a nonzero byte lets query block qb of head h see
 *     key block kb.  Query i sees key j iff block (i / 128, j / 128) is on
 *     and, when causal, j <= i.  A row that sees no key gets O = 0,
 *     LSE = -inf.  Key tiles whose blocks are off are neither loaded nor
 *     computed.
 * Supported: BF16 with d = 64, 128 (FA_ERR_UNSUPPORTED otherwise) and
 * N <= 131072 (FA_ERR_INVALID_SHAPE otherwise: a workgroup keeps its rows of
 * the mask in on-chip memory).
 */
fa_status fa_fwd_blocksparse(const void* Q, const void* K, const void* V, void* O, float* LSE,
                             const unsigned char* block_mask, int B, int H, int H_kv, int N, int d,
                             float scale, int causal, fa_dtype dtype, hipStream_t stream);

/*
 * Backward of fa_fwd_blocksparse (the same block mask): arguments and
 * workspace as in fa_bwd.  Supported: BF16 with d = 64, 128, N <= 131072 and
 * (H / H_kv) * ceil(N / 128) <= 16384.
 */
fa_status fa_bwd_blocksparse(const void* Q, const void* K, const void* V, const void* O,
                             const float* LSE, const void* dO, void* dQ, void* dK, void* dV,
                             void* workspace, size_t workspace_bytes,
                             const unsigned char* block_mask, int B, int H, int H_kv, int N, int d,
                             float scale, int causal, fa_dtype dtype, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs for this problem (0 on invalid
 * arguments).  The workspace holds two fp32 [B][H][N] arrays: D = rowsum(dO * O)
 * and the forward's LSE in base-2 units.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int H_kv, int N, int d, fa_dtype dtype);

/*
 * Backward pass by recomputation.
 *   Q, K, V, O, dO as in the forward (O and LSE are the forward's outputs for
 *   the same Q, K, V, scale and causal flag).  dQ, dK, dV have the layouts and
 *   dtype of Q, K, V; dK/dV of a GQA group are summed over its query heads.
 *   workspace: caller-owned device memory of at least
 *   fa_bwd_workspace_bytes(...) bytes, 256-byte aligned; its contents on
 *   entry do not matter and are garbage on return.
 * Supported: BF16 d=64,128,256.  FP8 has no backward (FA_ERR_UNSUPPORTED).
 */
fa_status fa_bwd(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                 const void* dO, void* dQ, void* dK, void* dV, void* workspace,
                 size_t workspace_bytes, int B, int H, int H_kv, int N, int d, float scale,
                 int causal, fa_dtype dtype, hipStream_t stream);

/*
 * fa_bwd without a workspace, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Arguments, results and errors are those of fa_bwd; the
 * per-row statistics go to a static device array of the library instead of a
 * caller workspace.  Nothing is allocated or freed by the call.
 *   Limit: fa_bwd_workspace_bytes(B, H, H_kv, N, d, dtype) <= 16 MiB
 *     (16777216 bytes; B * H * N <= 2^21 rows); larger problems return
 *     FA_ERR_WORKSPACE.
 *   Each GPU the library runs on holds its own 16 MiB array until the
 *   process ends.  Every call on one GPU uses that same array, so calls that
 *   overlap in time on one GPU (concurrent streams, or threads) race and
 *   must be serialised by the caller; calls on different GPUs do not share
 *   it.  Its contents between calls are meaningless.
 *   FA_ERR_HIP also covers a failed lookup of the array's device address.
 */
fa_status fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                         const void* dO, void* dQ, void* dK, void* dV, int B, int H, int H_kv, int N,
                         int d, float scale, int causal, fa_dtype dtype, hipStream_t stream);

/*
 * Bytes of device workspace fa_fwd_kvcache needs for this problem (0 on
 * invalid arguments or an unsupported (dtype, d)).  A pure function of its
 * arguments.
 */
size_t fa_fwd_kvcache_workspace_bytes(int B, int H, int H_kv, int N_q, int N_kv, int d,
                                      fa_dtype dtype);

/*
 * Forward pass of N_q new queries against a KV cache (decode).  In decode the
 * query side is a single token (or a few) and the cost moves to reading the
 * cache; the read is split over many workgroups, as "FlashAttentionとは？…"
 * describes for FA2's KV-cache entry point (section 短い系列の効果とデコード
 * 向け最適化の違い), and the per-chunk results are merged with their
 * logsumexps by a second kernel.
 *   Q [B][H][N_q][d]; K_cache, V_cache [B][H_kv][N_kv][d] (N_kv is the cache
 *   capacity; GQA as in fa_fwd); O [B][H][N_q][d] bf16; LSE [B][H][N_q] fp32
 *   or NULL.
 *   kv_len: DEVICE int32 [B], the number of cache rows batch b uses, or NULL
 *     for N_kv everywhere.  Values are clamped to [0, N_kv] on the device
 *     (they cannot be checked on the host without a synchronisation).
 *   The N_q queries are the last N_q positions of each sequence: with
 *   causal != 0, query i of batch b sees keys 0 .. kv_len[b] - N_q + i
 *   (bottom-right alignment); otherwise all kv_len[b] keys.  A query row that
 *   sees no key gets O = 0 and LSE = -inf.
 *   workspace: caller-owned device memory of at least
 *   fa_fwd_kvcache_workspace_bytes(...) bytes, 256-byte aligned; contents on
 *   entry do not matter and are garbage on return.
 * Supported: BF16 with d = 64, 128, 256.  Any N_q >= 1, N_kv >= 1; the split
 * pays off for small N_q (G * N_q <= 32 query rows per K/V head read once).
 */
fa_status fa_fwd_kvcache(const void* Q, const void* K_cache, const void* V_cache, const int* kv_len,
                         void* O, float* LSE, void* workspace, size_t workspace_bytes, int B, int H,
                         int H_kv, int N_q, int N_kv, int d, float scale, int causal, fa_dtype dtype,
                         hipStream_t stream);

/*
 * Backward of fa_fwd_masked (same seqlens and window, which must be the ones
 * the forward used): arguments and workspace as in fa_bwd.  Gradient rows of
 * padding positions (query rows and keys at or past seqlens[b]) are written
 * as zero.  Supported: BF16 with d = 64, 128, 256; FA_ERR_UNSUPPORTED otherwise;
 * FA_ERR_INVALID_VALUE for window >= 0 without causal or a bad seqlens
 * pointer.
 */
fa_status fa_bwd_masked(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                        const void* dO, void* dQ, void* dK, void* dV, void* workspace,
                        size_t workspace_bytes, const int* seqlens, int window, int B, int H, int H_kv,
                        int N, int d, float scale, int causal, fa_dtype dtype, hipStream_t stream);

/* 1 if a kernel exists for (dtype, d, backward != 0), else 0. */
int fa_supported(fa_dtype dtype, int d, int backward);

/* 1 if fa_fwd_kvcache has a kernel for (dtype, d), else 0. */
int fa_kvcache_supported(fa_dtype dtype, int d);

/* Static, never-NULL description of a status code. */
const char* fa_status_string(fa_status s);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
