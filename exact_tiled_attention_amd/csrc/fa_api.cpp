// The C ABI of libfa.so: argument validation, then one launch sequence on the
// caller's stream.  Validation finishes before any HIP runtime call, so every
// error code can be produced without a device.
#include <math.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "fa_kernels.hpp"

namespace {

constexpr int kMaxN = 1 << 28;

size_t elem_bytes(fa_dtype t) { return t == FA_DTYPE_F32 ? 4 : (t == FA_DTYPE_BF16 ? 2 : 1); }
size_t out_bytes(fa_dtype t) { return t == FA_DTYPE_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// The kernels fold the scale into the exponent's FMA and mask with -inf
// scores, which is only sound for a positive scale (attention's is 1/sqrt(d)).
bool valid_scale(float s) { return isfinite(s) && s > 0.f; }

bool valid_dtype(int t) { return t == FA_DTYPE_F32 || t == FA_DTYPE_BF16 || t == FA_DTYPE_FP8_E4M3; }

// Shape checks shared by both directions; also guards every size product.
fa_status check_shape(int B, int H, int H_kv, int N, int d) {
  if (B <= 0 || H <= 0 || H_kv <= 0 || N <= 0 || d <= 0) return FA_ERR_INVALID_SHAPE;
  if (H % H_kv != 0) return FA_ERR_INVALID_SHAPE;
  if (N > kMaxN) return FA_ERR_INVALID_SHAPE;
  const unsigned long long rows = (unsigned long long)B * H * N;
  if (rows > (1ull << 40) || rows * (unsigned long long)d > (1ull << 44)) return FA_ERR_INVALID_SHAPE;
  // grid sizes (work items of 32-row tiles at worst) must fit a 32-bit int
  if ((unsigned long long)B * H * ((N + 31) / 32) > 0x7fffffffull) return FA_ERR_INVALID_SHAPE;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_supported(fa_dtype dtype, int d, int backward) {
  if (!valid_dtype(dtype)) return 0;
  if (backward) return dtype == FA_DTYPE_BF16 && (d == 64 || d == 128 || d == 256);
  switch (dtype) {
    case FA_DTYPE_F32: return d == 64;
    case FA_DTYPE_BF16: return d == 64 || d == 128 || d == 256;
    case FA_DTYPE_FP8_E4M3: return d == 128;
  }
  return 0;
}

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL_POINTER: return "FA_ERR_NULL_POINTER: a required pointer is NULL";
    case FA_ERR_INVALID_SHAPE: return "FA_ERR_INVALID_SHAPE: non-positive size, H not a multiple of H_kv, or size overflow";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: no kernel for this (dtype, head dim, direction)";
    case FA_ERR_INVALID_VALUE: return "FA_ERR_INVALID_VALUE: scale not finite and positive, misaligned pointer, aliasing output, or misplaced descale";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing, misaligned or too small (fa_bwd_noalloc: the problem needs more than its static scratch)";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported an error at launch";
  }
  return "unknown fa_status";
}

fa_status fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                 const float* q_descale, const float* k_descale, const float* v_descale,
                 int B, int H, int H_kv, int N, int d, float scale, int causal,
                 fa_dtype dtype, hipStream_t stream) {
  if (!Q || !K || !V || !O) return FA_ERR_NULL_POINTER;
  if (!valid_dtype(dtype)) return FA_ERR_UNSUPPORTED;
  const bool fp8 = dtype == FA_DTYPE_FP8_E4M3;
  if (fp8 && (!q_descale || !k_descale || !v_descale)) return FA_ERR_NULL_POINTER;
  if (fa_status s = check_shape(B, H, H_kv, N, d); s != FA_OK) return s;
  if (!fa_supported(dtype, d, 0)) return FA_ERR_UNSUPPORTED;
  if (!valid_scale(scale)) return FA_ERR_INVALID_VALUE;
  if (!fp8 && (q_descale || k_descale || v_descale)) return FA_ERR_INVALID_VALUE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
    return FA_ERR_INVALID_VALUE;
  if (fp8 && (!aligned16(q_descale) || !aligned16(k_descale) || !aligned16(v_descale)))
    return FA_ERR_INVALID_VALUE;
  const size_t nq = (size_t)B * H * N * d, nkv = (size_t)B * H_kv * N * d;
  const size_t ob = nq * out_bytes(dtype), lb = LSE ? (size_t)B * H * N * 4 : 0;
  const size_t eb = elem_bytes(dtype);
  if (overlap(O, ob, Q, nq * eb) || overlap(O, ob, K, nkv * eb) || overlap(O, ob, V, nkv * eb) ||
      overlap(LSE, lb, Q, nq * eb) || overlap(LSE, lb, K, nkv * eb) || overlap(LSE, lb, V, nkv * eb) ||
      overlap(LSE, lb, O, ob))
    return FA_ERR_INVALID_VALUE;

  fa::FwdParams p{};
  p.q = Q; p.k = K; p.v = V; p.o = O; p.lse = LSE;
  p.qs = q_descale; p.ks = k_descale; p.vs = v_descale;
  p.B = B; p.H = H; p.H_kv = H_kv; p.N = N;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.seqlens = nullptr;
  p.window = -1;
  hipError_t e;
  switch (dtype) {
    case FA_DTYPE_F32: e = fa::launch_fwd_f32(d, causal != 0, p, stream); break;
    case FA_DTYPE_BF16: e = fa::launch_fwd_bf16(d, causal != 0, p, stream); break;
    default: e = fa::launch_fwd_fp8(d, causal != 0, p, stream); break;
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_masked(const void* Q, const void* K, const void* V, void* O, float* LSE,
                        const int* seqlens, int window, int B, int H, int H_kv, int N, int d,
                        float scale, int causal, fa_dtype dtype, hipStream_t stream) {
  if (!Q || !K || !V || !O) return FA_ERR_NULL_POINTER;
  if (!valid_dtype(dtype)) return FA_ERR_UNSUPPORTED;
  if (fa_status s = check_shape(B, H, H_kv, N, d); s != FA_OK) return s;
  if (dtype != FA_DTYPE_BF16 || !fa_supported(dtype, d, 0)) return FA_ERR_UNSUPPORTED;
  if (!valid_scale(scale)) return FA_ERR_INVALID_VALUE;
  if (window >= 0 && !causal) return FA_ERR_INVALID_VALUE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE) ||
      (reinterpret_cast<uintptr_t>(seqlens) & 3u))
    return FA_ERR_INVALID_VALUE;
  const size_t eb = elem_bytes(dtype);
  const size_t nq = (size_t)B * H * N * d * eb, nkv = (size_t)B * H_kv * N * d * eb;
  const size_t ob = (size_t)B * H * N * d * out_bytes(dtype), lb = LSE ? (size_t)B * H * N * 4 : 0;
  const size_t sb = seqlens ? (size_t)B * 4 : 0;
  const void* ins[] = {Q, K, V, seqlens};
  const size_t insz[] = {nq, nkv, nkv, sb};
  for (int j = 0; j < 4; ++j)
    if (overlap(O, ob, ins[j], insz[j]) || overlap(LSE, lb, ins[j], insz[j])) return FA_ERR_INVALID_VALUE;
  if (overlap(LSE, lb, O, ob)) return FA_ERR_INVALID_VALUE;

  fa::FwdParams p{};
  p.q = Q; p.k = K; p.v = V; p.o = O; p.lse = LSE;
  p.B = B; p.H = H; p.H_kv = H_kv; p.N = N;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.seqlens = seqlens;
  p.window = window < 0 ? -1 : window;
  const hipError_t e = fa::launch_fwd_bf16(d, causal != 0, p, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_blocksparse(const void* Q, const void* K, const void* V, void* O, float* LSE,
                             const unsigned char* block_mask, int B, int H, int H_kv, int N, int d,
                             float scale, int causal, fa_dtype dtype, hipStream_t stream) {
  if (!Q || !K || !V || !O || !block_mask) return FA_ERR_NULL_POINTER;
  if (!valid_dtype(dtype)) return FA_ERR_UNSUPPORTED;
  if (fa_status s = check_shape(B, H, H_kv, N, d); s != FA_OK) return s;
  if (dtype != FA_DTYPE_BF16 || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
  if (!valid_scale(scale)) return FA_ERR_INVALID_VALUE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
    return FA_ERR_INVALID_VALUE;
  const size_t nb = ((size_t)N + 127) / 128;
  if (nb > 1024) return FA_ERR_INVALID_SHAPE;   // block masks cover N <= 131072
  const size_t eb = elem_bytes(dtype);
  const size_t nq = (size_t)B * H * N * d * eb, nkv = (size_t)B * H_kv * N * d * eb;
  const size_t ob = nq, lb = LSE ? (size_t)B * H * N * 4 : 0, mb = (size_t)H * nb * nb;
  const void* ins[] = {Q, K, V, block_mask};
  const size_t insz[] = {nq, nkv, nkv, mb};
  for (int j = 0; j < 4; ++j)
    if (overlap(O, ob, ins[j], insz[j]) || overlap(LSE, lb, ins[j], insz[j])) return FA_ERR_INVALID_VALUE;
  if (overlap(LSE, lb, O, ob)) return FA_ERR_INVALID_VALUE;

  fa::FwdParams p{};
  p.q = Q; p.k = K; p.v = V; p.o = O; p.lse = LSE;
  p.B = B; p.H = H; p.H_kv = H_kv; p.N = N;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.seqlens = nullptr;
  p.window = -1;
  p.block_mask = block_mask;
  p.nb = (int)nb;
  const hipError_t e = fa::launch_fwd_bf16(d, causal != 0, p, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_bytes(int B, int H, int H_kv, int N, int d, fa_dtype dtype) {
  if (!valid_dtype(dtype) || check_shape(B, H, H_kv, N, d) != FA_OK) return 0;
  const size_t row_stats = ((size_t)B * H * N * sizeof(float) + 255) & ~(size_t)255;
  return 2 * row_stats;   // D = rowsum(dO * O), then LSE in base-2 units
}

// Validation and launch of every backward entry point.  With `noalloc` the
// workspace arguments are ignored: the statistics go to the library's static
// device scratch, after the same checks (and the size limit of the scratch).
static fa_status bwd_common(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                            const void* dO, void* dQ, void* dK, void* dV, void* workspace,
                            size_t workspace_bytes, const int* seqlens, int window,
                            const unsigned char* block_mask, int B, int H, int H_kv,
                            int N, int d, float scale, int causal, fa_dtype dtype, hipStream_t stream,
                            bool noalloc = false) {
  if (!Q || !K || !V || !O || !LSE || !dO || !dQ || !dK || !dV) return FA_ERR_NULL_POINTER;
  if (!valid_dtype(dtype)) return FA_ERR_UNSUPPORTED;
  if (fa_status s = check_shape(B, H, H_kv, N, d); s != FA_OK) return s;
  if (!fa_supported(dtype, d, 1)) return FA_ERR_UNSUPPORTED;
  if (!valid_scale(scale)) return FA_ERR_INVALID_VALUE;
  if (window >= 0 && !causal) return FA_ERR_INVALID_VALUE;
  const void* ptrs[] = {Q, K, V, O, LSE, dO, dQ, dK, dV};
  for (const void* q : ptrs)
    if (!aligned16(q)) return FA_ERR_INVALID_VALUE;
  if (reinterpret_cast<uintptr_t>(seqlens) & 3u) return FA_ERR_INVALID_VALUE;
  const size_t need = fa_bwd_workspace_bytes(B, H, H_kv, N, d, dtype);
  if (noalloc) {
    if (need > fa::kBwdScratchBytes) return FA_ERR_WORKSPACE;
    workspace = nullptr;   // resolved below, after every check
    workspace_bytes = need;
  } else if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u)) {
    return FA_ERR_WORKSPACE;
  }
  const size_t eb = elem_bytes(dtype);
  const size_t nq = (size_t)B * H * N * d * eb, nkv = (size_t)B * H_kv * N * d * eb;
  const size_t nl = (size_t)B * H * N * 4;
  const size_t nbk = ((size_t)N + 127) / 128;
  const void* ins[] = {Q, K, V, O, LSE, dO, seqlens, block_mask};
  const size_t insz[] = {nq, nkv, nkv, nq, nl, nq, seqlens ? (size_t)B * 4 : 0,
                         block_mask ? (size_t)H * nbk * nbk : 0};
  void* outs[] = {dQ, dK, dV, workspace};
  const size_t outsz[] = {nq, nkv, nkv, need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 8; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j])) return FA_ERR_INVALID_VALUE;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return FA_ERR_INVALID_VALUE;
  }

  if (noalloc && fa::bwd_scratch(&workspace) != hipSuccess) return FA_ERR_HIP;

  fa::BwdParams p{};
  p.q = Q; p.k = K; p.v = V; p.o = O; p.lse = LSE; p.dout = dO;
  p.dq = dQ; p.dk = dK; p.dv = dV;
  p.delta = (float*)workspace;
  p.lse2 = (float*)((char*)workspace + need / 2);
  p.B = B; p.H = H; p.H_kv = H_kv; p.N = N;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.seqlens = seqlens;
  p.window = window < 0 ? -1 : window;
  p.block_mask = block_mask;
  p.nb = (int)nbk;
  const hipError_t e = fa::launch_bwd_bf16(d, causal != 0, p, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_bwd(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                 const void* dO, void* dQ, void* dK, void* dV, void* workspace,
                 size_t workspace_bytes, int B, int H, int H_kv, int N, int d, float scale,
                 int causal, fa_dtype dtype, hipStream_t stream) {
  return bwd_common(Q, K, V, O, LSE, dO, dQ, dK, dV, workspace, workspace_bytes, nullptr, -1, nullptr, B, H,
                    H_kv, N, d, scale, causal, dtype, stream);
}

fa_status fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                         const void* dO, void* dQ, void* dK, void* dV, int B, int H, int H_kv, int N, int d,
                         float scale, int causal, fa_dtype dtype, hipStream_t stream) {
  return bwd_common(Q, K, V, O, LSE, dO, dQ, dK, dV, nullptr, 0, nullptr, -1, nullptr, B, H, H_kv, N, d, scale,
                    causal, dtype, stream, /*noalloc=*/true);
}

fa_status fa_bwd_masked(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                        const void* dO, void* dQ, void* dK, void* dV, void* workspace,
                        size_t workspace_bytes, const int* seqlens, int window, int B, int H, int H_kv,
                        int N, int d, float scale, int causal, fa_dtype dtype, hipStream_t stream) {
  return bwd_common(Q, K, V, O, LSE, dO, dQ, dK, dV, workspace, workspace_bytes, seqlens, window, nullptr, B,
                    H, H_kv, N, d, scale, causal, dtype, stream);
}

fa_status fa_bwd_blocksparse(const void* Q, const void* K, const void* V, const void* O,
                             const float* LSE, const void* dO, void* dQ, void* dK, void* dV,
                             void* workspace, size_t workspace_bytes,
                             const unsigned char* block_mask, int B, int H, int H_kv, int N, int d,
                             float scale, int causal, fa_dtype dtype, hipStream_t stream) {
  if (!block_mask) return FA_ERR_NULL_POINTER;
  if (valid_dtype(dtype) && d == 256) return FA_ERR_UNSUPPORTED;
  // the flags of a key block's column for a GQA group fit 16 KB of LDS
  if (H_kv > 0 && H % H_kv == 0 && N > 0 && ((size_t)N + 127) / 128 * (H / H_kv) > 16384)
    return FA_ERR_INVALID_SHAPE;
  if (N > 0 && ((size_t)N + 127) / 128 > 1024) return FA_ERR_INVALID_SHAPE;
  return bwd_common(Q, K, V, O, LSE, dO, dQ, dK, dV, workspace, workspace_bytes, nullptr, -1, block_mask, B,
                    H, H_kv, N, d, scale, causal, dtype, stream);
}

int fa_kvcache_supported(fa_dtype dtype, int d) {
  return dtype == FA_DTYPE_BF16 && (d == 64 || d == 128 || d == 256);
}

size_t fa_fwd_kvcache_workspace_bytes(int B, int H, int H_kv, int N_q, int N_kv, int d,
                                      fa_dtype dtype) {
  if (!valid_dtype(dtype) || !fa_kvcache_supported(dtype, d)) return 0;
  if (check_shape(B, H, H_kv, N_q, d) != FA_OK || check_shape(B, H_kv, H_kv, N_kv, d) != FA_OK) return 0;
  const fa::KvPlan plan = fa::kv_plan(B, H, H_kv, N_q, N_kv, d);
  return plan.max_tiles > 0x7fffffffll || plan.W > 0x7fffffffll ? 0 : plan.ws_bytes;
}

fa_status fa_fwd_kvcache(const void* Q, const void* K_cache, const void* V_cache, const int* kv_len,
                         void* O, float* LSE, void* workspace, size_t workspace_bytes, int B, int H,
                         int H_kv, int N_q, int N_kv, int d, float scale, int causal, fa_dtype dtype,
                         hipStream_t stream) {
  if (!Q || !K_cache || !V_cache || !O) return FA_ERR_NULL_POINTER;
  if (!valid_dtype(dtype)) return FA_ERR_UNSUPPORTED;
  if (fa_status s = check_shape(B, H, H_kv, N_q, d); s != FA_OK) return s;
  if (fa_status s = check_shape(B, H_kv, H_kv, N_kv, d); s != FA_OK) return s;
  // one combine workgroup per query row
  if ((unsigned long long)B * H * N_q > 0x7fffffffull) return FA_ERR_INVALID_SHAPE;
  if (!fa_kvcache_supported(dtype, d)) return FA_ERR_UNSUPPORTED;
  if (!valid_scale(scale)) return FA_ERR_INVALID_VALUE;
  if (!aligned16(Q) || !aligned16(K_cache) || !aligned16(V_cache) || !aligned16(O) || !aligned16(LSE) ||
      (reinterpret_cast<uintptr_t>(kv_len) & 3u))
    return FA_ERR_INVALID_VALUE;
  const fa::KvPlan plan = fa::kv_plan(B, H, H_kv, N_q, N_kv, d);
  // tile and wave indices are 32-bit
  if (plan.max_tiles > 0x7fffffffll || plan.W > 0x7fffffffll) return FA_ERR_INVALID_SHAPE;
  if (!workspace || workspace_bytes < plan.ws_bytes || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return FA_ERR_WORKSPACE;
  const size_t eb = elem_bytes(dtype);
  const size_t nq = (size_t)B * H * N_q * d * eb, nkv = (size_t)B * H_kv * N_kv * d * eb;
  const size_t ob = (size_t)B * H * N_q * d * out_bytes(dtype), lb = LSE ? (size_t)B * H * N_q * 4 : 0;
  const size_t klb = kv_len ? (size_t)B * 4 : 0;
  const void* ins[] = {Q, K_cache, V_cache, kv_len};
  const size_t insz[] = {nq, nkv, nkv, klb};
  void* outs[] = {O, LSE, workspace};
  const size_t outsz[] = {ob, lb, plan.ws_bytes};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j])) return FA_ERR_INVALID_VALUE;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return FA_ERR_INVALID_VALUE;
  }

  fa::KvParams p{};
  p.q = Q; p.k = K_cache; p.v = V_cache; p.kv_len = kv_len; p.o = O; p.lse = LSE;
  p.part_lse = (float*)workspace;
  p.part_o = (float*)((char*)workspace + plan.lse_bytes);
  p.B = B; p.H = H; p.H_kv = H_kv; p.Nq = N_q; p.Nkv = N_kv;
  p.G = plan.G; p.R = plan.R; p.n_rg = plan.n_rg; p.R_pad = plan.R_pad;
  p.upb = H_kv * plan.n_rg;
  p.W = (int)plan.W; p.nw = plan.nw;
  p.scale_log2 = scale * 1.4426950408889634f;
  const hipError_t e = fa::launch_kvcache_bf16(d, causal != 0, p, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
