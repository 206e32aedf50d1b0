// Host-only driver of the C ABI's argument validation, built with g++ under
// -fsanitize=address,undefined by tests/test_abi_sanitized.py (no GPU, no
// HIP runtime calls).  It links the library's own fa_api.cpp and fa_plan.cpp
// against stub launchers that record what would have been launched, and
// checks every status code the validation can return, that a valid call
// reaches exactly one launcher with the caller's sizes, and that a launch
// error maps to FA_ERR_HIP.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../exact_tiled_attention_amd/csrc/fa_kernels.hpp"
#include "../include/fa.h"

namespace fa {
// ---- stub launchers --------------------------------------------------------
static int g_calls = 0;
static const char* g_last = "";
static hipError_t g_result = hipSuccess;
static FwdParams g_fwd;
static BwdParams g_bwd;
static KvParams g_kv;

hipError_t launch_fwd_f32(int, bool, FwdParams& p, hipStream_t) { ++g_calls; g_last = "fwd_f32"; g_fwd = p; return g_result; }
hipError_t launch_fwd_bf16(int, bool, FwdParams& p, hipStream_t) { ++g_calls; g_last = "fwd_bf16"; g_fwd = p; return g_result; }
hipError_t launch_fwd_fp8(int, bool, FwdParams& p, hipStream_t) { ++g_calls; g_last = "fwd_fp8"; g_fwd = p; return g_result; }
hipError_t launch_bwd_bf16(int, bool, BwdParams& p, hipStream_t) { ++g_calls; g_last = "bwd_bf16"; g_bwd = p; return g_result; }
hipError_t launch_kvcache_bf16(int, bool, KvParams& p, hipStream_t) { ++g_calls; g_last = "kvcache"; g_kv = p; return g_result; }
static int g_scratch_lookups = 0;
hipError_t bwd_scratch(void** ptr) { ++g_scratch_lookups; *ptr = reinterpret_cast<void*>((uintptr_t)77 << 32); return hipSuccess; }
}  // namespace fa

static int failures = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

// Fake, 256-byte aligned device addresses: validation never dereferences them.
static void* A(int i) { return reinterpret_cast<void*>((uintptr_t)(i + 1) << 32); }
static const float* F(int i) { return reinterpret_cast<const float*>(A(i)); }

static fa_status fwd(const void* q, const void* k, const void* v, void* o, float* lse, const float* qs,
                     const float* ks, const float* vs, int B, int H, int Hkv, int N, int d, float scale,
                     int causal, fa_dtype dt) {
  return fa_fwd(q, k, v, o, lse, qs, ks, vs, B, H, Hkv, N, d, scale, causal, dt, nullptr);
}

static void check_forward() {
  float* lse = (float*)A(4);
  // a valid call reaches one launcher with the caller's sizes
  fa::g_calls = 0;
  EXPECT(fwd(A(0), A(1), A(2), A(3), lse, nullptr, nullptr, nullptr, 2, 8, 2, 1000, 128, 0.088f, 1,
             FA_DTYPE_BF16) == FA_OK);
  EXPECT(fa::g_calls == 1 && strcmp(fa::g_last, "fwd_bf16") == 0);
  EXPECT(fa::g_fwd.B == 2 && fa::g_fwd.H == 8 && fa::g_fwd.H_kv == 2 && fa::g_fwd.N == 1000);
  EXPECT(fabsf(fa::g_fwd.scale_log2 - 0.088f * 1.4426950408889634f) < 1e-7f);
  EXPECT(fa::g_fwd.seqlens == nullptr && fa::g_fwd.window == -1 && fa::g_fwd.block_mask == nullptr);
  EXPECT(fwd(A(0), A(1), A(2), A(3), nullptr, nullptr, nullptr, nullptr, 1, 1, 1, 1, 64, 1.f, 0,
             FA_DTYPE_F32) == FA_OK);
  EXPECT(strcmp(fa::g_last, "fwd_f32") == 0);
  EXPECT(fwd(A(0), A(1), A(2), A(3), lse, F(5), F(6), F(7), 1, 4, 4, 300, 128, 0.088f, 1,
             FA_DTYPE_FP8_E4M3) == FA_OK);
  EXPECT(strcmp(fa::g_last, "fwd_fp8") == 0 && fa::g_fwd.qs == F(5));

  const int before = fa::g_calls;
  // null pointers
  EXPECT(fwd(nullptr, A(1), A(2), A(3), lse, nullptr, nullptr, nullptr, 1, 1, 1, 16, 64, 1.f, 1, FA_DTYPE_BF16) ==
         FA_ERR_NULL_POINTER);
  EXPECT(fwd(A(0), A(1), A(2), nullptr, lse, nullptr, nullptr, nullptr, 1, 1, 1, 16, 64, 1.f, 1, FA_DTYPE_BF16) ==
         FA_ERR_NULL_POINTER);
  EXPECT(fwd(A(0), A(1), A(2), A(3), lse, F(5), nullptr, F(7), 1, 1, 1, 16, 128, 1.f, 1, FA_DTYPE_FP8_E4M3) ==
         FA_ERR_NULL_POINTER);
  // shapes
  const int bad_shapes[][5] = {{0, 1, 1, 16, 64}, {1, 0, 1, 16, 64}, {1, 1, 0, 16, 64}, {1, 1, 1, 0, 64},
                               {1, 1, 1, 16, 0}, {1, 3, 2, 16, 64}, {1, 1, 1, -5, 64}, {1, 1, 1, (1 << 28) + 1, 64},
                               {1 << 20, 1 << 10, 1, 1 << 12, 64}, {-1, 1, 1, 16, 64}};
  for (const auto& s : bad_shapes)
    EXPECT(fwd(A(0), A(1), A(2), A(3), lse, nullptr, nullptr, nullptr, s[0], s[1], s[2], s[3], s[4], 1.f, 1,
               FA_DTYPE_BF16) == FA_ERR_INVALID_SHAPE);
  // unsupported instances and dtypes
  for (int d : {32, 96, 192, 512})
    EXPECT(fwd(A(0), A(1), A(2), A(3), lse, nullptr, nullptr, nullptr, 1, 1, 1, 16, d, 1.f, 1, FA_DTYPE_BF16) ==
           FA_ERR_UNSUPPORTED);
  EXPECT(fwd(A(0), A(1), A(2), A(3), lse, nullptr, nullptr, nullptr, 1, 1, 1, 16, 128, 1.f, 1, FA_DTYPE_F32) ==
         FA_ERR_UNSUPPORTED);
  EXPECT(fwd(A(0), A(1), A(2), A(3), lse, F(5), F(6), F(7), 1, 1, 1, 16, 64, 1.f, 1, FA_DTYPE_FP8_E4M3) ==
         FA_ERR_UNSUPPORTED);
  EXPECT(fwd(A(0), A(1), A(2), A(3), lse, nullptr, nullptr, nullptr, 1, 1, 1, 16, 64, 1.f, 1, (fa_dtype)7) ==
         FA_ERR_UNSUPPORTED);
  // values: scale, descales on a non-fp8 call, alignment, aliasing
  for (float sc : {0.f, -1.f, NAN, INFINITY, -INFINITY})
    EXPECT(fwd(A(0), A(1), A(2), A(3), lse, nullptr, nullptr, nullptr, 1, 1, 1, 16, 64, sc, 1, FA_DTYPE_BF16) ==
           FA_ERR_INVALID_VALUE);
  EXPECT(fwd(A(0), A(1), A(2), A(3), lse, F(5), nullptr, nullptr, 1, 1, 1, 16, 64, 1.f, 1, FA_DTYPE_BF16) ==
         FA_ERR_INVALID_VALUE);
  EXPECT(fwd((char*)A(0) + 8, A(1), A(2), A(3), lse, nullptr, nullptr, nullptr, 1, 1, 1, 16, 64, 1.f, 1,
             FA_DTYPE_BF16) == FA_ERR_INVALID_VALUE);
  EXPECT(fwd(A(0), A(1), A(2), A(3), (float*)((char*)lse + 4), nullptr, nullptr, nullptr, 1, 1, 1, 16, 64, 1.f,
             1, FA_DTYPE_BF16) == FA_ERR_INVALID_VALUE);
  EXPECT(fwd(A(0), A(1), A(2), A(0), lse, nullptr, nullptr, nullptr, 1, 1, 1, 16, 64, 1.f, 1, FA_DTYPE_BF16) ==
         FA_ERR_INVALID_VALUE);                                    // O is Q
  EXPECT(fwd(A(0), A(1), A(2), (char*)A(1) + 1024, lse, nullptr, nullptr, nullptr, 1, 1, 1, 16, 64, 1.f, 1,
             FA_DTYPE_BF16) == FA_ERR_INVALID_VALUE);               // O inside K
  EXPECT(fwd(A(0), A(1), A(2), A(3), (float*)A(3), nullptr, nullptr, nullptr, 1, 1, 1, 16, 64, 1.f, 1,
             FA_DTYPE_BF16) == FA_ERR_INVALID_VALUE);               // LSE is O
  EXPECT(fa::g_calls == before);                                  // nothing was launched

  // a launch error is reported as FA_ERR_HIP
  fa::g_result = hipErrorInvalidConfiguration;
  EXPECT(fwd(A(0), A(1), A(2), A(3), lse, nullptr, nullptr, nullptr, 1, 1, 1, 16, 64, 1.f, 1, FA_DTYPE_BF16) ==
         FA_ERR_HIP);
  fa::g_result = hipSuccess;
}

static void check_masked_and_sparse() {
  float* lse = (float*)A(4);
  EXPECT(fa_fwd_masked(A(0), A(1), A(2), A(3), lse, (const int*)A(5), 100, 2, 4, 2, 500, 128, 0.1f, 1,
                       FA_DTYPE_BF16, nullptr) == FA_OK);
  EXPECT(fa::g_fwd.window == 100 && fa::g_fwd.seqlens == (const int*)A(5));
  EXPECT(fa_fwd_masked(A(0), A(1), A(2), A(3), lse, nullptr, 100, 2, 4, 2, 500, 128, 0.1f, 0, FA_DTYPE_BF16,
                       nullptr) == FA_ERR_INVALID_VALUE);           // a window is causal
  EXPECT(fa_fwd_masked(A(0), A(1), A(2), A(3), lse, (const int*)((char*)A(5) + 2), -1, 2, 4, 2, 500, 128, 0.1f,
                       1, FA_DTYPE_BF16, nullptr) == FA_ERR_INVALID_VALUE);
  EXPECT(fa_fwd_masked(A(0), A(1), A(2), A(3), lse, nullptr, -1, 2, 4, 2, 500, 64, 0.1f, 1, FA_DTYPE_F32,
                       nullptr) == FA_ERR_UNSUPPORTED);
  const unsigned char* bm = (const unsigned char*)A(6);
  EXPECT(fa_fwd_blocksparse(A(0), A(1), A(2), A(3), lse, bm, 1, 4, 2, 1000, 128, 0.1f, 1, FA_DTYPE_BF16,
                            nullptr) == FA_OK);
  EXPECT(fa::g_fwd.block_mask == bm && fa::g_fwd.nb == 8);
  EXPECT(fa_fwd_blocksparse(A(0), A(1), A(2), A(3), lse, nullptr, 1, 4, 2, 1000, 128, 0.1f, 1, FA_DTYPE_BF16,
                            nullptr) == FA_ERR_NULL_POINTER);
  EXPECT(fa_fwd_blocksparse(A(0), A(1), A(2), A(3), lse, bm, 1, 4, 2, 131072 + 128, 128, 0.1f, 1,
                            FA_DTYPE_BF16, nullptr) == FA_ERR_INVALID_SHAPE);
  EXPECT(fa_fwd_blocksparse(A(0), A(1), A(2), A(3), lse, bm, 1, 4, 2, 1000, 256, 0.1f, 1, FA_DTYPE_BF16,
                            nullptr) == FA_ERR_UNSUPPORTED);
}

static void check_backward() {
  const int B = 2, H = 4, Hkv = 2, N = 300, d = 64;
  const size_t need = fa_bwd_workspace_bytes(B, H, Hkv, N, d, FA_DTYPE_BF16);
  EXPECT(need >= 2 * (size_t)B * H * N * 4 && need % 256 == 0);
  EXPECT(fa_bwd_workspace_bytes(0, H, Hkv, N, d, FA_DTYPE_BF16) == 0);
  EXPECT(fa_bwd_workspace_bytes(B, 3, 2, N, d, FA_DTYPE_BF16) == 0);
  auto bwd = [&](void* ws, size_t wsb, int dd, fa_dtype dt, void* dq = A(6)) {
    return fa_bwd(A(0), A(1), A(2), A(3), (const float*)A(4), A(5), dq, A(7), A(8), ws, wsb, B, H, Hkv, N, dd,
                  0.125f, 1, dt, nullptr);
  };
  fa::g_calls = 0;
  EXPECT(bwd(A(9), need, d, FA_DTYPE_BF16) == FA_OK);
  EXPECT(fa::g_calls == 1 && strcmp(fa::g_last, "bwd_bf16") == 0);
  EXPECT(fa::g_bwd.delta == (float*)A(9) && (char*)fa::g_bwd.lse2 == (char*)A(9) + need / 2);
  EXPECT(fabsf(fa::g_bwd.scale - 0.125f) == 0.f);
  EXPECT(bwd(nullptr, need, d, FA_DTYPE_BF16) == FA_ERR_WORKSPACE);
  EXPECT(bwd(A(9), need - 1, d, FA_DTYPE_BF16) == FA_ERR_WORKSPACE);
  EXPECT(bwd((char*)A(9) + 16, need, d, FA_DTYPE_BF16) == FA_ERR_WORKSPACE);
  EXPECT(bwd(A(9), need, 128, FA_DTYPE_FP8_E4M3) == FA_ERR_UNSUPPORTED);
  EXPECT(bwd(A(9), need, 64, FA_DTYPE_F32) == FA_ERR_UNSUPPORTED);
  EXPECT(bwd(A(9), need, 96, FA_DTYPE_BF16) == FA_ERR_UNSUPPORTED);
  EXPECT(bwd(A(9), need, d, FA_DTYPE_BF16, A(0)) == FA_ERR_INVALID_VALUE);   // dQ is Q
  EXPECT(bwd(A(9), need, d, FA_DTYPE_BF16, A(7)) == FA_ERR_INVALID_VALUE);   // dQ is dK
  EXPECT(bwd(A(6), need, d, FA_DTYPE_BF16) == FA_ERR_INVALID_VALUE);         // workspace is dQ
  EXPECT(fa_bwd(A(0), A(1), A(2), A(3), nullptr, A(5), A(6), A(7), A(8), A(9), need, B, H, Hkv, N, d, 0.125f, 1,
                FA_DTYPE_BF16, nullptr) == FA_ERR_NULL_POINTER);
  EXPECT(fa::g_calls == 1);
  EXPECT(fa_bwd_masked(A(0), A(1), A(2), A(3), (const float*)A(4), A(5), A(6), A(7), A(8), A(9), need, nullptr,
                       10, B, H, Hkv, N, d, 0.125f, 0, FA_DTYPE_BF16, nullptr) == FA_ERR_INVALID_VALUE);
  EXPECT(fa_bwd_blocksparse(A(0), A(1), A(2), A(3), (const float*)A(4), A(5), A(6), A(7), A(8), A(9), need,
                            (const unsigned char*)A(10), B, H, Hkv, N, 256, 0.125f, 1, FA_DTYPE_BF16,
                            nullptr) == FA_ERR_UNSUPPORTED);
  // a GQA group's mask column must fit on chip: (H / H_kv) * ceil(N / 128) <= 16384
  EXPECT(fa_bwd_blocksparse(A(0), A(1), A(2), A(3), (const float*)A(4), A(5), A(6), A(7), A(8), A(9), 1ull << 40,
                            (const unsigned char*)A(10), 1, 64, 1, 65536, 64, 0.125f, 1, FA_DTYPE_BF16,
                            nullptr) == FA_ERR_INVALID_SHAPE);
}

static void check_noalloc() {
  // the static scratch replaces the workspace; problems beyond it are refused
  fa::g_calls = 0;
  fa::g_scratch_lookups = 0;
  EXPECT(fa_bwd_noalloc(A(0), A(1), A(2), A(3), (const float*)A(4), A(5), A(6), A(7), A(8), 2, 4, 2, 300, 64,
                        0.125f, 1, FA_DTYPE_BF16, nullptr) == FA_OK);
  EXPECT(fa::g_calls == 1 && fa::g_scratch_lookups == 1);
  EXPECT(fa::g_bwd.delta == (float*)((uintptr_t)77 << 32));
  EXPECT(fa_bwd_workspace_bytes(1, 1, 1, 1 << 21, 64, FA_DTYPE_BF16) <= fa::kBwdScratchBytes);
  EXPECT(fa_bwd_noalloc(A(0), A(1), A(2), A(3), (const float*)A(4), A(5), A(6), A(7), A(8), 1, 1, 1, 1 << 21,
                        64, 0.125f, 1, FA_DTYPE_BF16, nullptr) == FA_OK);
  EXPECT(fa_bwd_noalloc(A(0), A(1), A(2), A(3), (const float*)A(4), A(5), A(6), A(7), A(8), 1, 1, 1,
                        (1 << 21) + 1, 64, 0.125f, 1, FA_DTYPE_BF16, nullptr) == FA_ERR_WORKSPACE);
  EXPECT(fa_bwd_noalloc(A(0), A(1), A(2), A(3), (const float*)A(4), A(5), A(6), A(7), A(8), 2, 4, 2, 300, 128,
                        0.125f, 1, FA_DTYPE_FP8_E4M3, nullptr) == FA_ERR_UNSUPPORTED);
  EXPECT(fa_bwd_noalloc(A(0), A(1), A(2), A(3), (const float*)A(4), A(5), A(0), A(7), A(8), 2, 4, 2, 300, 64,
                        0.125f, 1, FA_DTYPE_BF16, nullptr) == FA_ERR_INVALID_VALUE);
  EXPECT(fa::g_calls == 2 && fa::g_scratch_lookups == 2);      // refused calls look nothing up
}

static void check_kvcache() {
  const size_t need = fa_fwd_kvcache_workspace_bytes(8, 32, 8, 1, 32768, 128, FA_DTYPE_BF16);
  EXPECT(need > 0 && need == fa_fwd_kvcache_workspace_bytes(8, 32, 8, 1, 32768, 128, FA_DTYPE_BF16));
  EXPECT(fa_fwd_kvcache_workspace_bytes(8, 32, 8, 1, 32768, 96, FA_DTYPE_BF16) == 0);
  EXPECT(fa_fwd_kvcache_workspace_bytes(8, 32, 8, 1, 32768, 128, FA_DTYPE_F32) == 0);
  fa::g_calls = 0;
  EXPECT(fa_fwd_kvcache(A(0), A(1), A(2), (const int*)A(3), A(4), (float*)A(5), A(6), need, 8, 32, 8, 1, 32768,
                        128, 0.088f, 1, FA_DTYPE_BF16, nullptr) == FA_OK);
  EXPECT(fa::g_calls == 1 && fa::g_kv.G == 4 && fa::g_kv.Nkv == 32768 && fa::g_kv.part_lse == (float*)A(6));
  EXPECT(fa_fwd_kvcache(A(0), A(1), A(2), nullptr, A(4), (float*)A(5), A(6), need - 1, 8, 32, 8, 1, 32768, 128,
                        0.088f, 1, FA_DTYPE_BF16, nullptr) == FA_ERR_WORKSPACE);
  EXPECT(fa_fwd_kvcache(A(0), A(1), A(2), (const int*)((char*)A(3) + 1), A(4), (float*)A(5), A(6), need, 8, 32,
                        8, 1, 32768, 128, 0.088f, 1, FA_DTYPE_BF16, nullptr) == FA_ERR_INVALID_VALUE);
  EXPECT(fa_fwd_kvcache(A(0), A(1), A(2), nullptr, A(4), (float*)A(5), A(6), need, 8, 32, 8, 0, 32768, 128,
                        0.088f, 1, FA_DTYPE_BF16, nullptr) == FA_ERR_INVALID_SHAPE);
  EXPECT(fa::g_calls == 1);
}

static void check_strings() {
  for (int s = 0; s <= 6; ++s) {
    const char* t = fa_status_string((fa_status)s);
    EXPECT(t != nullptr && strncmp(t, "FA_", 3) == 0);
  }
  EXPECT(strcmp(fa_status_string((fa_status)99), "unknown fa_status") == 0);
  EXPECT(fa_supported(FA_DTYPE_BF16, 128, 0) && !fa_supported(FA_DTYPE_FP8_E4M3, 128, 1));
}

int main() {
  check_forward();
  check_masked_and_sparse();
  check_backward();
  check_noalloc();
  check_kvcache();
  check_strings();
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("abi_check: all expectations hold\n");
  return 0;
}
