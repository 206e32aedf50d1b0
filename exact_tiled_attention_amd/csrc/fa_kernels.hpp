// Kernel parameter blocks and the host-side launchers the C ABI calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;          // may be null
  const float* qs;     // fp8 block scales (null otherwise)
  const float* ks;
  const float* vs;
  int B, H, H_kv, N;
  int n_qt;            // q-tiles per head
  int total;           // B * H * n_qt work items (= grid size)
  int remap;           // XCD work map: 0 none, 1 contiguous, 2 groups dealt in turn
  int group_items;     // items of one (batch, K/V head) group
  float scale_log2;    // scale * log2(e)
  const int* seqlens;  // [B] valid rows per sequence (padding mask), or null
  int window;          // causal sliding window: query i sees keys i - window .. i; < 0: none
  const unsigned char* block_mask;   // [H][nb][nb] 128 x 128 block mask, or null
  int nb;              // ceil(N / 128)
};

// True when a forward call carries a padding mask, a sliding window or a
// block mask.
inline bool masked(const FwdParams& p) {
  return p.seqlens != nullptr || p.window >= 0 || p.block_mask != nullptr;
}

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;        // workspace: rowsum(dO * O), [B][H][N]
  float* lse2;         // workspace: LSE * log2(e), [B][H][N]
  int B, H, H_kv, N;
  int n_tiles;         // tiles per head of the kernel being launched
  int total;
  int remap;           // as in FwdParams
  int group_items;
  float scale;         // softmax scale
  float scale_log2;    // scale * log2(e)
  const int* seqlens;  // [B] valid rows per sequence (padding mask), or null
  int window;          // causal sliding window as in FwdParams; < 0: none
  const unsigned char* block_mask;   // as in FwdParams
  int nb;
};

// Attention of N_q new queries against a KV cache, split over the cache.
struct KvParams {
  const void* q;       // [B][H][Nq][d]
  const void* k;       // [B][H_kv][Nkv][d]
  const void* v;
  const int* kv_len;   // [B] rows of the cache in use, or null (all Nkv)
  void* o;             // [B][H][Nq][d]
  float* lse;          // [B][H][Nq] or null
  float* part_lse;     // workspace: [W][R_pad] partial logsumexp per wave (base 2, scaled)
  float* part_o;       // workspace: [W][R_pad][d] partial outputs per wave (normalised)
  int B, H, H_kv, Nq, Nkv;
  int G, R, n_rg, R_pad; // heads per group, rows per group (G*Nq), 32-row groups, min(R, 32)
  int upb;             // units per batch: H_kv * n_rg
  int W, nw;           // waves of the split grid, waves per workgroup
  float scale_log2;
};

// Shape of the decode split kernel per head dim: waves per workgroup and LDS
// stages (32-key tiles) per wave, sized so one workgroup's stages fill about
// 128 KB of the CU's 160 KB of LDS; and the fewest 32-key tiles a wave is
// given (small problems use fewer waves).
template <int D>
struct KvCfg;
template <> struct KvCfg<64> { static constexpr int NW = 4, NST = 4; };
template <> struct KvCfg<128> { static constexpr int NW = 4, NST = 2; };
template <> struct KvCfg<256> { static constexpr int NW = 2, NST = 2; };
constexpr int kKvMinTiles = 2;

// Launch shape and workspace of a KV-cache problem: a pure function of the shape.
struct KvPlan {
  int G, R, n_rg, R_pad, nw;
  long long W;         // waves of the split grid
  size_t lse_bytes;    // offset of part_o in the workspace (256-aligned)
  size_t ws_bytes;     // total workspace
  long long max_tiles; // 32-key tiles of the whole problem at full caches
};
KvPlan kv_plan(int B, int H, int H_kv, int Nq, int Nkv, int d);

// Size of the static device scratch behind fa_bwd_noalloc (per GPU), and the
// lookup of its device address on the current device.
constexpr size_t kBwdScratchBytes = 16u << 20;
hipError_t bwd_scratch(void** ptr);

// Enqueue one kernel on stream s and return that launch's own status.
// (hipLaunchKernel reports the launch it makes; hipGetLastError after a
// triple-chevron launch would also return an error left behind by earlier,
// unrelated work on the calling thread.)
template <typename P>
inline hipError_t launch_kernel(void (*kernel)(P), dim3 grid, dim3 block, hipStream_t s, const P& p) {
  void* args[] = {const_cast<P*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, s);
}

// Each returns hipSuccess or the launch error; unsupported shapes never reach
// them (the C ABI validates first).
hipError_t launch_fwd_f32(int d, bool causal, FwdParams& p, hipStream_t s);
hipError_t launch_fwd_bf16(int d, bool causal, FwdParams& p, hipStream_t s);
hipError_t launch_fwd_fp8(int d, bool causal, FwdParams& p, hipStream_t s);
hipError_t launch_bwd_bf16(int d, bool causal, BwdParams& p, hipStream_t s);
hipError_t launch_kvcache_bf16(int d, bool causal, KvParams& p, hipStream_t s);

}  // namespace fa
