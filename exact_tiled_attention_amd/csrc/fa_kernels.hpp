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
  int remap;           // 1: XCD-contiguous work map
  float scale_log2;    // scale * log2(e)
};

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
  int remap;
  float scale;         // softmax scale
  float scale_log2;    // scale * log2(e)
};

// Each returns hipSuccess or the launch error; unsupported shapes never reach
// them (the C ABI validates first).
hipError_t launch_fwd_f32(int d, bool causal, FwdParams& p, hipStream_t s);
hipError_t launch_fwd_bf16(int d, bool causal, FwdParams& p, hipStream_t s);
hipError_t launch_fwd_fp8(int d, bool causal, FwdParams& p, hipStream_t s);
hipError_t launch_bwd_bf16(int d, bool causal, BwdParams& p, hipStream_t s);

}  // namespace fa
