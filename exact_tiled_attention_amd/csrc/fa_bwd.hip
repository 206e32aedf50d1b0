// Backward attention kernels for gfx950 (bf16 MFMA), by recomputation.
//
// The forward keeps only O and one logsumexp per row; the backward rebuilds
// the probabilities tile by tile from Q, K and that statistic instead of
// storing the N x N matrix ("FlashAttentionとは？…", subsection 逆伝播でL×L行列を
// 保存せず再計算する設計).  With P_ij = exp(scale q_i.k_j - LSE_i):
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  D_i = sum_d dO_id O_id,
//   dQ = scale dS K,  dK = scale dS^T Q.
// (D_i = rowsum(dO o O) equals rowsum(P o dP) because O = P V.)
//
// Three launches:
//   bwd_delta  D = rowsum(dO o O)                       -- HBM-bound sweep
//   bwd_dkdv   one workgroup per 128 keys of a K/V head; loops over the
//              query tiles (and the query heads of a GQA group) that see
//              those keys; dK and dV accumulate in registers, no atomics
//   bwd_dq     one workgroup per 128 queries; loops over the key tiles they
//              see; dQ accumulates in registers
// Recomputing S and dP in both kernels costs 7 tile GEMMs instead of 5 but
// keeps every gradient deterministic and free of atomic traffic.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

// ============================================================ delta ======
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdParams p) {
  constexpr int LPR = D / 8;                  // lanes per row (8 bf16 each)
  constexpr int RPB = 256 / LPR;              // rows per block
  const int row = blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  const int rows = p.B * p.H * p.N;
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 o = *(const bf16x8*)((const bf16*)p.o + (size_t)row * D + part * 8);
    const bf16x8 d = *(const bf16x8*)((const bf16*)p.dout + (size_t)row * D + part * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)d[e], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (row < rows && part == 0) p.delta[row] = acc;
}

// ============================================================= dK dV ======
template <int D, bool CAUSAL>
struct DkdvCfg {
  static constexpr int NW = 4, NT = 256;
  static constexpr int BKV = NW * 32;         // keys per workgroup (32 per wave)
  static constexpr int BQ = 64;               // queries per staged tile
  static constexpr int QS = D + 8;            // row stride of Q / dO (bf16)
  static constexpr int TS = BQ + 4;           // row stride of Q^T / dO^T (bf16)
  static constexpr int ROWB = BQ * QS;        // elements
  static constexpr int TRB = D * TS;
  static constexpr int BUF_E = 2 * ROWB + 2 * TRB;       // bf16 elements
  static constexpr int BUF_B = BUF_E * 2 + 2 * BQ * 4;    // + lse2, delta (fp32)
  static constexpr int NBLK = (BQ / 4) * (D / 8);         // 4 rows x 8 cols blocks
  static constexpr int BPT = (NBLK + NT - 1) / NT;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdParams p) {
  using C = DkdvCfg<D, CAUSAL>;
  constexpr int BKV = C::BKV, BQ = C::BQ, NT = C::NT;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * C::BUF_B];

  const int tid = threadIdx.x;
  const int wid = tid >> 6, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const WorkItem wi = map_work(blockIdx.x, p.total, p.n_tiles, p.remap);
  const int kt = p.n_tiles - 1 - wi.qt;       // lightest-last: small key tiles see most queries
  const int N = p.N;
  const int bkv = wi.bh;                      // (b, kv head)
  const int b = bkv / p.H_kv, kvh = bkv - b * p.H_kv;
  const int G = p.H / p.H_kv;
  const int k_first = kt * BKV;
  const int kw0 = k_first + wid * 32;         // this wave's first key
  const int mykey = kw0 + lr;                 // this lane's key (column of S)

  const bf16* kgp = (const bf16*)p.k + (size_t)bkv * N * D;
  const bf16* vgp = (const bf16*)p.v + (size_t)bkv * N * D;

  // K and V operands (B of S = Q K^T and of dP = dO V^T): lane holds its key.
  bf16x8 kr[D / 16], vr[D / 16];
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) {
    bf16x8 xk = {}, xv = {};
    if (mykey < N) {
      xk = *(const bf16x8*)(kgp + (size_t)mykey * D + kb * 16 + 8 * g);
      xv = *(const bf16x8*)(vgp + (size_t)mykey * D + kb * 16 + 8 * g);
    }
    kr[kb] = xk;
    vr[kb] = xv;
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  const int n_qt = (N + BQ - 1) / BQ;
  const int qt_start = CAUSAL ? k_first / BQ : 0;
  const int per_head = n_qt - qt_start;
  const int n_iter = G * per_head;
  const float c = p.scale_log2;

  i32x4 qreg[C::BPT][4], doreg[C::BPT][4];
  float st_val = 0.f;
  auto load_tile = [&](int it_idx) {
    const int gi = it_idx / per_head;
    const int qt = qt_start + (it_idx - gi * per_head);
    const size_t bh = (size_t)b * p.H + kvh * G + gi;
    const int qrow0 = qt * BQ;
    const bf16* qgp = (const bf16*)p.q + bh * N * D;
    const bf16* dgp = (const bf16*)p.dout + bh * N * D;
#pragma unroll
    for (int it = 0; it < C::BPT; ++it) {
      const int blk = tid + it * NT;
      const int rq = blk % (BQ / 4), cc = blk / (BQ / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = qrow0 + rq * 4 + r;
        i32x4 xq = {}, xd = {};
        if (blk < C::NBLK && row < N) {
          xq = *(const i32x4*)(qgp + (size_t)row * D + cc * 8);
          xd = *(const i32x4*)(dgp + (size_t)row * D + cc * 8);
        }
        qreg[it][r] = xq;
        doreg[it][r] = xd;
      }
    }
    // threads 0..BQ-1 fetch LSE (as log2 units), BQ..2BQ-1 fetch D
    if (tid < 2 * BQ) {
      const int row = qrow0 + (tid % BQ);
      if (tid < BQ)
        st_val = row < N ? p.lse[bh * N + row] * kLog2e : INFINITY;  // padded rows get P = 0
      else
        st_val = row < N ? p.delta[bh * N + row] : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
    bf16* base = (bf16*)(smem + buf * C::BUF_B);
    bf16* qs = base;
    bf16* ds = base + C::ROWB;
    bf16* qt = base + 2 * C::ROWB;
    bf16* dt = qt + C::TRB;
    float* stat = (float*)(base + C::BUF_E);
#pragma unroll
    for (int it = 0; it < C::BPT; ++it) {
      const int blk = tid + it * NT;
      if (blk < C::NBLK) {
        const int rq = blk % (BQ / 4), cc = blk / (BQ / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          *(i32x4*)(qs + (rq * 4 + r) * C::QS + cc * 8) = qreg[it][r];
          *(i32x4*)(ds + (rq * 4 + r) * C::QS + cc * 8) = doreg[it][r];
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int col = cc * 8 + w * 2;
          uint32_t a0 = qreg[it][0][w], a1 = qreg[it][1][w], a2 = qreg[it][2][w], a3 = qreg[it][3][w];
          *(i32x2*)(qt + col * C::TS + rq * 4) = i32x2{(int)perm_lo16(a0, a1), (int)perm_lo16(a2, a3)};
          *(i32x2*)(qt + (col + 1) * C::TS + rq * 4) = i32x2{(int)perm_hi16(a0, a1), (int)perm_hi16(a2, a3)};
          a0 = doreg[it][0][w]; a1 = doreg[it][1][w]; a2 = doreg[it][2][w]; a3 = doreg[it][3][w];
          *(i32x2*)(dt + col * C::TS + rq * 4) = i32x2{(int)perm_lo16(a0, a1), (int)perm_lo16(a2, a3)};
          *(i32x2*)(dt + (col + 1) * C::TS + rq * 4) = i32x2{(int)perm_hi16(a0, a1), (int)perm_hi16(a2, a3)};
        }
      }
    }
    if (tid < 2 * BQ) stat[tid] = st_val;
  };

  if (n_iter > 0) {
    load_tile(0);
    store_tile(0);
  }
  for (int it_idx = 0; it_idx < n_iter; ++it_idx) {
    __syncthreads();
    if (it_idx + 1 < n_iter) load_tile(it_idx + 1);
    const int gi = it_idx / per_head;
    const int qrow0 = (qt_start + (it_idx - gi * per_head)) * BQ;
    const bf16* base = (const bf16*)(smem + (it_idx & 1) * C::BUF_B);
    const bf16* qs = base;
    const bf16* ds = base + C::ROWB;
    const bf16* qt = base + 2 * C::ROWB;
    const bf16* dt = qt + C::TRB;
    const float* lse2 = (const float*)(base + C::BUF_E);
    const float* dl = lse2 + BQ;
#pragma unroll
    for (int qb = 0; qb < BQ / 32; ++qb) {
      const int qq0 = qrow0 + qb * 32;
      if (CAUSAL && qq0 + 31 < kw0) continue;   // every query precedes every key
      // ---- S = Q K^T (lane: key column, registers: query rows) -------------
      f32x16 s = {};
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) {
        const bf16x8 a = *(const bf16x8*)(qs + (qb * 32 + lr) * C::QS + kb * 16 + 8 * g);
        s = mfma_bf16(a, kr[kb], s);
      }
      // ---- P = exp2(S c - LSE2) -------------------------------------------
      float lrow[16], drow[16];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 lv = *(const f32x4*)(lse2 + qb * 32 + 8 * a4 + 4 * g);
        const f32x4 dvv = *(const f32x4*)(dl + qb * 32 + 8 * a4 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lrow[4 * a4 + e] = lv[e];
          drow[4 * a4 + e] = dvv[e];
        }
      }
      const bool need_mask = CAUSAL && qq0 < kw0 + 31;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = fast_exp2(fmaf(s[r], c, -lrow[r]));
        if (need_mask) {
          const int q = qq0 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (mykey > q) e = 0.f;
        }
        s[r] = e;
      }
      // ---- dV^T += dO^T P ----------------------------------------------------
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = s[half * 8 + e];
        const bf16x8 pb = pack_bf16x8(pv);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16* row = dt + (db * 32 + lr) * C::TS + qb * 32 + 16 * half + 4 * g;
          const bf16x4 lo = *(const bf16x4*)row;
          const bf16x4 hi = *(const bf16x4*)(row + 8);
          dv[db] = mfma_bf16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb, dv[db]);
        }
      }
      // ---- dP = dO V^T; dS = P (dP - D) --------------------------------------
      f32x16 dp = {};
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) {
        const bf16x8 a = *(const bf16x8*)(ds + (qb * 32 + lr) * C::QS + kb * 16 + 8 * g);
        dp = mfma_bf16(a, vr[kb], dp);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = s[r] * (dp[r] - drow[r]);
      // ---- dK^T += Q^T dS ----------------------------------------------------
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = s[half * 8 + e];
        const bf16x8 pb = pack_bf16x8(pv);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16* row = qt + (db * 32 + lr) * C::TS + qb * 32 + 16 * half + 4 * g;
          const bf16x4 lo = *(const bf16x4*)row;
          const bf16x4 hi = *(const bf16x4*)(row + 8);
          dk[db] = mfma_bf16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb, dk[db]);
        }
      }
    }
    if (it_idx + 1 < n_iter) store_tile((it_idx + 1) & 1);
  }

  if (mykey < N) {
    bf16* dkr = (bf16*)p.dk + ((size_t)bkv * N + mykey) * D;
    bf16* dvr = (bf16*)p.dv + ((size_t)bkv * N + mykey) * D;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int col = db * 32 + 8 * a + 4 * g;
        *(i32x2*)(dkr + col) = i32x2{(int)pack_bf16(dk[db][4 * a] * sc, dk[db][4 * a + 1] * sc),
                                     (int)pack_bf16(dk[db][4 * a + 2] * sc, dk[db][4 * a + 3] * sc)};
        *(i32x2*)(dvr + col) = i32x2{(int)pack_bf16(dv[db][4 * a], dv[db][4 * a + 1]),
                                     (int)pack_bf16(dv[db][4 * a + 2], dv[db][4 * a + 3])};
      }
  }
}

// ================================================================ dQ ======
template <int D, bool CAUSAL>
struct DqCfg {
  static constexpr int NW = 4, NT = 256;
  static constexpr int BR = NW * 32;          // queries per workgroup
  static constexpr int BC = 64;               // keys per tile
  static constexpr int RS = D + 8;            // row stride of K / V (bf16)
  static constexpr int TS = BC + 4;           // row stride of K^T (bf16)
  static constexpr int ROWB = BC * RS;
  static constexpr int TRB = D * TS;
  static constexpr int BUF_E = 2 * ROWB + TRB;
  static constexpr int NBLK = (BC / 4) * (D / 8);
  static constexpr int BPT = (NBLK + NT - 1) / NT;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdParams p) {
  using C = DqCfg<D, CAUSAL>;
  constexpr int BR = C::BR, BC = C::BC, NT = C::NT;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * C::BUF_E];

  const int tid = threadIdx.x;
  const int wid = tid >> 6, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const WorkItem wi = map_work(blockIdx.x, p.total, p.n_tiles, p.remap);
  const int N = p.N;
  const int b = wi.bh / p.H, h = wi.bh - b * p.H;
  const int bkv = b * p.H_kv + h / (p.H / p.H_kv);
  const int q_first = wi.qt * BR;
  const int q0 = q_first + wid * 32;
  const int myq = q0 + lr;
  const bf16* qgp = (const bf16*)p.q + (size_t)wi.bh * N * D;
  const bf16* dgp = (const bf16*)p.dout + (size_t)wi.bh * N * D;
  const bf16* kgp = (const bf16*)p.k + (size_t)bkv * N * D;
  const bf16* vgp = (const bf16*)p.v + (size_t)bkv * N * D;

  bf16x8 qr[D / 16], dor[D / 16];
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) {
    bf16x8 xq = {}, xd = {};
    if (myq < N) {
      xq = *(const bf16x8*)(qgp + (size_t)myq * D + kb * 16 + 8 * g);
      xd = *(const bf16x8*)(dgp + (size_t)myq * D + kb * 16 + 8 * g);
    }
    qr[kb] = xq;
    dor[kb] = xd;
  }
  const float lse2 = myq < N ? p.lse[(size_t)wi.bh * N + myq] * kLog2e : INFINITY;
  const float dlt = myq < N ? p.delta[(size_t)wi.bh * N + myq] : 0.f;
  const float c = p.scale_log2;
  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq[i] = f32x16{};

  const int kv_end = CAUSAL ? min(N, q_first + BR) : N;
  const int n_tiles = (kv_end + BC - 1) / BC;

  i32x4 kreg[C::BPT][4], vreg[C::BPT][4];
  auto load_tile = [&](int j) {
    const int key0 = j * BC;
#pragma unroll
    for (int it = 0; it < C::BPT; ++it) {
      const int blk = tid + it * NT;
      const int rq = blk % (BC / 4), cc = blk / (BC / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + rq * 4 + r;
        i32x4 xk = {}, xv = {};
        if (blk < C::NBLK && key < N) {
          xk = *(const i32x4*)(kgp + (size_t)key * D + cc * 8);
          xv = *(const i32x4*)(vgp + (size_t)key * D + cc * 8);
        }
        kreg[it][r] = xk;
        vreg[it][r] = xv;
      }
    }
  };
  auto store_tile = [&](int buf) {
    bf16* ks = smem + buf * C::BUF_E;
    bf16* vs = ks + C::ROWB;
    bf16* kt = vs + C::ROWB;
#pragma unroll
    for (int it = 0; it < C::BPT; ++it) {
      const int blk = tid + it * NT;
      if (blk < C::NBLK) {
        const int rq = blk % (BC / 4), cc = blk / (BC / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          *(i32x4*)(ks + (rq * 4 + r) * C::RS + cc * 8) = kreg[it][r];
          *(i32x4*)(vs + (rq * 4 + r) * C::RS + cc * 8) = vreg[it][r];
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int col = cc * 8 + w * 2;
          const uint32_t a0 = kreg[it][0][w], a1 = kreg[it][1][w];
          const uint32_t a2 = kreg[it][2][w], a3 = kreg[it][3][w];
          *(i32x2*)(kt + col * C::TS + rq * 4) = i32x2{(int)perm_lo16(a0, a1), (int)perm_lo16(a2, a3)};
          *(i32x2*)(kt + (col + 1) * C::TS + rq * 4) = i32x2{(int)perm_hi16(a0, a1), (int)perm_hi16(a2, a3)};
        }
      }
    }
  };

  load_tile(0);
  store_tile(0);
  for (int j = 0; j < n_tiles; ++j) {
    __syncthreads();
    if (j + 1 < n_tiles) load_tile(j + 1);
    const int key0 = j * BC;
    const bool active = !CAUSAL || key0 <= q0 + 31;
    if (active) {
      const bf16* ks = smem + (j & 1) * C::BUF_E;
      const bf16* vs = ks + C::ROWB;
      const bf16* kt = vs + C::ROWB;
      const bool need_mask = (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > q0);
      f32x16 pt[BC / 32];
#pragma unroll
      for (int kb32 = 0; kb32 < BC / 32; ++kb32) {
        // S^T = K Q^T and dP^T = V dO^T (lane: query column, registers: keys)
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb) {
          const bf16x8 ak = *(const bf16x8*)(ks + (kb32 * 32 + lr) * C::RS + kb * 16 + 8 * g);
          s = mfma_bf16(ak, qr[kb], s);
        }
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb) {
          const bf16x8 av = *(const bf16x8*)(vs + (kb32 * 32 + lr) * C::RS + kb * 16 + 8 * g);
          dp = mfma_bf16(av, dor[kb], dp);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = fast_exp2(fmaf(s[r], c, -lse2));
          if (need_mask) {
            const int key = key0 + kb32 * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if ((CAUSAL && key > myq) || key >= N) e = 0.f;
          }
          s[r] = e * (dp[r] - dlt);
        }
        pt[kb32] = s;
      }
      // ---- dQ^T += K^T dS^T ---------------------------------------------------
#pragma unroll
      for (int kb32 = 0; kb32 < BC / 32; ++kb32)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = pt[kb32][half * 8 + e];
          const bf16x8 pb = pack_bf16x8(pv);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const bf16* row = kt + (db * 32 + lr) * C::TS + kb32 * 32 + 16 * half + 4 * g;
            const bf16x4 lo = *(const bf16x4*)row;
            const bf16x4 hi = *(const bf16x4*)(row + 8);
            dq[db] = mfma_bf16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb, dq[db]);
          }
        }
    }
    if (j + 1 < n_tiles) store_tile((j + 1) & 1);
  }

  if (myq < N) {
    bf16* dqr = (bf16*)p.dq + ((size_t)wi.bh * N + myq) * D;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *(i32x2*)(dqr + db * 32 + 8 * a + 4 * g) =
            i32x2{(int)pack_bf16(dq[db][4 * a] * sc, dq[db][4 * a + 1] * sc),
                  (int)pack_bf16(dq[db][4 * a + 2] * sc, dq[db][4 * a + 3] * sc)};
  }
}

// ========================================================= launchers ======
template <int D, bool CAUSAL>
static hipError_t launch_bwd(BwdParams p, hipStream_t s) {
  {
    constexpr int RPB = 256 / (D / 8);
    const long rows = (long)p.B * p.H * p.N;
    hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s, p);
  }
  {
    BwdParams q = p;
    q.n_tiles = (p.N + DkdvCfg<D, CAUSAL>::BKV - 1) / DkdvCfg<D, CAUSAL>::BKV;
    q.total = p.B * p.H_kv * q.n_tiles;
    q.remap = (q.total % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(q.total), dim3(256), 0, s, q);
  }
  {
    BwdParams q = p;
    q.n_tiles = (p.N + DqCfg<D, CAUSAL>::BR - 1) / DqCfg<D, CAUSAL>::BR;
    q.total = p.B * p.H * q.n_tiles;
    q.remap = (q.total % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(q.total), dim3(256), 0, s, q);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(int d, bool causal, BwdParams& p, hipStream_t s) {
  switch (d) {
    case 64: return causal ? launch_bwd<64, true>(p, s) : launch_bwd<64, false>(p, s);
    case 128: return causal ? launch_bwd<128, true>(p, s) : launch_bwd<128, false>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
