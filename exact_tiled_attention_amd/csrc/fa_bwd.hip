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
//   bwd_prep   D = rowsum(dO o O) and LSE in base-2 units  -- HBM-bound sweep
//   bwd_dkdv   one workgroup per 128 keys of a K/V head; loops over the
//              query tiles (and the query heads of a GQA group) that see
//              those keys; dK and dV accumulate in registers, no atomics
//   bwd_dq     one workgroup per 128 queries; loops over the key tiles they
//              see; dQ accumulates in registers
// Recomputing S and dP in both kernels costs 7 tile GEMMs instead of 5 but
// keeps every gradient deterministic and free of atomic traffic.
//
// Tiles move HBM -> LDS by DMA (buffer_load ... lds, rows past the end read
// as zero), row-swizzled so they can be read both as rows (the A operand of
// Q K^T, dO V^T, K Q^T, V dO^T) and transposed with ds_read_b64_tr_b16 (the A
// operand of Q^T dS, dO^T P and K^T dS^T) without bank conflicts.
#include <atomic>
#include <type_traits>

#include "fa_common.hpp"
#include "fa_kernels.hpp"


namespace fa {

// ====================================================== static scratch ===
// Device memory of fa_bwd_noalloc: the backward's per-row statistics (D and
// the base-2 LSE, kBwdScratchBytes at most) live in this file-scope array
// instead of a caller workspace.  Each GPU holds its own copy for as long as
// the process runs, and every call on that GPU shares it, so calls that
// overlap on one GPU race.  Nothing in it needs clearing: the prep kernel
// writes every row the other two kernels read.
static __device__ __align__(256) unsigned char scratch[kBwdScratchBytes];

// Device address of this GPU's copy.  In host code `scratch` names a host-side
// stand-in, not device memory, so kernels get the address from
// hipGetSymbolAddress, looked up once per device with that device current.
hipError_t bwd_scratch(void** ptr) {
  static std::atomic<void*> cache[64];
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    cache[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

// ============================================================ prep ======
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
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
  if (row < rows && part == 0) {
    p.delta[row] = acc;
    p.lse2[row] = p.lse[row] * kLog2e;
  }
}

// Valid rows of sequence b under a padding mask (N without one).
template <bool MASK>
__device__ __forceinline__ int valid_len(const BwdParams& p, int b) {
  return MASK && p.seqlens ? min(max(p.seqlens[b], 0), p.N) : p.N;
}
// Block-sparse: the dK/dV kernel keeps, in LDS, one bit per step (query tile
// and GQA head) of its key block's column of the mask (H / H_kv) * 2 nb <=
// kMaxMaskBits: 4 KB, so its occupancy is unchanged) and steps from one
// set bit to the next; the dQ kernel runs over a list of its key tiles that
// are on.
constexpr int kMaxMaskBits = 32768;
// A 64-bit LDS word every lane of the wave reads at one address, made
// scalar (so loops over it stay uniform).
__device__ __forceinline__ unsigned long long lds_u64_uniform(const unsigned long long* a) {
  const unsigned long long w = *a;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)w);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(w >> 32));
  return ((unsigned long long)hi << 32) | lo;
}
// Zero gradient rows (bf16) for padding positions; lanes l and l ^ 32 each
// write half of the row.
__device__ __forceinline__ void zero_row(void* base, size_t row, int g, int d) {
  bf16* r = (bf16*)base + row * d;
  for (int c = 4 * g; c < d; c += 8) *(i32x2*)(r + c) = i32x2{0, 0};
}

// Offsets of the transposing read of a row-major tile: for 16-row block
// base b (a multiple of 16), second = 0/1 selects rows b+0..7 / b+8..15 of the
// block (4 rows per lane group), column block db selects 32 columns.  Lane i
// of each 16-lane group receives 4 consecutive rows of one column.
template <int RB>
__device__ __forceinline__ int tr_off(int lane, int second, int db) {
  const int s16 = lane & 15, G = lane >> 4;
  const int row = 8 * second + 4 * (G >> 1) + (s16 >> 2);
  const int u = db * 4 + 2 * (G & 1) + ((s16 & 3) >> 1);
  return row * RB + rt_swz<RB>(row, u) * 16 + (s16 & 1) * 8;
}

// ============================================================= dK dV ======
template <int D>
struct DkdvCfg {
  static constexpr int NW = 4, NT = 256;
  static constexpr int BKV = NW * 32;         // keys per workgroup (32 per wave)
  static constexpr int BQ = 64;               // queries per staged tile
  static constexpr int RB = D * 2;
  static constexpr int QTILE = BQ * RB;
  static constexpr int IPW = QTILE / 1024 / NW;
  static constexpr int STAGE = 2 * QTILE + 2 * BQ * 4;   // Q, dO, LSE2, D
  static_assert(IPW >= 1, "tile too small for the DMA split");
};

// d = 128 keeps K, V, dK and dV of 32 keys in registers (192 a lane) at two
// waves a SIMD (faster than one wave a SIMD: 710 vs 649 TFLOP/s causal at
// B=2, H=16, N=8192); the causal and masked instances still spill two values.
// With MASK (padding mask and/or sliding window, as in the forward) a key
// block sees only the query tiles whose rows are valid and whose windows
// reach it, and keys past the valid length get zero gradients.
template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D > 128 ? 1 : 2, D > 128 ? 1 : 2)))
void bwd_dkdv_kernel(BwdParams p) {
  using C = DkdvCfg<D>;
  constexpr int BKV = C::BKV, BQ = C::BQ, RB = C::RB, IPW = C::IPW;
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[C::STAGE];

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const WorkItem wi = map_work(blockIdx.x, p.total, p.n_tiles, p.remap, p.group_items);
  const int kt = p.n_tiles - 1 - wi.qt;       // small key tiles (most queries) first
  const int N = p.N;
  const int bkv = wi.bh;                      // (b, kv head)
  const int b = bkv / p.H_kv, kvh = bkv - b * p.H_kv;
  const int G = p.H / p.H_kv;
  const int k_first = kt * BKV;
  const int kw0 = k_first + wid * 32;         // this wave's first key
  const int mykey = kw0 + lr;                 // this lane's key (column of S)
  const int L = valid_len<MASK>(p, b);
  const int W = MASK ? p.window : -1;
  if (MASK && k_first >= L) {                 // every key of the block is padding
    if (mykey < N) {
      zero_row(p.dk, (size_t)bkv * N + mykey, g, D);
      zero_row(p.dv, (size_t)bkv * N + mykey, g, D);
    }
    return;
  }

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

  const int dma0_ = dma_base<RB, kSwzRt>(wid * IPW, lane);
  // LDS read offsets of block 0 (the others are formed per tile, below)
  const int roff0 = lr * RB + rt_swz<RB>(lr, g) * 16;
  const int troff0 = tr_off<RB>(lane, 0, 0);

  const int n_qt = (L + BQ - 1) / BQ;        // tiles holding valid query rows
  const int qt_start = CAUSAL ? k_first / BQ : 0;
  // with a window, queries past the block's last key + W see none of it
  const int qt_stop = MASK && W >= 0 ? min(n_qt, (k_first + BKV - 1 + W) / BQ + 1) : n_qt;
  const int per_head = max(0, qt_stop - qt_start);
  const int n_iter = G * per_head;
  const float c = p.scale_log2;
  // Step it takes query tile qt_stop - 1 - it / G of group head it % G: the
  // latest query tiles first, the group's heads innermost.  So all running
  // workgroups of one (batch, K/V head) read the same Q and dO tile at the
  // same time, and each tile comes from HBM once and from L2 after that
  // (taking each head's tiles upward from the diagonal instead spread them
  // over many tiles at once: 6x the compulsory reads on the GQA prefill
  // shape, against 1x for the dQ kernel).
  auto step_tile = [&](int it, int& gi, int& qt) {
    const int qi = it / G;
    gi = it - qi * G;
    qt = qt_stop - 1 - qi;
  };

  // Block-sparse: the key block is one 128-key block (BKV = 128).  Bit it
  // is set when step it's tile is in a query block that has the key block
  // on for its head, and steps visit only the set bits.
  static_assert(!MASK || BKV == 128, "block masks assume one key block per workgroup");
  const bool bs = MASK && p.block_mask;
  __shared__ unsigned long long bm_col[MASK ? kMaxMaskBits / 64 : 1];
  if (bs) {
    for (int base = 0; base < n_iter; base += 256) {   // uniform trip count: every lane votes
      const int i = base + tid;
      bool on = false;
      if (i < n_iter) {
        int gi, qt;
        step_tile(i, gi, qt);
        on = p.block_mask[((size_t)(kvh * G + gi) * p.nb + ((qt * BQ) >> 7)) * p.nb + (k_first >> 7)] != 0;
      }
      const unsigned long long bits = __ballot(on);
      if ((tid & 63) == 0) bm_col[(base + tid) >> 6] = bits;
    }
    __syncthreads();
  }
  // first step >= it whose tile is on (n_iter if none)
  auto next_on = [&](int it) -> int {
    if (!bs || it >= n_iter) return it;
    int word = it >> 6;
    unsigned long long w = lds_u64_uniform(bm_col + word) & (~0ull << (it & 63));
    while (w == 0) {
      if (++word >= (n_iter + 63) >> 6) return n_iter;
      w = lds_u64_uniform(bm_col + word);
    }
    return word * 64 + __builtin_ctzll(w);
  };
  auto issue = [&](int it_idx, unsigned char* st) {
    int gi, qt;
    step_tile(it_idx, gi, qt);
    const int dma0 = D == 128 ? dma_base<RB, kSwzRt>(wid * IPW,
                                                      __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)))
                              : dma0_;
    const size_t bh = (size_t)b * p.H + kvh * G + gi;
    const int row0 = qt * BQ;
    const int rows = min(L - row0, BQ);          // rows past the valid ones read as zero
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const bf16*)p.q + (bh * N + row0) * D, rows * RB);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc((const bf16*)p.dout + (bh * N + row0) * D, rows * RB);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      dma16_buf<0>(rq, dma_off<RB, kSwzRt>(dma0, i), st + (wid * IPW + i) * 1024);
      dma16_buf<0>(rd, dma_off<RB, kSwzRt>(dma0, i), st + C::QTILE + (wid * IPW + i) * 1024);
    }
    if (wid < 2) {   // wave 0: LSE2 of the tile's rows, wave 1: D (padded rows read 0)
      const float* src = (wid == 0 ? p.lse2 : p.delta) + bh * N + row0;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, rows * 4);
      dma4_buf(rs, lane * 4, st + 2 * C::QTILE + wid * BQ * 4);
    }
  };

  // MASKED false: a step no query of which precedes a key of the block (no
  // element needs the mask, so the step carries no mask code at all)
  auto consume = [&](int it_idx, const unsigned char* st, auto MASKED) __attribute__((always_inline)) {
    int gi, qt;
    step_tile(it_idx, gi, qt);
    const int qrow0 = qt * BQ;
    // The read offsets from one register each: block kb's, or section sec
    // and column block db's, are block 0's XOR a constant (the swizzle is
    // XOR-linear in bits no lane bit shares, as for the DMA copies); made
    // opaque once per tile so they are formed here instead of kept live.
    // (at d = 128 the bases are formed from the lane id per tile: three
    // registers fewer across the loop, which kept the kernel from spilling)
    int rb0 = roff0, tb0 = troff0;
    if constexpr (D == 128) {
      const int ln = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      rb0 = (ln & 31) * RB + rt_swz<RB>(ln & 31, ln >> 5) * 16;
      tb0 = tr_off<RB>(ln, 0, 0);
    }
    asm volatile("" : "+v"(rb0), "+v"(tb0));
    auto RO = [&](int kb) { return rb0 ^ (rt_swz<RB>(0, 2 * kb) * 16); };
    auto TO = [&](int sec, int db) { return (tb0 ^ (rt_swz<RB>(8 * sec, db * 4) * 16)) + sec * 8 * RB; };
    const unsigned char* qs = st;
    const unsigned char* ds = st + C::QTILE;
    const float* lse2 = (const float*)(st + 2 * C::QTILE);
    const float* dl = lse2 + BQ;
    // (at d >= 128 the two 32-query halves run one after the other: unrolled,
    // their temporaries do not fit next to K, V, dK and dV; at d = 128 that
    // and the offsets formed per tile took the spills from 44 to 8 bytes and
    // the GQA prefill backward from 565 to 632 TFLOP/s)
#pragma unroll (D >= 128 ? 1 : BQ / 32)
    for (int qb = 0; qb < BQ / 32; ++qb) {
      const int qq0 = qrow0 + qb * 32;
      if (CAUSAL && qq0 + 31 < kw0) continue;   // every query precedes every key
      if (MASK && (qq0 >= L || (W >= 0 && qq0 > kw0 + 31 + W))) continue;   // padding, or past every window
      // ---- S = Q K^T and dP = dO V^T (lane: key column, registers: query rows)
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) {
        const bf16x8 aq = *(const bf16x8*)(qs + qb * 32 * RB + RO(kb));
        const bf16x8 ad = *(const bf16x8*)(ds + qb * 32 * RB + RO(kb));
        s = mfma_bf16(aq, kr[kb], s);
        dp = mfma_bf16(ad, vr[kb], dp);
      }
      // ---- P = exp2(S c - LSE2), dS = P (dP - D) -------------------------------
      // (the row statistics are read four rows at a time, as the registers use them)
      const bool need_mask = bool(MASKED) && ((CAUSAL && qq0 < kw0 + 31) ||
                                              (MASK && (qq0 + 31 >= L || (W >= 0 && qq0 + 31 > kw0 + W))));
      const int lim = mykey - qq0 - 4 * g;     // query row offset must be >= this
      const int top = MASK ? min(L - 1, W >= 0 ? mykey + W : L - 1) - qq0 - 4 * g : 0;   // ... and <= this
      uint32_t pw[8], sw[8];
      // (at d = 64, two copies behind a wave-uniform branch: as one, the
      // compiler turns the mask into a compare and a select per element on
      // every tile; at d = 128 the second copy costs registers, and spills)
      auto p_ds = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4 lv = *(const f32x4*)(lse2 + qb * 32 + 8 * a4 + 4 * g);
          const f32x4 dvv = *(const f32x4*)(dl + qb * 32 + 8 * a4 + 4 * g);
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            float pe[2], se[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int r = 4 * a4 + 2 * h2 + e;
              float pv = fast_exp2(fmaf(s[r], c, -lv[2 * h2 + e]));
              if (bool(masked) && ((CAUSAL && (8 * (r >> 2) + (r & 3)) < lim) ||
                                   (MASK && (8 * (r >> 2) + (r & 3)) > top)))
                pv = 0.f;
              pe[e] = pv;
              se[e] = pv * (dp[r] - dvv[2 * h2 + e]);
            }
            pw[2 * a4 + h2] = pack_bf16(pe[0], pe[1]);
            sw[2 * a4 + h2] = pack_bf16(se[0], se[1]);
          }
        }
      };
      if constexpr (D <= 64) {
        if (need_mask) p_ds(std::true_type{});
        else p_ds(std::false_type{});
      } else {
        p_ds(need_mask);
      }
      // ---- dV^T += dO^T P,  dK^T += Q^T dS (transposed operands by tr reads) ---
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 pb = __builtin_bit_cast(bf16x8, i32x4{(int)pw[4 * half], (int)pw[4 * half + 1],
                                                              (int)pw[4 * half + 2], (int)pw[4 * half + 3]});
        const bf16x8 sb = __builtin_bit_cast(bf16x8, i32x4{(int)sw[4 * half], (int)sw[4 * half + 1],
                                                              (int)sw[4 * half + 2], (int)sw[4 * half + 3]});
        const int rb = (qb * 32 + 16 * half) * RB;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x4 dlo = lds_read_tr16(ds + rb + TO(0, db));
          const bf16x4 dhi = lds_read_tr16(ds + rb + TO(1, db));
          const bf16x4 qlo = lds_read_tr16(qs + rb + TO(0, db));
          const bf16x4 qhi = lds_read_tr16(qs + rb + TO(1, db));
          dv[db] = mfma_bf16(__builtin_shufflevector(dlo, dhi, 0, 1, 2, 3, 4, 5, 6, 7), pb, dv[db]);
          dk[db] = mfma_bf16(__builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7), sb, dk[db]);
        }
      }
    }
  };

  if constexpr (MASK) {
    // (without a block mask the steps are 0, 1, .., n_iter - 1)
    int cur = next_on(0);
    if (cur < n_iter) issue(cur, stage0);
    while (cur < n_iter) {
      int nxt = next_on(cur + 1);
      wait_vmem();
      __syncthreads();
      if (nxt < n_iter) issue(nxt, stage1);
      consume(cur, stage0, std::true_type{});
      cur = nxt;
      if (cur >= n_iter) break;
      nxt = next_on(cur + 1);
      wait_vmem();
      __syncthreads();
      if (nxt < n_iter) issue(nxt, stage0);
      consume(cur, stage1, std::true_type{});
      cur = nxt;
    }
  } else {
    // Steps from it_split on may hold queries before a key of the block (the
    // causal diagonal: query tiles at or below qt_m, visited last); the ones
    // before it run a copy of the step without mask code.  (it_split even, so
    // both loops start on stage 0.  At d = 128 the second copy spills and
    // measured 2-4% slower: one loop, masked where needed.)
    const int qt_m = (k_first + BKV - 2) / BQ;
    const int it_split = !CAUSAL ? n_iter : D == 128 ? 0 : min(n_iter, max(0, G * (qt_stop - 1 - qt_m))) & ~1;
    auto run = [&](int it_begin, int it_end, auto MASKED) __attribute__((always_inline)) {
      for (int it = it_begin; it < it_end; it += 2) {
        wait_vmem();
        __syncthreads();
        if (it + 1 < n_iter) issue(it + 1, stage1);
        consume(it, stage0, MASKED);
        if (it + 1 < it_end) {
          wait_vmem();
          __syncthreads();
          if (it + 2 < n_iter) issue(it + 2, stage0);
          consume(it + 1, stage1, MASKED);
        }
      }
    };
    if (n_iter > 0) issue(0, stage0);
    run(0, it_split, std::false_type{});
    run(it_split, n_iter, std::true_type{});
  }

  if (MASK && mykey >= L) {
    if (mykey < N) {
      zero_row(p.dk, (size_t)bkv * N + mykey, g, D);
      zero_row(p.dv, (size_t)bkv * N + mykey, g, D);
    }
  } else if (mykey < N) {
    bf16* dkr = (bf16*)p.dk + ((size_t)bkv * N + mykey) * D;
    bf16* dvr = (bf16*)p.dv + ((size_t)bkv * N + mykey) * D;
    const float sc = p.scale;
    // (the lane's half, formed again from the lane id in the unmasked
    // instances: kept live across the loop it was the one register the causal
    // d = 128 instance spilled)
    const int g_e = MASK ? g : __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int col = db * 32 + 8 * a + 4 * g_e;
        *(i32x2*)(dkr + col) = i32x2{(int)pack_bf16(dk[db][4 * a] * sc, dk[db][4 * a + 1] * sc),
                                     (int)pack_bf16(dk[db][4 * a + 2] * sc, dk[db][4 * a + 3] * sc)};
        *(i32x2*)(dvr + col) = i32x2{(int)pack_bf16(dv[db][4 * a], dv[db][4 * a + 1]),
                                     (int)pack_bf16(dv[db][4 * a + 2], dv[db][4 * a + 3])};
      }
  }
}

// ================================================================ dQ ======
template <int D>
struct DqCfg {
  static constexpr int NW = 4, NT = 256;
  static constexpr int BR = NW * 32;          // queries per workgroup
  static constexpr int BC = 64;               // keys per tile
  static constexpr int RB = D * 2;
  static constexpr int KTILE = BC * RB;
  static constexpr int IPW = KTILE / 1024 / NW;
  static constexpr int STAGE = 2 * KTILE;     // K, V
  static_assert(IPW >= 1, "tile too small for the DMA split");
};

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D > 128 ? 1 : 2, D > 128 ? 1 : 2)))
void bwd_dq_kernel(BwdParams p) {
  using C = DqCfg<D>;
  constexpr int BR = C::BR, BC = C::BC, RB = C::RB, IPW = C::IPW;
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[C::STAGE];

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const WorkItem wi = map_work(blockIdx.x, p.total, p.n_tiles, p.remap, p.group_items);
  const int N = p.N;
  const int b = wi.bh / p.H, h = wi.bh - b * p.H;
  const int bkv = b * p.H_kv + h / (p.H / p.H_kv);
  const int q_first = wi.qt * BR;
  const int q0 = q_first + wid * 32;
  const int myq = q0 + lr;
  const int L = valid_len<MASK>(p, b);
  const int W = MASK ? p.window : -1;
  if (MASK && q_first >= L) {                 // every row of the block is padding
    if (myq < N) zero_row(p.dq, (size_t)wi.bh * N + myq, g, D);
    return;
  }
  const bf16* qgp = (const bf16*)p.q + (size_t)wi.bh * N * D;
  const bf16* dgp = (const bf16*)p.dout + (size_t)wi.bh * N * D;
  const unsigned char* kg = (const unsigned char*)p.k + (size_t)bkv * N * RB;
  const unsigned char* vg = (const unsigned char*)p.v + (size_t)bkv * N * RB;

  // Q and dO operands (B of S^T = K Q^T and dP^T = V dO^T): lane holds its row.
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
  // (a padding row takes P = 0 everywhere: its statistic reads as +inf)
  const float lse2 = myq < L ? p.lse2[(size_t)wi.bh * N + myq] : (MASK ? INFINITY : 0.f);
  const float dlt = myq < N ? p.delta[(size_t)wi.bh * N + myq] : 0.f;
  const float c = p.scale_log2;
  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq[i] = f32x16{};

  const int dma0 = dma_base<RB, kSwzRt>(wid * IPW, lane);
  int roff[D / 16];
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) roff[kb] = lr * RB + rt_swz<RB>(lr, 2 * kb + g) * 16;
  int troff[2][D / 32];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) troff[sec][db] = tr_off<RB>(lane, sec, db);

  const int kv_end = CAUSAL ? min(L, q_first + BR) : L;
  const int t0 = MASK && W >= 0 ? max(0, q_first - W) / BC : 0;   // tiles j = 0.. stand for t0 + j
  int n_tiles = (kv_end + BC - 1) / BC - t0;

  // Block-sparse: the rows are one 128-row query block (BR = 128); step j
  // takes the j-th tile of the list of key tiles that are on.
  static_assert(!MASK || BR == 128, "block masks assume one query block per workgroup");
  const bool bs = MASK && p.block_mask;
  __shared__ unsigned short tlist[MASK ? kMaxTiles : 1];
  __shared__ int tcount;
  if (bs) n_tiles = list_tiles<BC, 1>(p.block_mask, p.nb, h, q_first >> 7, t0, n_tiles, tlist, &tcount);
  auto tile_of = [&](int j) -> int {
    return bs ? __builtin_amdgcn_readfirstlane((int)tlist[j]) >> 2 : t0 + j;
  };
  auto issue = [&](int j, unsigned char* st) {
    const int key0 = tile_of(j) * BC;
    const int bytes = min(L - key0, BC) * RB;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + (size_t)key0 * RB, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + (size_t)key0 * RB, bytes);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      dma16_buf<0>(rk, dma_off<RB, kSwzRt>(dma0, i), st + (wid * IPW + i) * 1024);
      dma16_buf<0>(rv, dma_off<RB, kSwzRt>(dma0, i), st + C::KTILE + (wid * IPW + i) * 1024);
    }
  };

  auto consume = [&](int j, const unsigned char* st) {
    const unsigned char* ks = st;
    const unsigned char* vs = st + C::KTILE;
    auto RO = [&](int kb) { return roff[kb]; };
    auto TO = [&](int sec, int db) { return troff[sec][db]; };
    const int key0 = tile_of(j) * BC;
    if (CAUSAL && key0 > q0 + 31) return;     // every key follows every row of the wave
    if (MASK && W >= 0 && key0 + BC - 1 < q0 - W) return;   // below every row's window
    const bool need_mask = (key0 + BC > L) || (CAUSAL && key0 + BC - 1 > q0) ||
                           (MASK && W >= 0 && key0 < q0 + 31 - W);
    const int lim = min(CAUSAL ? myq : L - 1, L - 1) - key0 - 4 * g;
    const int lo = MASK && W >= 0 ? myq - W - key0 - 4 * g : -BC;   // first visible key offset
    // dS^T = P^T o (dP^T - D) of one 32-key block, packed to bf16 (two copies
    // behind a wave-uniform branch: as one, the compiler turns the mask into
    // a compare and a select per element on every tile)
    auto ds_block = [&](int kb32, const f32x16& s, const f32x16& dp, uint32_t* sw) __attribute__((always_inline)) {
      auto body = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int r2 = 0; r2 < 8; ++r2) {
          float se[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int r = 2 * r2 + e;
            float pv = fast_exp2(fmaf(s[r], c, -lse2));
            if (decltype(masked)::value && ((kb32 * 32 + 8 * (r >> 2) + (r & 3)) > lim ||
                                            (MASK && (kb32 * 32 + 8 * (r >> 2) + (r & 3)) < lo)))
              pv = 0.f;
            se[e] = pv * (dp[r] - dlt);
          }
          sw[r2] = pack_bf16(se[0], se[1]);
        }
      };
      if (need_mask) body(std::true_type{});
      else body(std::false_type{});
    };
    // dS^T of one 32-key block (lane: query column, registers: keys) ...
    auto block_ds = [&](int kb32, bf16x8* ds2) __attribute__((always_inline)) {
      // S^T = K Q^T and dP^T = V dO^T
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) {
        const bf16x8 ak = *(const bf16x8*)(ks + kb32 * 32 * RB + RO(kb));
        const bf16x8 av = *(const bf16x8*)(vs + kb32 * 32 * RB + RO(kb));
        s = mfma_bf16(ak, qr[kb], s);
        dp = mfma_bf16(av, dor[kb], dp);
      }
      uint32_t sw[8];
      ds_block(kb32, s, dp, sw);
#pragma unroll
      for (int half = 0; half < 2; ++half)
        ds2[half] = __builtin_bit_cast(bf16x8, i32x4{(int)sw[4 * half], (int)sw[4 * half + 1],
                                                     (int)sw[4 * half + 2], (int)sw[4 * half + 3]});
    };
    // ... and dQ^T += K^T dS^T for it (K^T by transposing reads of the K rows)
    auto block_dq = [&](int kb32, const bf16x8* ds2) __attribute__((always_inline)) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int rb = (kb32 * 32 + 16 * half) * RB;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x4 lo4 = lds_read_tr16(ks + rb + TO(0, db));
          const bf16x4 hi4 = lds_read_tr16(ks + rb + TO(1, db));
          dq[db] = mfma_bf16(__builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7), ds2[half], dq[db]);
        }
      }
    };
    if constexpr (D > 128) {
      // one block at a time: two blocks' temporaries do not fit next to Q, dO and dQ
#pragma unroll 1
      for (int kb32 = 0; kb32 < BC / 32; ++kb32) {
        bf16x8 ds2[2];
        block_ds(kb32, ds2);
        block_dq(kb32, ds2);
      }
    } else {
      bf16x8 dsb[BC / 32][2];
#pragma unroll
      for (int kb32 = 0; kb32 < BC / 32; ++kb32) {
        // S^T = K Q^T and dP^T = V dO^T (lane: query column, registers: keys)
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int kb = 0; kb < D / 16; ++kb) {
          const bf16x8 ak = *(const bf16x8*)(ks + kb32 * 32 * RB + RO(kb));
          const bf16x8 av = *(const bf16x8*)(vs + kb32 * 32 * RB + RO(kb));
          s = mfma_bf16(ak, qr[kb], s);
          dp = mfma_bf16(av, dor[kb], dp);
        }
        uint32_t sw[8];
        ds_block(kb32, s, dp, sw);
#pragma unroll
        for (int half = 0; half < 2; ++half)
          dsb[kb32][half] = __builtin_bit_cast(bf16x8, i32x4{(int)sw[4 * half], (int)sw[4 * half + 1],
                                                             (int)sw[4 * half + 2], (int)sw[4 * half + 3]});
      }
      // ---- dQ^T += K^T dS^T (K^T by transposing reads of the K rows) ---------
#pragma unroll
      for (int kb32 = 0; kb32 < BC / 32; ++kb32)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int rb = (kb32 * 32 + 16 * half) * RB;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const bf16x4 lo4 = lds_read_tr16(ks + rb + TO(0, db));
            const bf16x4 hi4 = lds_read_tr16(ks + rb + TO(1, db));
            dq[db] = mfma_bf16(__builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7), dsb[kb32][half], dq[db]);
          }
        }
    }
  };

  if (n_tiles > 0) issue(0, stage0);   // (a block-sparse list can be empty)
  for (int j = 0; j < n_tiles; j += 2) {
    wait_vmem();
    __syncthreads();
    if (j + 1 < n_tiles) issue(j + 1, stage1);
    consume(j, stage0);
    if (j + 1 < n_tiles) {
      wait_vmem();
      __syncthreads();
      if (j + 2 < n_tiles) issue(j + 2, stage0);
      consume(j + 1, stage1);
    }
  }

  if (MASK && myq >= L) {
    if (myq < N) zero_row(p.dq, (size_t)wi.bh * N + myq, g, D);
  } else if (myq < N) {
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

// ========================================================== dQ, d = 256 ===
// At d = 256 a wave that keeps Q, dO and dQ of 32 queries needs all 512
// registers of a SIMD lane, so bwd_dq_kernel runs one wave a SIMD and nothing
// hides its softmax work or its operand waits.  Here the two waves of a SIMD
// share 32 queries and split the work by role: wave A (waves 0-3) keeps Q and
// columns 0-127 of dQ, wave B (waves 4-7, on the same SIMDs) keeps dO and
// columns 128-255.  Per 32-key block j, between two barriers: A forms S_j and
// P_j = exp2(S_j c - LSE2) (masked) and hands P_j (fp32) over through LDS,
// while B forms dP_j; then B forms dS_j = P_j (dP_j - D), hands it back and
// adds its half of K_j^T dS_j, while A adds its half of K_{j-1}^T dS_{j-1}
// (one block behind, so neither waits on the other inside a phase).  Both
// halves see the same dS values in the same order as bwd_dq_kernel, so dQ
// is the same bit for bit.  K/V tiles (64 keys, two blocks) are staged by
// LDS DMA; the copy of stage s + 1 goes out at the second block of stage s,
// when the block before it (still read by A) is done.  No masks other than
// the causal one (padding, window and block-sparse calls keep bwd_dq_kernel).
template <bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_pair_kernel(BwdParams p) {
  constexpr int D = 256;
  using C = DqCfg<D>;
  constexpr int BR = C::BR, BC = C::BC, RB = C::RB, NW = 8, HD = D / 64;   // HD: 32-column blocks a half
  constexpr int IPW = C::KTILE / 1024 / NW;   // 1 KB copies per wave and tensor
  static_assert(BR == 4 * 32 && BC == 64, "four pairs of 32 queries, two 32-key blocks a stage");
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) float xp[4][16][64];                  // P_j, per pair
  __shared__ __attribute__((aligned(1024))) unsigned long long xs[2][4][4][64];   // dS_j, dS_{j-1}

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wid >> 2, pr = wid & 3;
  const int lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const WorkItem wi = map_work(blockIdx.x, p.total, p.n_tiles, p.remap, p.group_items);
  const int N = p.N;
  const int b = wi.bh / p.H, h = wi.bh - b * p.H;
  const int bkv = b * p.H_kv + h / (p.H / p.H_kv);
  const int q_first = wi.qt * BR;
  const int q0 = q_first + pr * 32;           // the pair's first query
  const int myq = q0 + lr;
  const unsigned char* kg = (const unsigned char*)p.k + (size_t)bkv * N * RB;
  const unsigned char* vg = (const unsigned char*)p.v + (size_t)bkv * N * RB;

  // A: Q rows (B operand of S^T = K Q^T); B: dO rows (of dP^T = V dO^T)
  const bf16* src = (const bf16*)(grp == 0 ? p.q : p.dout) + (size_t)wi.bh * N * D;
  bf16x8 qd[D / 16];
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) {
    bf16x8 x = {};
    if (myq < N) x = *(const bf16x8*)(src + (size_t)myq * D + kb * 16 + 8 * g);
    qd[kb] = x;
  }
  const float lse2 = myq < N ? p.lse2[(size_t)wi.bh * N + myq] : 0.f;
  const float dlt = myq < N ? p.delta[(size_t)wi.bh * N + myq] : 0.f;
  const float c = p.scale_log2;
  f32x16 dq[HD];                              // A: columns 0-127, B: 128-255
#pragma unroll
  for (int i = 0; i < HD; ++i) dq[i] = f32x16{};

  const int kv_end = CAUSAL ? min(N, q_first + BR) : N;
  const int n_st = (kv_end + BC - 1) / BC;   // stages (64-key tiles)
  const int NB = 2 * n_st;                    // 32-key blocks
  // a block some of whose keys precede some query of the pair
  auto live = [&](int jb) { return jb >= 0 && jb < NB && !(CAUSAL && jb * 32 > q0 + 31); };

  auto issue = [&](int t, unsigned char* st) {
    const int key0 = t * BC;
    const int bytes = min(N - key0, BC) * RB;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + (size_t)key0 * RB, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + (size_t)key0 * RB, bytes);
    const int dma0 = dma_base<RB, kSwzRt>(wid * IPW, __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      dma16_buf<0>(rk, dma_off<RB, kSwzRt>(dma0, i), st + (wid * IPW + i) * 1024);
      dma16_buf<0>(rv, dma_off<RB, kSwzRt>(dma0, i), st + C::KTILE + (wid * IPW + i) * 1024);
    }
  };
  auto stage_of = [&](int jb) -> unsigned char* { return ((jb >> 1) & 1) ? stage1 : stage0; };
  auto offs = [&](int& rb0, int& tb0) {
    const int ln = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    rb0 = (ln & 31) * RB + rt_swz<RB>(ln & 31, ln >> 5) * 16;
    tb0 = tr_off<RB>(ln, 0, 0);
    asm volatile("" : "+v"(rb0), "+v"(tb0));
  };
  // S^T (A: K rows) or dP^T (B: V rows) of block jb: lane = query, registers = keys
  auto prod = [&](const unsigned char* rows) -> f32x16 {
    int rb0, tb0;
    offs(rb0, tb0);
    f32x16 r = {};
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      const bf16x8 a = *(const bf16x8*)(rows + (rb0 ^ (rt_swz<RB>(0, 2 * kb) * 16)));
      r = mfma_bf16(a, qd[kb], r);
    }
    return r;
  };
  // this wave's half of dQ^T += K^T dS^T for the block's K rows (transposing reads)
  auto add_dq = [&](const unsigned char* krows, const unsigned long long* sw64) {
    int rb0, tb0;
    offs(rb0, tb0);
    uint32_t sw[8];
#pragma unroll
    for (int j2 = 0; j2 < 4; ++j2) {
      const unsigned long long x = sw64[j2 * 64 + lane];
      sw[2 * j2] = (uint32_t)x;
      sw[2 * j2 + 1] = (uint32_t)(x >> 32);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const bf16x8 ds = __builtin_bit_cast(bf16x8, i32x4{(int)sw[4 * half], (int)sw[4 * half + 1],
                                                          (int)sw[4 * half + 2], (int)sw[4 * half + 3]});
      const unsigned char* rb = krows + 16 * half * RB;
#pragma unroll
      for (int i = 0; i < HD; ++i) {
        const int db = grp * HD + i;
        const bf16x4 lo4 = lds_read_tr16(rb + (tb0 ^ (rt_swz<RB>(0, db * 4) * 16)));
        const bf16x4 hi4 = lds_read_tr16(rb + (tb0 ^ (rt_swz<RB>(8, db * 4) * 16)) + 8 * RB);
        dq[i] = mfma_bf16(__builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7), ds, dq[i]);
      }
    }
  };

  if (n_st > 0) issue(0, stage0);
  if (grp == 0) {
    // ---- A: S_j and P_j (to B); its half of K_{j-1}^T dS_{j-1} ----------------------
    for (int jb = 0; jb <= NB; ++jb) {
      if ((jb & 1) == 0) wait_vmem();
      __syncthreads();
      if ((jb & 1) == 1 && (jb >> 1) + 1 < n_st) issue((jb >> 1) + 1, stage_of(jb + 1));
      if (live(jb)) {
        const f32x16 s = prod(stage_of(jb) + (jb & 1) * 32 * RB);
        const int key0 = jb * 32;
        const bool masked = (key0 + 32 > N) || (CAUSAL && key0 + 31 > q0);
        const int lim = min(CAUSAL ? myq : N - 1, N - 1) - key0 - 4 * g;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = fast_exp2(fmaf(s[r], c, -lse2));
          if (masked && (8 * (r >> 2) + (r & 3)) > lim) pv = 0.f;
          xp[pr][r][lane] = pv;
        }
      }
      __syncthreads();
      if (live(jb - 1)) add_dq(stage_of(jb - 1) + ((jb - 1) & 1) * 32 * RB, &xs[(jb - 1) & 1][pr][0][0]);
    }
  } else {
    // ---- B: dP_j; dS_j = P_j (dP_j - D) (to A) and its half of K_j^T dS_j ----------------
    for (int jb = 0; jb <= NB; ++jb) {
      if ((jb & 1) == 0) wait_vmem();
      __syncthreads();
      if ((jb & 1) == 1 && (jb >> 1) + 1 < n_st) issue((jb >> 1) + 1, stage_of(jb + 1));
      f32x16 dp = {};
      const bool lv = live(jb);
      if (lv) dp = prod(stage_of(jb) + C::KTILE + (jb & 1) * 32 * RB);
      __syncthreads();
      if (lv) {
        unsigned long long* dst = &xs[jb & 1][pr][0][0];
#pragma unroll
        for (int j2 = 0; j2 < 4; ++j2) {
          const int r = 4 * j2;
          const uint32_t lo = pack_bf16(xp[pr][r][lane] * (dp[r] - dlt), xp[pr][r + 1][lane] * (dp[r + 1] - dlt));
          const uint32_t hi = pack_bf16(xp[pr][r + 2][lane] * (dp[r + 2] - dlt), xp[pr][r + 3][lane] * (dp[r + 3] - dlt));
          dst[j2 * 64 + lane] = (unsigned long long)lo | ((unsigned long long)hi << 32);
        }
        add_dq(stage_of(jb) + (jb & 1) * 32 * RB, dst);
      }
    }
  }

  if (myq < N) {
    bf16* dqr = (bf16*)p.dq + ((size_t)wi.bh * N + myq) * D + grp * (D / 2);
    const float sc = p.scale;
    const int g_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 5;
#pragma unroll
    for (int i = 0; i < HD; ++i)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *(i32x2*)(dqr + i * 32 + 8 * a + 4 * g_e) =
            i32x2{(int)pack_bf16(dq[i][4 * a] * sc, dq[i][4 * a + 1] * sc),
                  (int)pack_bf16(dq[i][4 * a + 2] * sc, dq[i][4 * a + 3] * sc)};
  }
}

// ========================================================= launchers ======
template <int D, bool CAUSAL, bool MASK>
static hipError_t launch_bwd(BwdParams p, hipStream_t s) {
  {
    constexpr int RPB = 256 / (D / 8);
    const long rows = (long)p.B * p.H * p.N;
    if (hipError_t e = launch_kernel(bwd_prep_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), s, p);
        e != hipSuccess)
      return e;
  }
  {
    BwdParams q = p;
    q.n_tiles = (p.N + DkdvCfg<D>::BKV - 1) / DkdvCfg<D>::BKV;
    q.total = p.B * p.H_kv * q.n_tiles;
    q.group_items = q.n_tiles;                  // one (batch, K/V head) group per bh
    // (remap 3: each XCD takes its groups in turn, heaviest key tiles first)
    q.remap = p.seqlens ? ((p.B * p.H_kv) % 8 == 0 ? 2 : 0)
                        : q.total % 8 != 0 ? 0 : (q.total / 8) % q.n_tiles == 0 ? 3 : 1;
    if (hipError_t e = launch_kernel(bwd_dkdv_kernel<D, CAUSAL, MASK>, dim3(q.total), dim3(DkdvCfg<D>::NT), s, q);
        e != hipSuccess)
      return e;
  }
  {
    BwdParams q = p;
    q.n_tiles = (p.N + DqCfg<D>::BR - 1) / DqCfg<D>::BR;
    q.total = p.B * p.H * q.n_tiles;
    q.group_items = (p.H / p.H_kv) * q.n_tiles;
    q.remap = p.seqlens ? ((p.B * p.H_kv) % 8 == 0 ? 2 : 0) : (q.total % 8 == 0 ? 1 : 0);
    if (q.remap == 1 && (q.total / 8) % q.group_items == 0) {
      // whole (batch, K/V head) groups per XCD, their heads taken in turn
      // (heaviest query tiles of every head first)
      q.remap = 3;
      q.group_items = q.n_tiles;
    }
    if constexpr (D == 256) {
      // without padding, window or block masks: the paired-role kernel
      if (p.seqlens == nullptr && p.window < 0 && p.block_mask == nullptr)
        return launch_kernel(bwd_dq_pair_kernel<CAUSAL>, dim3(q.total), dim3(512), s, q);
    }
    return launch_kernel(bwd_dq_kernel<D, CAUSAL, MASK>, dim3(q.total), dim3(DqCfg<D>::NT), s, q);
  }
}

hipError_t launch_bwd_bf16(int d, bool causal, BwdParams& p, hipStream_t s) {
  const bool m = p.seqlens != nullptr || p.window >= 0 || p.block_mask != nullptr;
  switch (d) {
    case 64:
      if (m) return causal ? launch_bwd<64, true, true>(p, s) : launch_bwd<64, false, true>(p, s);
      return causal ? launch_bwd<64, true, false>(p, s) : launch_bwd<64, false, false>(p, s);
    case 128:
      if (m) return causal ? launch_bwd<128, true, true>(p, s) : launch_bwd<128, false, true>(p, s);
      return causal ? launch_bwd<128, true, false>(p, s) : launch_bwd<128, false, false>(p, s);
    case 256:
      // (without a mask the masked instances compute the same; the unmasked
      // non-causal one spills a few registers and the masked one does not)
      if (m || !causal) return causal ? launch_bwd<256, true, true>(p, s) : launch_bwd<256, false, true>(p, s);
      return launch_bwd<256, true, false>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
