// Forward attention kernels for gfx950 (bf16 / fp8 MFMA and fp32 MFMA).
//
// One workgroup owns BR consecutive query rows of one head and streams the
// head's K/V tiles (BC keys each) through LDS, double buffered: the global
// loads of tile j+1 are issued before tile j is consumed and land in the
// other LDS buffer afterwards.  This is the tiling of "FlashAttentionとは？…"
// (QKVをブロック分割してSRAMへ載せるタイリングの手順) with the loop order of
// FlashAttention-2 (queries outside, keys inside; parallel over query tiles,
// "Flash Attention 2 / 3 とは 2026年版", FA2 の改善): the output accumulator
// never leaves registers until the epilogue.
//
// Each wave owns 32 query rows.  Scores are computed transposed,
// S^T = K Q^T, so that in the MFMA output layout one lane holds one query
// row (16 keys per 32-key block, the other 16 in lane l^32): the row max and
// row sum need one cross-half exchange instead of a 32-lane reduction.  The
// probabilities then feed O^T += V^T P^T directly as the B operand, with the
// V^T fragments taken from row-major V tiles by the transposing LDS read.
//
// Online softmax ("FlashAttentionとは？…", 最大値と正規化項を持ち回るオンライン
// softmaxの再スケール): running max m and running sum l per row; exp2 with
// scale*log2(e) folded into one FMA; 1/l applied once in the epilogue.  The
// result is exact up to rounding for any m, as long as numerator and
// denominator use the same one and exp2(score - m) stays in range, so m is
// moved (and the accumulator rescaled) only when needed.  The fp32 kernel
// takes each tile's max and moves m when it exceeds m by more than
// kRescaleSlack; the bf16 and fp8 kernels do not even take the max: they
// form P against the current m and fall back to the max-and-rescale path
// only when a lane's partial row sum leaves [0, kSumBound] (a wave-uniform
// test that also catches the first tile, where m is still -inf).
//
// Causal: key tiles past the work-group's last query are never loaded; the
// mask is applied only on tiles that straddle the diagonal or the sequence
// end (FA2's causal optimisation, "Flash Attention 2 / 3 とは 2026年版").
#include <float.h>

#include <atomic>
#include <type_traits>

#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

// Schedule constants, each the best of a sweep on MI355X:
//  kQkPrefetch   K-fragment LDS reads kept in flight ahead of the MFMA that
//                uses them (4, 8 and 12 measured within 1% on the d = 128
//                causal forward);
//  kPvPrefetch   the same for the transposing V-fragment reads (two a MFMA);
//  kSpValuPerMfma  VALU instructions the pipelined d = 64 kernel places
//                between two of its MFMAs;
//  kNst64        LDS stages of the four-wave d = 64 kernel (four measured
//                11% slower).
constexpr int kQkPrefetch = 8;
constexpr int kPvPrefetch = 8;
constexpr int kSpValuPerMfma = 8;
constexpr int kNst64 = 2;
// fp8 forward: which waves copy the K and raw V tiles and decode V (1: group
// 0 copies, group 1 decodes after its softmax; 2: group 0 does both; 3: all
// waves do both at the top of the phase).
constexpr int kFp8Plan = 1;

// ------------------------------------------------------ mask variants -----
// The per-sequence padding mask and the causal sliding window shrink the
// keys a query sees: query i of sequence b (valid for its first len_b rows)
// sees keys max(0, i - window) .. min(i, len_b - 1) (causal) or
// 0 .. len_b - 1; rows at or past len_b are padding and get O = 0,
// LSE = -inf.  Only the tile range and the element mask change.
struct ItemMask {
  int len;       // valid rows of the sequence (N without a padding mask)
  int window;    // < 0: none
  int t_begin;   // first key tile that any row of the item sees
};
template <bool MASK>
__device__ __forceinline__ ItemMask mask_of(const FwdParams& p, int b, int q_first, int bc) {
  ItemMask m{p.N, -1, 0};
  if constexpr (MASK) {
    m.len = p.seqlens ? min(max(p.seqlens[b], 0), p.N) : p.N;
    m.window = p.window;
    if (p.window >= 0) m.t_begin = max(0, q_first - p.window) / bc;
  }
  return m;
}
// O = 0 (bf16) and LSE = -inf for a padding row, or a row that sees no key;
// lanes l and l ^ 32 each write half of the row.
__device__ __forceinline__ void write_empty_rows(const FwdParams& p, int bh, int myq, int g, int d) {
  if (myq >= p.N) return;
  bf16* orow = (bf16*)p.o + ((size_t)bh * p.N + myq) * d;
  for (int c = 4 * g; c < d; c += 8) *(i32x2*)(orow + c) = i32x2{0, 0};
  if (p.lse && g == 0) p.lse[(size_t)bh * p.N + myq] = -INFINITY;
}

// ====================================================== bf16, LDS DMA =====
// The bf16 forward proper.  K and V tiles go straight from HBM to LDS
// (global_load_lds: no staging registers, no VALU), unpadded and XOR-swizzled
// per row so that the K operand reads (16 B per lane) and the transposing V
// reads (ds_read_b64_tr_b16, which hands each lane a column of V) are free of
// bank conflicts.  The two stages live in two distinct LDS arrays and the
// tile loop is unrolled by two, so the compiler can see that the prefetch into
// one stage never aliases the reads from the other.
template <int D, int NW_, int BC_, int NST_>
struct Bf16Cfg {
  static constexpr int NW = NW_, NT = NW * 64, BR = NW * 32, BC = BC_, NST = NST_;
  static constexpr int RB = D * 2;              // bytes per K/V row in LDS
  static constexpr int TILE = BC * RB;          // bytes per K (or V) tile
  static constexpr int IPW = TILE / 1024 / NW;  // 1 KB DMA issues per wave per tensor
  static_assert(IPW >= 1, "tile too small for the DMA split");
  static_assert(NST >= 2 && NST <= 4, "two to four stages");
  static_assert(2 * IPW * (NST - 2) < 64, "DMA count must fit the vmcnt field");
};
template <int D, bool CAUSAL, int NW, int BC_, int NST, bool MASK>
__device__ __forceinline__ void fwd_bf16_kernel_item(const FwdParams& p, const WorkItem wi) {
  using C = Bf16Cfg<D, NW, BC_, NST>;
  constexpr int BR = C::BR, BC = C::BC, RB = C::RB, IPW = C::IPW;
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[2 * C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[2 * C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char stage2[NST > 2 ? 2 * C::TILE : 1];
  __shared__ __attribute__((aligned(1024))) unsigned char stage3[NST > 3 ? 2 * C::TILE : 1];

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int N = p.N;
  const int b = wi.bh / p.H, h = wi.bh - b * p.H;
  const int bkv = b * p.H_kv + h / (p.H / p.H_kv);
  const unsigned char* qg = (const unsigned char*)p.q + (size_t)wi.bh * N * RB;
  const unsigned char* kg = (const unsigned char*)p.k + (size_t)bkv * N * RB;
  const unsigned char* vg = (const unsigned char*)p.v + (size_t)bkv * N * RB;
  const int q_first = wi.qt * BR;
  const int q0 = q_first + wid * 32;
  const int myq = q0 + lr;
  const ItemMask mk = mask_of<MASK>(p, b, q_first, BC);
  const int L = mk.len;
  if (MASK && q_first >= L) {           // every row of the item is padding
    write_empty_rows(p, wi.bh, myq, g, D);
    return;
  }
  const int kv_end = CAUSAL ? min(L, q_first + BR) : L;
  const int t0 = mk.t_begin;            // tiles j = 0.. stand for t0 + j
  int n_tiles = (kv_end + BC - 1) / BC - t0;
  // Block-sparse: the workgroup's rows are one 128-row query block
  // (BR = 128); step j takes the j-th tile of the list of tiles that are on.
  static_assert(!MASK || BR == 128, "block masks assume one query block per workgroup");
  const bool bs = MASK && p.block_mask;
  __shared__ unsigned short tlist[MASK ? kMaxTiles : 1];
  __shared__ int tcount;
  if (bs) n_tiles = list_tiles<BC, 1>(p.block_mask, p.nb, h, q_first >> 7, t0, n_tiles, tlist, &tcount);
  auto tile_of = [&](int j) -> int {
    return bs ? __builtin_amdgcn_readfirstlane((int)tlist[j]) >> 2 : t0 + j;
  };

  // Q operand (B of S^T = K Q^T): slot (kb, g, e) <-> column kb*16 + 8g + e.
  bf16x8 qr[D / 16];
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) {
    bf16x8 x = {};
    if (myq < N) x = *(const bf16x8*)(qg + (size_t)myq * RB + (kb * 16 + 8 * g) * 2);
    qr[kb] = x;
  }

  // Per-lane byte offsets, fixed for the whole loop.
  int dma_k[IPW], dma_v[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int byte = (wid * IPW + i) * 1024 + lane * 16;
    const int row = byte / RB, pu = (byte % RB) / 16;
    dma_k[i] = row * RB + k_swz<RB>(row, pu) * 16;   // the swizzle is an involution
    dma_v[i] = row * RB + v_swz<RB>(row, pu) * 16;
  }
  // The swizzles touch only the low 4 bits of a 16-byte unit index, so units
  // 16 apart share one per-lane offset (+256 bytes, an immediate).
  constexpr int NKO = D / 16 < 8 ? D / 16 : 8, NVO = D / 32 < 4 ? D / 32 : 4;
  int koff[NKO];
#pragma unroll
  for (int kb = 0; kb < NKO; ++kb) koff[kb] = lr * RB + k_swz<RB>(lr, 2 * kb + g) * 16;
  const int s16 = lane & 15, G = lane >> 4;
  const int vrow = 4 * (G >> 1) + (s16 >> 2);
  int voff[NVO];
#pragma unroll
  for (int db = 0; db < NVO; ++db)
    voff[db] = vrow * RB + v_swz<RB>(vrow, db * 4 + 2 * (G & 1) + ((s16 & 3) >> 1)) * 16 + (s16 & 1) * 8;

  const float c = p.scale_log2;
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  auto issue = [&](int j, unsigned char* st) {
    const int key0 = tile_of(j) * BC;
    const int bytes = min(L - key0, BC) * RB;   // rows past the end read as zero
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + (size_t)key0 * RB, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + (size_t)key0 * RB, bytes);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      dma16_buf<0>(rk, dma_k[i], st + (wid * IPW + i) * 1024);
      dma16_buf<0>(rv, dma_v[i], st + C::TILE + (wid * IPW + i) * 1024);
    }
  };

  auto consume = [&](int j, const unsigned char* kl) {
    const unsigned char* vl = kl + C::TILE;
    const int key0 = tile_of(j) * BC;
    if (CAUSAL && key0 > q0 + 31) return;   // every key of the tile follows every row of the wave
    if (MASK && mk.window >= 0 && key0 + BC - 1 < q0 - mk.window) return;   // below every row's window
    f32x16 s[BC / 32];
#pragma unroll
    for (int kb32 = 0; kb32 < BC / 32; ++kb32) {
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) {
        const bf16x8 a = *(const bf16x8*)(kl + kb32 * 32 * RB + (kb / NKO) * 256 + koff[kb % NKO]);
        acc = mfma_bf16(a, qr[kb], acc);
      }
      s[kb32] = acc;
    }
    // Keep kQkPrefetch K fragments in flight ahead of the MFMA that uses them,
    // so LDS latency overlaps the MFMA chain instead of stalling each step.
    {
      constexpr int NM = (BC / 32) * (D / 16);
      __builtin_amdgcn_sched_group_barrier(0x100, kQkPrefetch, 0);
#pragma unroll
      for (int i = 0; i < NM - kQkPrefetch; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kQkPrefetch, 0);
    }
    if ((key0 + BC > L) || (CAUSAL && key0 + BC - 1 > q0) ||
        (MASK && mk.window >= 0 && key0 < q0 + 31 - mk.window)) {
#pragma unroll
      for (int kb32 = 0; kb32 < BC / 32; ++kb32)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb32 * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if ((CAUSAL && key > myq) || key >= L || (MASK && mk.window >= 0 && key < myq - mk.window))
            s[kb32][r] = -INFINITY;
        }
    }
    // P against the running max first; the tile max is only taken when some
    // lane's partial row sum leaves [0, kSumBound]: a score far above the
    // running max, or the first tile of the rows (running max still -inf).
    // P is rounded to bf16 (the PV operand) and the row sum is taken from the
    // same rounded values, two at a time, so numerator and denominator agree.
    bf16x8 pk[BC / 32][2];
    auto expo = [&](float m) -> float {
      float t = 0.f;
#pragma unroll
      for (int kb32 = 0; kb32 < BC / 32; ++kb32)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint32_t w4[4];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float e0 = fast_exp2(fmaf(s[kb32][half * 8 + 2 * w], c, -m));
            const float e1 = fast_exp2(fmaf(s[kb32][half * 8 + 2 * w + 1], c, -m));
            w4[w] = pack_bf16(e0, e1);
            t += e0 + e1;
          }
          pk[kb32][half] = __builtin_bit_cast(bf16x8, i32x4{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]});
        }
      return t;
    };
    float ts = expo(m_run);
    if (__any(!(ts <= kSumBound))) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb32 = 0; kb32 < BC / 32; ++kb32)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb32][r]);
      mx = max_halves(mx);
      const float m_new = fmaxf(m_run, mx * c);
      // (with MASK a row may have seen no key yet: it keeps m = -inf, l = 0,
      // O = 0 and takes its exponentials against 0, so masked scores give 0)
      const bool none = MASK && m_new == -INFINITY;
      const float alpha = none ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      ts = expo(none ? 0.f : m_run);
    }
    l_run += ts;
#pragma unroll
    for (int kb32 = 0; kb32 < BC / 32; ++kb32)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 pb = pk[kb32][half];
        const unsigned char* vb = vl + (kb32 * 32 + 16 * half) * RB;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const unsigned char* vr = vb + (db / NVO) * 256 + voff[db % NVO];
          const bf16x4 lo = lds_read_tr16(vr);
          const bf16x4 hi = lds_read_tr16(vr + 8 * RB);
          o[db] = mfma_bf16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb, o[db]);
        }
      }
  };

  // Tile j lives in stage j % NST and is loaded NST - 1 tiles ahead.  Before
  // tile j is read, each wave waits for its own DMA of that tile (the later
  // tiles' DMAs, issued after it, may stay in flight) and the barrier makes
  // every wave's part visible; the same barrier retires the stage that the
  // next prefetch overwrites (tile j - 1's).
  auto stage = [&](int u) -> unsigned char* {
    return u == 0 ? stage0 : (u == 1 ? stage1 : (u == 2 ? stage2 : stage3));
  };
#pragma unroll
  for (int u = 0; u < NST - 1; ++u)
    if (u < n_tiles) issue(u, stage(u));
  for (int j0 = 0; j0 < n_tiles; j0 += NST) {
#pragma unroll
    for (int u = 0; u < NST; ++u) {
      const int j = j0 + u;
      if (j < n_tiles) {
        const int later = min(NST - 2, n_tiles - 1 - j);   // tiles issued after j
        if (NST > 3 && later >= 2) wait_vmem_upto<2 * 2 * IPW>();
        else if (NST > 2 && later >= 1) wait_vmem_upto<2 * IPW>();
        else wait_vmem();
        barrier_lds();
        if (j + NST - 1 < n_tiles) issue(j + NST - 1, stage((u + NST - 1) % NST));
        consume(j, stage(u));
      }
    }
  }

  const float l_tot = sum_halves(l_run);
  if (MASK && (myq >= L || l_tot == 0.f)) {   // padding, or a row that sees no key
    write_empty_rows(p, wi.bh, myq, g, D);
  } else if (myq < N) {
    const float inv = 1.f / l_tot;
    bf16* orow = (bf16*)p.o + ((size_t)wi.bh * N + myq) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int col = db * 32 + 8 * a + 4 * g;
        const uint32_t lo = pack_bf16(o[db][4 * a] * inv, o[db][4 * a + 1] * inv);
        const uint32_t hi = pack_bf16(o[db][4 * a + 2] * inv, o[db][4 * a + 3] * inv);
        *(i32x2*)(orow + col) = i32x2{(int)lo, (int)hi};
      }
    if (p.lse && g == 0) p.lse[(size_t)wi.bh * N + myq] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL, int NW, int BC_, int NST, bool PERSIST, bool MASK>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(FwdParams p) {
  if constexpr (PERSIST) {
    const PersistentMap pm = persistent_map(blockIdx.x, gridDim.x, p.total, p.remap, p.group_items);
    for (int r = 0;; ++r) {
      const int w = persistent_item(pm, r);
      if (w < 0) break;
      if (r > 0) __syncthreads();
      fwd_bf16_kernel_item<D, CAUSAL, NW, BC_, NST, MASK>(p, item_of(w, p.n_qt));
    }
  } else {
    fwd_bf16_kernel_item<D, CAUSAL, NW, BC_, NST, MASK>(p, map_work(blockIdx.x, p.total, p.n_qt, p.remap, p.group_items));
  }
}

// ============================================ bf16, software-pipelined ====
// Four independent waves of 32 rows (128 per workgroup), as above, but each
// wave overlaps its own work: the MFMAs of S_{j+1} = K_{j+1} Q^T are issued
// among the exponentials of tile j (they do not depend on each other, so the
// matrix pipe runs under the VALU), then P_j V_j follows.  A wave alone on
// its SIMD (the last, longest items of a short causal grid) no longer leaves
// one pipe idle while the other works.  K and V have stages of their own:
// in step j the wave reads K_{j+1} and V_j while K_{j+2} and V_{j+1} load.
// No tile is skipped for a wave (a tile past the wave's rows is masked out
// instead), so every step has the same shape.  Every row sees a key of its
// first tile (no mask but the causal one), which the lazy max relies on.
//
// With SPLIT the workgroup owns 64 rows, and its waves split the keys: waves
// 0 and 1 (rows 0-31 and 32-63 of the item) take the even 64-key tiles,
// waves 2 and 3 the odd ones; a step loads a pair of tiles and each wave
// works on its half.  At the end the odd waves hand their running max, sum
// and O to their partners through LDS, which merge them with the same
// rescaling as between tiles.  Twice the items, each half as long per wave:
// when a short causal grid has about as many items as resident workgroups
// the longest items no longer leave most of the GPU idle at the end.
template <int D, bool CAUSAL, bool SPLIT>
__device__ __forceinline__ void fwd_bf16_sp_item(const FwdParams& p, const WorkItem wi) {
  using C = Bf16Cfg<D, 4, SPLIT ? 128 : 64, 2>;
  constexpr int BC = 64, RB = C::RB, IPW = C::IPW, NKB = BC / 32;
  constexpr int BR = SPLIT ? 64 : C::BR;   // rows per item
  constexpr int BT = C::BC;                // keys loaded per step
  __shared__ __attribute__((aligned(1024))) unsigned char ks0[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char ks1[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vs0[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char vs1[C::TILE];

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int N = p.N;
  const int b = wi.bh / p.H, h = wi.bh - b * p.H;
  const int bkv = b * p.H_kv + h / (p.H / p.H_kv);
  const unsigned char* qg = (const unsigned char*)p.q + (size_t)wi.bh * N * RB;
  const unsigned char* kg = (const unsigned char*)p.k + (size_t)bkv * N * RB;
  const unsigned char* vg = (const unsigned char*)p.v + (size_t)bkv * N * RB;
  const int q_first = wi.qt * BR;
  const int rb = SPLIT ? (wid & 1) : wid;  // this wave's 32-row block of the item
  const int par = SPLIT ? (wid >> 1) : 0;  // (SPLIT) which 64-key half of a step
  const int q0 = q_first + rb * 32;
  const int myq = q0 + lr;
  const int kv_end = CAUSAL ? min(N, q_first + BR) : N;
  const int n_tiles = (kv_end + BT - 1) / BT;   // steps
  auto key_of = [&](int j) -> int { return j * BT + par * BC; };   // this wave's first key of step j
  const int hoff = par * BC * RB;                                    // its half of a stage

  bf16x8 qr[D / 16];
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) {
    bf16x8 x = {};
    if (myq < N) x = *(const bf16x8*)(qg + (size_t)myq * RB + (kb * 16 + 8 * g) * 2);
    qr[kb] = x;
  }
  int dma_k[IPW], dma_v[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int byte = (wid * IPW + i) * 1024 + lane * 16;
    const int row = byte / RB, pu = (byte % RB) / 16;
    dma_k[i] = row * RB + k_swz<RB>(row, pu) * 16;
    dma_v[i] = row * RB + v_swz<RB>(row, pu) * 16;
  }
  constexpr int NKO = D / 16 < 8 ? D / 16 : 8, NVO = D / 32 < 4 ? D / 32 : 4;
  int koff[NKO];
#pragma unroll
  for (int kb = 0; kb < NKO; ++kb) koff[kb] = lr * RB + k_swz<RB>(lr, 2 * kb + g) * 16;
  const int s16 = lane & 15, G = lane >> 4;
  const int vrow = 4 * (G >> 1) + (s16 >> 2);
  int voff[NVO];
#pragma unroll
  for (int db = 0; db < NVO; ++db)
    voff[db] = vrow * RB + v_swz<RB>(vrow, db * 4 + 2 * (G & 1) + ((s16 & 3) >> 1)) * 16 + (s16 & 1) * 8;

  const float c = p.scale_log2;
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  auto issue = [&](const unsigned char* src, const int* off, int j, unsigned char* st) {
    const int key0 = j * BT;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src + (size_t)key0 * RB, min(N - key0, BT) * RB);
#pragma unroll
    for (int i = 0; i < IPW; ++i) dma16_buf<0>(r, off[i], st + (wid * IPW + i) * 1024);
  };
  auto qk = [&](const unsigned char* kl, f32x16* s) __attribute__((always_inline)) {
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32) s[kb32] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb)
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32) {
        const bf16x8 a = *(const bf16x8*)(kl + kb32 * 32 * RB + (kb / NKO) * 256 + koff[kb % NKO]);
        s[kb32] = mfma_bf16(a, qr[kb], s[kb32]);
      }
  };
  // causal diagonal and ragged tail: scores of keys a row does not see -> -inf
  auto mask_tile = [&](int j, f32x16* s) __attribute__((always_inline)) {
    const int key0 = key_of(j);
    if ((key0 + BC > N) || (CAUSAL && key0 + BC - 1 > q0)) {
      const int lim = min(CAUSAL ? myq : N - 1, N - 1) - key0 - 4 * g;
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb32 * 32 + 8 * (r >> 2) + (r & 3) > lim) s[kb32][r] = -INFINITY;
    }
  };
  // P = exp2(S c - m) rounded to bf16, and the row sum of the rounded values
  auto expo = [&](const f32x16* s, float m, bf16x8 (*pk)[2]) __attribute__((always_inline)) -> float {
    float t = 0.f;
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t w4[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float e0 = fast_exp2(fmaf(s[kb32][half * 8 + 2 * w], c, -m));
          const float e1 = fast_exp2(fmaf(s[kb32][half * 8 + 2 * w + 1], c, -m));
          w4[w] = pack_bf16(e0, e1);
          t += e0 + e1;
        }
        pk[kb32][half] = __builtin_bit_cast(bf16x8, i32x4{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]});
      }
    return t;
  };
  auto pv = [&](const unsigned char* vl, bf16x8 (*pk)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const unsigned char* vb = vl + (kb32 * 32 + 16 * half) * RB;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const unsigned char* vr = vb + (db / NVO) * 256 + voff[db % NVO];
          const bf16x4 lo = lds_read_tr16(vr);
          const bf16x4 hi = lds_read_tr16(vr + 8 * RB);
          o[db] = mfma_bf16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pk[kb32][half], o[db]);
        }
      }
  };
  // Step j: S_j is in scur; K_{j+1} and V_j were issued one step earlier.
  auto step = [&](int j, f32x16* scur, f32x16* snext, const unsigned char* knext, const unsigned char* vcur,
                  unsigned char* k_load, unsigned char* v_load) __attribute__((always_inline)) {
    wait_vmem();
    barrier_lds();   // K_{j+1}, V_j visible; the stages of K_j and V_{j-1} free
    if (j + 1 < n_tiles) issue(vg, dma_v, j + 1, v_load);
    if (j + 2 < n_tiles) issue(kg, dma_k, j + 2, k_load);
    mask_tile(j, scur);
    bf16x8 pk[NKB][2];
    float ts;
    if (j + 1 < n_tiles) {
      qk(knext + hoff, snext);
      ts = expo(scur, m_run, pk);
      // the K reads lead; then each MFMA is followed by its share of the VALU
      constexpr int NM = NKB * (D / 16);
      constexpr int PF = kQkPrefetch < NM ? kQkPrefetch : NM;
      __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + PF < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kSpValuPerMfma, 0);
      }
    } else {
      ts = expo(scur, m_run, pk);
    }
    // the tile max only when some partial row sum leaves [0, kSumBound]
    if (__any(!(ts <= kSumBound))) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, scur[kb32][r]);
      mx = max_halves(mx);
      const float m_new = fmaxf(m_run, mx * c);
      // (SPLIT: an odd wave's rows may have seen no key yet; they keep
      // m = -inf, l = 0, O = 0 and take their exponentials against 0)
      const bool none = SPLIT && m_new == -INFINITY;
      const float alpha = none ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      ts = expo(scur, none ? 0.f : m_run, pk);
    }
    l_run += ts;
    pv(vcur + hoff, pk);
  };

  f32x16 sa[NKB], sb[NKB];
  issue(kg, dma_k, 0, ks0);
  issue(vg, dma_v, 0, vs0);
  if (n_tiles > 1) issue(kg, dma_k, 1, ks1);
  wait_vmem();
  barrier_lds();
  qk(ks0 + hoff, sa);
  for (int j = 0; j < n_tiles; j += 2) {
    step(j, sa, sb, ks1, vs0, ks0, vs1);
    if (j + 1 < n_tiles) step(j + 1, sb, sa, ks0, vs1, ks1, vs0);
  }

  if constexpr (SPLIT) {
    // odd waves -> LDS (in their own register order, so each lane of the
    // partner reads back exactly its own row and columns) -> even waves merge
    constexpr int NV = (D / 32) * 16 + 2;   // floats per lane
    static_assert(64 * NV * 4 <= C::TILE, "a row block's merge area must fit one stage");
    float* xbuf = (float*)(rb ? ks1 : ks0);   // each row block its own area (whole stages)
    barrier_lds();                            // every wave done with the stages
    if (par == 1) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xbuf[(db * 16 + r) * 64 + lane] = o[db][r];
      xbuf[(NV - 2) * 64 + lane] = m_run;
      xbuf[(NV - 1) * 64 + lane] = l_run;
    }
    barrier_lds();
    if (par == 1) return;
    const float m1 = xbuf[(NV - 2) * 64 + lane], l1 = xbuf[(NV - 1) * 64 + lane];
    const float mm = fmaxf(m_run, m1);                 // finite: every row sees key 0 (causal) or N keys
    const float a0 = fast_exp2(m_run - mm), a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mm);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * a0 + xbuf[(db * 16 + r) * 64 + lane] * a1;
    l_run = l_run * a0 + l1 * a1;
    m_run = mm;
  }
  const float l_tot = sum_halves(l_run);
  if (myq < N) {
    const float inv = 1.f / l_tot;
    bf16* orow = (bf16*)p.o + ((size_t)wi.bh * N + myq) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int col = db * 32 + 8 * a + 4 * g;
        const uint32_t lo = pack_bf16(o[db][4 * a] * inv, o[db][4 * a + 1] * inv);
        const uint32_t hi = pack_bf16(o[db][4 * a + 2] * inv, o[db][4 * a + 3] * inv);
        *(i32x2*)(orow + col) = i32x2{(int)lo, (int)hi};
      }
    if (p.lse && g == 0) p.lse[(size_t)wi.bh * N + myq] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_sp_kernel(FwdParams p) {
  fwd_bf16_sp_item<D, CAUSAL, SPLIT>(p, map_work(blockIdx.x, p.total, p.n_qt, p.remap, p.group_items));
}

// =================================================== bf16, ping-pong =====
// Eight waves, two per SIMD (waves w and w + 4 share one).  In phase j every
// wave adds P_{j-1} V_{j-1} and forms S_j = K_j Q^T (32 products); group 0
// (waves 0-3) then runs the softmax of S_j, while group 1 ran the softmax of
// S_{j-1} at the start of the phase.  So on each SIMD one wave's softmax
// (VALU) always runs under the other wave's products.
//
// K and V tiles reach LDS by DMA.  Issuing a DMA can stall a wave for
// hundreds of cycles when the whole CU issues at once.  With LATE, only group
// 0 issues, at the end of its phase, where it would otherwise wait at the
// barrier; tiles then load two phases ahead and K and V each take three
// stages.  Otherwise every wave issues its share at the start of the phase,
// one phase ahead, with two stages each.  (Measured: LATE wins for d = 64,
// where the softmax dominates the phase, and loses for d = 128.)
template <int D, int BC_, bool LATE>
struct PpCfg {
  static constexpr int NW = 8, NT = NW * 64, BR = NW * 32, BC = BC_;
  static constexpr int RB = D * 2;
  static constexpr int TILE = BC * RB;
  static constexpr int NST = LATE ? 3 : 2;                  // stages per tensor
  static constexpr int DW = LATE ? 4 : 8;                   // waves that issue DMA
  static constexpr int IPD = TILE / 1024 / DW;              // 1 KB issues per such wave per tensor
  static constexpr int NKB = BC / 32;
  static_assert(IPD >= 1, "tile too small for the DMA split");
  static_assert(2 * IPD < 64, "DMA count must fit the vmcnt field");
};

// One work item (head, 256-row query tile) of the ping-pong kernel.  With
// MASK, sequence b is valid for its first len_b rows (p.seqlens) and, with a
// window w >= 0, query i sees only keys i - w .. i (see mask_of).  (Block
// masks go to the four-wave kernel, whose workgroup is one query block.)
//
// On the looping grid (NEXT) the item's Q reaches the waves through LDS: each
// wave copies its own 32 rows by LDS DMA into its own part of a Q stage and
// reads its fragments from there, so no other wave touches them.  Right
// after an item's closing phase (where no K stage is read any more) each wave
// copies its rows of the next item's Q and its share of that item's first K
// tile, and the epilogue's stores overlap those copies, so the next item
// starts with its operands in LDS or on their way.  `nx` is the next item
// (bh < 0: none); `pre` says whether this item's Q and first K tile were
// copied so.
template <int D, bool CAUSAL, int BC_, bool LATE, bool MASK, bool NEXT>
__device__ __forceinline__ void pp_item(const FwdParams& p, const WorkItem wi, const WorkItem nx, bool pre) {
  using C = PpCfg<D, BC_, LATE>;
  constexpr int BR = C::BR, BC = C::BC, RB = C::RB, IPD = C::IPD, NKB = C::NKB, NST = C::NST;
  static_assert(!NEXT || (!LATE && !MASK && RB == 256), "next-item copies only on the plain d = 128 schedule");
  constexpr int QPW = BR * RB / 1024 / C::NW;    // 1 KB copies of one wave's Q rows
  __shared__ __attribute__((aligned(1024))) unsigned char k0[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char k2[NST > 2 ? C::TILE : 1];
  __shared__ __attribute__((aligned(1024))) unsigned char v0[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v1[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v2[NST > 2 ? C::TILE : 1];
  // Per-wave regions for NEXT: Q rows (32 x RB bytes) and the epilogue's O
  // staging (16 rows).  Being smaller than the K/V stages they are placed
  // after them, so the stages read every phase keep LDS addresses below
  // 64 KB, within reach of the read instructions' immediate offsets (one
  // 64 KB array would go first and cost an address add per read).
  constexpr int QW = NEXT ? 32 * RB : 1, OW = NEXT ? 16 * RB : 1;
  __shared__ __attribute__((aligned(1024))) unsigned char qs0[QW], qs1[QW], qs2[QW], qs3[QW];
  __shared__ __attribute__((aligned(1024))) unsigned char qs4[QW], qs5[QW], qs6[QW], qs7[QW];
  __shared__ __attribute__((aligned(1024))) unsigned char os0[OW], os1[OW], os2[OW], os3[OW];
  __shared__ __attribute__((aligned(1024))) unsigned char os4[OW], os5[OW], os6[OW], os7[OW];

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wid >> 2;
  const int lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int N = p.N;
  const int b = wi.bh / p.H, h = wi.bh - b * p.H;
  const int bkv = b * p.H_kv + h / (p.H / p.H_kv);
  const unsigned char* qg = (const unsigned char*)p.q + (size_t)wi.bh * N * RB;
  const unsigned char* kg = (const unsigned char*)p.k + (size_t)bkv * N * RB;
  const unsigned char* vg = (const unsigned char*)p.v + (size_t)bkv * N * RB;
  const int q_first = wi.qt * BR;
  const int q0 = q_first + wid * 32;
  const int myq = q0 + lr;
  const ItemMask mk = mask_of<MASK>(p, b, q_first, BC);
  const int L = mk.len;                 // valid rows (N without MASK)
  if (MASK && q_first >= L) {           // every row of the item is padding
    write_empty_rows(p, wi.bh, myq, g, D);
    return;
  }
  const int kv_end = CAUSAL ? min(L, q_first + BR) : L;
  const int t0 = mk.t_begin;            // first key tile any row of the item sees
  const int n_tiles = (kv_end + BC - 1) / BC - t0;   // tiles j = 0.. stand for t0 + j
  auto tile_of = [&](int j) -> int { return t0 + j; };

  const int dwid = wid & (C::DW - 1);   // this wave's share of a DMA'd tile
  int dma_k[IPD], dma_v[IPD];
#pragma unroll
  for (int i = 0; i < IPD; ++i) {
    const int byte = (dwid * IPD + i) * 1024 + lane * 16;
    const int row = byte / RB, pu = (byte % RB) / 16;
    dma_k[i] = row * RB + k_swz<RB>(row, pu) * 16;
    dma_v[i] = row * RB + v_swz<RB>(row, pu) * 16;
  }
  // The swizzles touch only the low 4 bits of a 16-byte unit index, so units
  // 16 apart share one per-lane offset (+256 bytes, an immediate).
  constexpr int NKO = D / 16 < 8 ? D / 16 : 8, NVO = D / 32 < 4 ? D / 32 : 4;
  int koff[NKO];
#pragma unroll
  for (int kb = 0; kb < NKO; ++kb) koff[kb] = lr * RB + k_swz<RB>(lr, 2 * kb + g) * 16;
  const int s16 = lane & 15, G = lane >> 4;
  const int vrow = 4 * (G >> 1) + (s16 >> 2);
  int voff[NVO];
#pragma unroll
  for (int db = 0; db < NVO; ++db)
    voff[db] = vrow * RB + v_swz<RB>(vrow, db * 4 + 2 * (G & 1) + ((s16 & 3) >> 1)) * 16 + (s16 & 1) * 8;

  // Copies for NEXT: the wave's 32 rows of an item's Q, swizzled as a K tile
  // (so its fragments are read as K's are: row lr, units 2 kb + g), and the
  // wave's share of an item's first K tile (no mask: keys 0 .. BC - 1).
  unsigned char* const qw = wid == 0 ? qs0 : wid == 1 ? qs1 : wid == 2 ? qs2 : wid == 3 ? qs3
                         : wid == 4 ? qs4 : wid == 5 ? qs5 : wid == 6 ? qs6 : qs7;
  unsigned char* const ow = wid == 0 ? os0 : wid == 1 ? os1 : wid == 2 ? os2 : wid == 3 ? os3
                         : wid == 4 ? os4 : wid == 5 ? os5 : wid == 6 ? os6 : os7;
  auto issue_q = [&](const WorkItem& it) {
    const int qf = it.qt * BR + wid * 32;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc((const unsigned char*)p.q + ((size_t)it.bh * N + qf) * RB, max(min(N - qf, 32), 0) * RB);
    const int base = dma_base<RB, kSwzK>(wid * QPW, lane) - wid * QPW * 1024;
#pragma unroll
    for (int i = 0; i < QPW; ++i)
      dma16_buf<0>(r, dma_off<RB, kSwzK>(base, i), qw + i * 1024);
  };
  auto issue_k0 = [&](const WorkItem& it) {
    const int bi = it.bh / p.H, hi = it.bh - bi * p.H;
    const size_t kv = (size_t)(bi * p.H_kv + hi / (p.H / p.H_kv)) * N * RB;
    const __amdgpu_buffer_rsrc_t r = make_rsrc((const unsigned char*)p.k + kv, min(N, BC) * RB);
#pragma unroll
    for (int i = 0; i < IPD; ++i) dma16_buf<0>(r, dma_k[i], k0 + (dwid * IPD + i) * 1024);
  };
  const bool has_nx = NEXT && nx.bh >= 0;
  bf16x8 qr[D / 16];
  if constexpr (NEXT) {
    if (!pre) {
      issue_q(wi);
      issue_k0(wi);
    }
    wait_vmem();   // this wave's Q rows (its own copies) are in LDS
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb)
      qr[kb] = *(const bf16x8*)(qw + (kb / NKO) * 256 + koff[kb % NKO]);
  } else {
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      bf16x8 x = {};
      if (myq < N) x = *(const bf16x8*)(qg + (size_t)myq * RB + (kb * 16 + 8 * g) * 2);
      qr[kb] = x;
    }
  }

  const float c = p.scale_log2;
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  bf16x8 pk[NKB][2];

  auto issue_one = [&](const unsigned char* src, const int* off, int j, unsigned char* st) {
    const int key0 = tile_of(j) * BC;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src + (size_t)key0 * RB, min(L - key0, BC) * RB);
#pragma unroll
    for (int i = 0; i < IPD; ++i) dma16_buf<0>(r, off[i], st + (dwid * IPD + i) * 1024);
  };
  // S_j = K_j Q^T into s (false if the wave sees none of the tile's keys), and
  // the online softmax of S_j into P_j (packed bf16).
  f32x16 s[NKB];
  auto qk = [&](int j, const unsigned char* kl) __attribute__((always_inline)) -> bool {
    const int key0 = tile_of(j) * BC;
    if (CAUSAL && key0 > q0 + 31) return false;
    if (MASK && mk.window >= 0 && key0 + BC - 1 < q0 - mk.window) return false;   // below every row's window
    // consecutive MFMAs go to different accumulators (no back-to-back chain)
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32) s[kb32] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb)
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32) {
        const bf16x8 a = *(const bf16x8*)(kl + kb32 * 32 * RB + (kb / NKO) * 256 + koff[kb % NKO]);
        s[kb32] = mfma_bf16(a, qr[kb], s[kb32]);
      }
    {
      constexpr int NM = NKB * (D / 16);
      __builtin_amdgcn_sched_group_barrier(0x100, kQkPrefetch, 0);
#pragma unroll
      for (int i = 0; i < NM - kQkPrefetch; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kQkPrefetch, 0);
    }
    return true;
  };
  auto softmax = [&](int j) __attribute__((always_inline)) {
    const int key0 = tile_of(j) * BC;
    if ((key0 + BC > L) || (CAUSAL && key0 + BC - 1 > q0)) {
      // key = key0 + 4g + rel, rel a compile-time constant per register
      const int lim = min(CAUSAL ? myq : L - 1, L - 1) - key0 - 4 * g;
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rel = kb32 * 32 + 8 * (r >> 2) + (r & 3);
          if (rel > lim) s[kb32][r] = -INFINITY;
        }
    }
    if (MASK && mk.window >= 0 && key0 < q0 + 31 - mk.window) {
      const int lo = myq - mk.window - key0 - 4 * g;   // first visible rel of this row
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rel = kb32 * 32 + 8 * (r >> 2) + (r & 3);
          if (rel < lo) s[kb32][r] = -INFINITY;
        }
    }
    // P against the running max first; the tile max is only taken when some
    // lane's partial row sum leaves [0, kSumBound]: a score far above the
    // running max, or the first tile of the rows (running max still -inf).
    auto expo = [&](float m) -> float {
      float t = 0.f;
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint32_t w4[4];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float e0 = fast_exp2(fmaf(s[kb32][half * 8 + 2 * w], c, -m));
            const float e1 = fast_exp2(fmaf(s[kb32][half * 8 + 2 * w + 1], c, -m));
            w4[w] = pack_bf16(e0, e1);
            t += e0 + e1;
          }
          pk[kb32][half] = __builtin_bit_cast(bf16x8, i32x4{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]});
        }
      return t;
    };
    float ts = expo(m_run);
    if (__any(!(ts <= kSumBound))) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb32][r]);
      mx = max_halves(mx);
      const float m_new = fmaxf(m_run, mx * c);
      // (with MASK a row may have seen no key yet: it keeps m = -inf, l = 0,
      // O = 0 and takes its exponentials against 0, so masked scores give 0)
      const bool none = MASK && m_new == -INFINITY;
      const float alpha = none ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      ts = expo(none ? 0.f : m_run);
    }
    l_run += ts;
  };
  auto pv = [&](const unsigned char* vl) {
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const unsigned char* vb = vl + (kb32 * 32 + 16 * half) * RB;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const unsigned char* vr = vb + (db / NVO) * 256 + voff[db % NVO];
          const bf16x4 lo = lds_read_tr16(vr);
          const bf16x4 hi = lds_read_tr16(vr + 8 * RB);
          o[db] = mfma_bf16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pk[kb32][half], o[db]);
        }
      }
    // V fragments run kPvPrefetch reads (two per MFMA) ahead of their MFMA.
    {
      constexpr int NM = NKB * 2 * (D / 32);
      constexpr int PF = kPvPrefetch < 2 * NM ? kPvPrefetch : 2 * NM;
      __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
      for (int i = 0; i < NM - PF / 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, PF / 2, 0);
    }
  };

  bool has_s = false, has_p = false;
  if constexpr (LATE) {
  // K_j lives in stage j % 3 of k, V_j in stage j % 3 of v.  Group 0 issues
  // K_{j+2} and V_{j+1} at the end of phase j; at the start of phase j it
  // needs K_j and V_{j-1} and may leave K_{j+1} and V_j (issued after them)
  // in flight.
  auto step = [&](int j, const unsigned char* kc, const unsigned char* vp, unsigned char* k_load,
                  unsigned char* v_load) __attribute__((always_inline)) {
    if (grp == 0) {
      if (j + 1 < n_tiles) wait_vmem_upto<2 * IPD>();
      else if (j < n_tiles) wait_vmem_upto<IPD>();
      else wait_vmem();
    }
    barrier_lds();
    if (grp == 1 && has_s) {
      softmax(j - 1);
      has_p = true;
    }
    if (has_p) pv(vp);
    has_p = false;
    has_s = j < n_tiles && qk(j, kc);
    if (grp == 0) {
      if (has_s) {
        softmax(j);
        has_p = true;
        has_s = false;
      }
      if (j + 2 < n_tiles) issue_one(kg, dma_k, j + 2, k_load);
      if (j + 1 < n_tiles) issue_one(vg, dma_v, j + 1, v_load);
    }
  };
  if (grp == 0) {
    issue_one(kg, dma_k, 0, k0);
    if (1 < n_tiles) issue_one(kg, dma_k, 1, k1);
    issue_one(vg, dma_v, 0, v0);
  }
  for (int j = 0; j <= n_tiles; j += 3) {
    step(j, k0, v2, k2, v1);
    if (j + 1 <= n_tiles) step(j + 1, k1, v0, k0, v2);
    if (j + 2 <= n_tiles) step(j + 2, k2, v1, k1, v0);
  }
  } else {
  // K_j lives in stage j % 2 of k, V_j in stage j % 2 of v; phase j loads
  // K_{j+1} and V_j.
  //
  // Issuing a DMA stalls the wave while the CU's texture path takes the
  // copies in (~300-500 clocks for a phase's 32 KB when every wave issues at
  // once).  Group 1's phase is the longer one (softmax, then its 32
  // products), so it issues its share after its softmax, where the copies
  // of group 0 have gone and its products wait for the matrix pipe anyway
  // (C3 0.595 -> 0.526 ms, Ta -3%; issuing later still, between its two
  // product blocks, left too little time for the copies to land: Tc +6%).
  auto step = [&](int j, const unsigned char* kc, const unsigned char* vp, unsigned char* kn,
                  unsigned char* vn) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
    if (grp == 0) {
      if (j + 1 < n_tiles) issue_one(kg, dma_k, j + 1, kn);
      if (j < n_tiles) issue_one(vg, dma_v, j, vn);
    }
    if (grp == 1 && has_s) {
      softmax(j - 1);
      has_p = true;
    }
    if (grp == 1) {
      if (j + 1 < n_tiles) issue_one(kg, dma_k, j + 1, kn);
      if (j < n_tiles) issue_one(vg, dma_v, j, vn);
    }
    if (has_p) pv(vp);
    has_p = false;
    has_s = j < n_tiles && qk(j, kc);
    if (grp == 0 && has_s) {
      softmax(j);
      has_p = true;
      has_s = false;
    }
  };
  if (!NEXT) issue_one(kg, dma_k, 0, k0);
  for (int j = 0; j <= n_tiles; j += 2) {
    step(j, k0, v1, k1, v0);
    if (j + 1 <= n_tiles) step(j + 1, k1, v0, k0, v1);
  }
  // The next item's copies go out before this item's epilogue, whose stores
  // they then overlap: the wave's Q rows, and K_0 into K stage 0, which no
  // wave reads after the closing phase's barrier.
  if (has_nx) {
    issue_q(nx);
    issue_k0(nx);
  }
  }

  const float l_tot = sum_halves(l_run);
  if constexpr (NEXT) {
    // O through the wave's 16-row staging region, two rounds of 16 rows: a
    // lane holds 8-byte pieces of its row, which as global stores would touch
    // 32 rows per instruction; staged, each store writes 1 KB of whole rows.
    // (16-byte unit u of staged row r sits at unit u ^ r: conflict-free
    // 8-byte writes down a column and 16-byte reads along rows.)
    const float inv = 1.f / l_tot;
    unsigned char* const og = (unsigned char*)p.o + ((size_t)wi.bh * N + q0) * RB;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      if ((lr >> 4) == rd) {
        const int row = lr & 15;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const uint32_t lo = pack_bf16(o[db][4 * a] * inv, o[db][4 * a + 1] * inv);
            const uint32_t hi = pack_bf16(o[db][4 * a + 2] * inv, o[db][4 * a + 3] * inv);
            *(i32x2*)(ow + row * RB + (((db * 4 + a) ^ row) << 4) + 8 * g) = i32x2{(int)lo, (int)hi};
          }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int k = 0; k < 16 * RB / 1024; ++k) {
        const int row = k * (1024 / RB) + (lane >> 4), u = lane & 15;
        const i32x4 val = *(const i32x4*)(ow + row * RB + ((u ^ row) << 4));
        if (q0 + 16 * rd + row < N) *(i32x4*)(og + (16 * rd + row) * RB + u * 16) = val;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    if (p.lse && g == 0 && myq < N) p.lse[(size_t)wi.bh * N + myq] = (m_run + fast_log2(l_tot)) * kLn2;
  } else if (MASK && (myq >= L || l_tot == 0.f)) {   // padding, or a row that sees no key
    write_empty_rows(p, wi.bh, myq, g, D);
  } else if (myq < N) {
    const float inv = 1.f / l_tot;
    bf16* orow = (bf16*)p.o + ((size_t)wi.bh * N + myq) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int col = db * 32 + 8 * a + 4 * g;
        const uint32_t lo = pack_bf16(o[db][4 * a] * inv, o[db][4 * a + 1] * inv);
        const uint32_t hi = pack_bf16(o[db][4 * a + 2] * inv, o[db][4 * a + 3] * inv);
        *(i32x2*)(orow + col) = i32x2{(int)lo, (int)hi};
      }
    if (p.lse && g == 0) p.lse[(size_t)wi.bh * N + myq] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

// With PERSIST, one workgroup per CU loops over its share of the items (see
// persistent_map); otherwise one workgroup per item.  Between items the
// workgroup synchronises: an item's first DMAs must not land in a stage a
// slower wave is still reading for the previous item.  With the next-item
// copies (NEXT) no such sync is needed: they go to stages nobody reads by then
// (the wave's own Q rows; K stage 0 after the closing phase's barrier), and
// an item's first tile copies follow its first phase's barrier.
template <int D, bool CAUSAL, int BC_, bool LATE, bool PERSIST, bool MASK>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_pp_kernel(FwdParams p) {
  if constexpr (PERSIST) {
    constexpr bool NEXT = !LATE && !MASK;
    const PersistentMap pm = persistent_map(blockIdx.x, gridDim.x, p.total, p.remap, p.group_items);
    int w = persistent_item(pm, 0);
    for (int r = 0; w >= 0; ++r) {
      const int wn = persistent_item(pm, r + 1);
      if (!NEXT && r > 0) __syncthreads();
      pp_item<D, CAUSAL, BC_, LATE, MASK, NEXT>(p, item_of(w, p.n_qt),
                                              wn >= 0 ? item_of(wn, p.n_qt) : WorkItem{-1, 0}, r > 0);
      w = wn;
    }
  } else {
    pp_item<D, CAUSAL, BC_, LATE, MASK, false>(p, map_work(blockIdx.x, p.total, p.n_qt, p.remap, p.group_items),
                                               WorkItem{-1, 0}, false);
  }
}

// ================================================ fp8, ping-pong (d = 128) ===
// The ping-pong kernel's schedule (eight waves, two a SIMD, 256 rows, 64-key
// tiles) for block-quantised e4m3 inputs: K and V tiles arrive by LDS DMA as
// fp8 (half the bytes of bf16); S = K Q^T runs on the fp8 MFMA (twice the
// bf16 rate) with the Q and K block scales folded into the exponent; each
// phase the workgroup decodes the previous V tile to bf16 once (one 16-byte
// chunk a thread, exact), behind a second barrier, and P V runs on the bf16
// MFMA as before, with V's block scale folded into P (P' = P sV, l += sum/sV).
template <int D, bool CAUSAL>
__device__ __forceinline__ void pp8_item(const FwdParams& p, const WorkItem wi) {
  constexpr int NW = 8, BR = NW * 32, BC = 64, NKB = BC / 32;
  constexpr int RB8 = D, RBV = 2 * D;            // bytes per fp8 row, per decoded bf16 row
  constexpr int T8 = BC * RB8, TV = BC * RBV;
  constexpr int IPD = T8 / 1024 / NW;            // 1 KB DMA issues per wave per tensor
  static_assert(IPD == 1 && T8 == NW * 64 * 16, "one 16-byte chunk of a tile per thread");
  __shared__ __attribute__((aligned(1024))) unsigned char k0[T8];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[T8];
  __shared__ __attribute__((aligned(1024))) unsigned char r0[T8];
  __shared__ __attribute__((aligned(1024))) unsigned char r1[T8];
  __shared__ __attribute__((aligned(1024))) unsigned char v0[TV];
  __shared__ __attribute__((aligned(1024))) unsigned char v1[TV];

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wid >> 2;
  const int lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int N = p.N;
  const int b = wi.bh / p.H, h = wi.bh - b * p.H;
  const int bkv = b * p.H_kv + h / (p.H / p.H_kv);
  const unsigned char* qg = (const unsigned char*)p.q + (size_t)wi.bh * N * D;
  const unsigned char* kg = (const unsigned char*)p.k + (size_t)bkv * N * D;
  const unsigned char* vg = (const unsigned char*)p.v + (size_t)bkv * N * D;
  const int q_first = wi.qt * BR;
  const int q0 = q_first + wid * 32;
  const int myq = q0 + lr;
  const int kv_end = CAUSAL ? min(N, q_first + BR) : N;
  const int n_tiles = (kv_end + BC - 1) / BC;
  const int nsb = (N + 127) >> 7;                // scale blocks per head

  // Q operand (B of S^T = K Q^T): slot kb <-> columns 64 kb + 32 g .. + 31
  i32x8 qr[D / 64];
#pragma unroll
  for (int kb = 0; kb < D / 64; ++kb) {
    i32x8 x = {};
    if (myq < N) {
      const i32x4* src = (const i32x4*)(qg + (size_t)myq * D + kb * 64 + 32 * g);
      x = __builtin_shufflevector(src[0], src[1], 0, 1, 2, 3, 4, 5, 6, 7);
    }
    qr[kb] = x;
  }
  // (the wave's rows share one 128-row scale block; rows past N take the last)
  const float cq = p.scale_log2 * p.qs[(size_t)wi.bh * nsb + (min(q0, N - 1) >> 7)];
  const float* ksc = p.ks + (size_t)bkv * nsb;
  const float* vsc = p.vs + (size_t)bkv * nsb;

  // Copies: with every wave issuing, wave w copies KB w of a tile; with
  // group 0 alone (kFp8Plan 1 and 2), wave w copies KBs 2w and 2w + 1.
  constexpr bool G0_DMA = kFp8Plan != 3;
  constexpr int NDMA = G0_DMA ? 2 : 1;
  const int dmw = G0_DMA ? 2 * (wid & 3) : wid;                // first KB this wave copies
  const int dma_k0 = dma_base<RB8, kSwzK>(dmw, lane);          // K rows swizzled for the fragment reads
  const int dma_r0 = dmw * 1024 + lane * 16;                   // raw V: a plain copy
  int koff[D / 64][2];   // K fragment: row lr, 16-byte units 4 kb + 2 g and + 1
#pragma unroll
  for (int kb = 0; kb < D / 64; ++kb)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) koff[kb][hh] = lr * RB8 + k_swz<RB8>(lr, 4 * kb + 2 * g + hh) * 16;
  constexpr int NVO = D / 32 < 4 ? D / 32 : 4;
  const int s16 = lane & 15, G = lane >> 4;
  const int vrow = 4 * (G >> 1) + (s16 >> 2);
  int voff[NVO];
#pragma unroll
  for (int db = 0; db < NVO; ++db)
    voff[db] = vrow * RBV + v_swz<RBV>(vrow, db * 4 + 2 * (G & 1) + ((s16 & 3) >> 1)) * 16 + (s16 & 1) * 8;
  // decode: 8 fp8 values (16 bytes of bf16, one unit of a decoded row) at a
  // time; 16 consecutive threads fill one row, so each 16-lane write covers 16
  // distinct units (two rows per write group would meet in the same banks:
  // the V swizzle never flips a unit's low bit)
  constexpr bool DEC1 = kFp8Plan != 3;
  constexpr int DTH = DEC1 ? 256 : 512;                        // decoding threads
  constexpr int UPR = RB8 / 8;                                 // 8-value pieces per row
  const int dt = DEC1 ? (tid & 255) : tid;
  const int drow = dt / UPR, du = dt % UPR;
  const int dst = drow * RBV + v_swz<RBV>(drow, du) * 16;     // rows DTH / UPR apart share the swizzle
  static_assert((DTH / UPR) % 4 == 0, "the V swizzle repeats every 4 rows");

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  bf16x8 pk[NKB][2];
  f32x16 s[NKB];

  auto issue_k = [&](int j, unsigned char* st) {
    const int key0 = j * BC;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(kg + (size_t)key0 * D, min(N - key0, BC) * D);
#pragma unroll
    for (int i = 0; i < NDMA; ++i) dma16_buf<0>(r, dma_off<RB8, kSwzK>(dma_k0, i), st + (dmw + i) * 1024);
  };
  auto issue_r = [&](int j, unsigned char* st) {
    const int key0 = j * BC;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(vg + (size_t)key0 * D, min(N - key0, BC) * D);
#pragma unroll
    for (int i = 0; i < NDMA; ++i) dma16_buf<0>(r, dma_r0 + i * 1024, st + (dmw + i) * 1024);
  };
  auto decode = [&](const unsigned char* rl, unsigned char* vl) {
#pragma unroll
    for (int i = 0; i < T8 / 8 / DTH; ++i) {
      const i32x2 x = *(const i32x2*)(rl + (dt + DTH * i) * 8);
      i32x4 y;
      y[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.f, false));
      y[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.f, true));
      y[2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.f, false));
      y[3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.f, true));
      *(i32x4*)(vl + dst + i * (DTH / UPR) * RBV) = y;
    }
  };
  auto qk = [&](int j, const unsigned char* kl) __attribute__((always_inline)) -> bool {
    const int key0 = j * BC;
    if (CAUSAL && key0 > q0 + 31) return false;
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32) s[kb32] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < D / 64; ++kb)
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32) {
        const unsigned char* kr = kl + kb32 * 32 * RB8;
        const i32x4 a0 = *(const i32x4*)(kr + koff[kb][0]);
        const i32x4 a1 = *(const i32x4*)(kr + koff[kb][1]);
        s[kb32] = mfma_fp8(__builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7), qr[kb], s[kb32]);
      }
    return true;
  };
  // (block scales of the wave's next softmax tile, loaded one softmax ahead)
  float ks_cur = ksc[0], vs_cur = vsc[0];
  auto softmax = [&](int j) __attribute__((always_inline)) {
    const int key0 = j * BC;
    // A zero Q or K block scale makes every score of the block 0: the factor
    // is kept positive (the smallest normal float), so raw scores, whatever
    // their codes, give exponent arguments of ~0 and masked (-inf) scores stay
    // -inf instead of 0 * -inf.  A zero V block scale (an all-zero V block)
    // adds nothing to O but its keys still count in the row sum: P' = 0 and
    // the sum taken unscaled.  (Block scales are uniform over the wave.)
    const float c = fmaxf(cq * ks_cur, FLT_MIN);
    const float sv = vs_cur;
    {
      const int kn = min(j + 1, n_tiles - 1) * BC;
      ks_cur = ksc[kn >> 7];
      vs_cur = vsc[kn >> 7];
    }
    const bool v_zero = !(sv > 0.f);
    const float lsv = v_zero ? 0.f : fast_log2(sv), inv_sv = v_zero ? 1.f : 1.f / sv;
    if ((key0 + BC > N) || (CAUSAL && key0 + BC - 1 > q0)) {
      const int lim = min(CAUSAL ? myq : N - 1, N - 1) - key0 - 4 * g;
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rel = kb32 * 32 + 8 * (r >> 2) + (r & 3);
          if (rel > lim) s[kb32][r] = -INFINITY;
        }
    }
    // P' = P sV against the running max first; the tile max only when some
    // lane's partial row sum of P leaves [0, kSumBound]
    auto expo = [&](float m) -> float {
      float t = 0.f;
      const float ma = m - lsv;
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint32_t w4[4];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float e0 = fast_exp2(fmaf(s[kb32][half * 8 + 2 * w], c, -ma));
            const float e1 = fast_exp2(fmaf(s[kb32][half * 8 + 2 * w + 1], c, -ma));
            w4[w] = pack_bf16(e0, e1);
            t += e0 + e1;
          }
          pk[kb32][half] = __builtin_bit_cast(bf16x8, i32x4{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]});
        }
      return t * inv_sv;
    };
    float ts = expo(m_run);
    if (__any(!(ts <= kSumBound))) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb32][r]);
      mx = max_halves(mx);
      const float m_new = fmaxf(m_run, mx * c);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      ts = expo(m_run);
    }
    if (v_zero) {
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32) pk[kb32][0] = pk[kb32][1] = bf16x8{};
    }
    l_run += ts;
  };
  auto pv = [&](const unsigned char* vl) {
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const unsigned char* vb = vl + (kb32 * 32 + 16 * half) * RBV;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const unsigned char* vr = vb + (db / NVO) * 256 + voff[db % NVO];
          const bf16x4 lo = lds_read_tr16(vr);
          const bf16x4 hi = lds_read_tr16(vr + 8 * RBV);
          o[db] = mfma_bf16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pk[kb32][half], o[db]);
        }
      }
  };

  // Phase j: K_j in k[j & 1]; the raw V_j in r[j & 1], loaded in phase j - 1;
  // V_j decoded in phase j into v[j & 1] and used in phase j + 1, whose
  // opening barrier makes it visible: one barrier per phase.
  bool has_s = false, has_p = false;
  auto step = [&](int j, const unsigned char* kc, unsigned char* kn, unsigned char* r_load,
                  const unsigned char* r_dec, unsigned char* v_dec, const unsigned char* v_use)
      __attribute__((always_inline)) {
    wait_vmem();
    barrier_lds();   // K_j, raw V_j and decoded V_{j-1} in place; the stages written below are free
    if (!G0_DMA || grp == 0) {
      if (j + 1 < n_tiles) issue_k(j + 1, kn);
      if (j + 1 < n_tiles) issue_r(j + 1, r_load);
    }
    if (kFp8Plan != 1 && (!DEC1 || grp == 0) && j < n_tiles) decode(r_dec, v_dec);
    if (grp == 1 && has_s) {
      softmax(j - 1);
      has_p = true;
    }
    if (kFp8Plan == 1 && grp == 1 && j < n_tiles) decode(r_dec, v_dec);
    if (has_p) pv(v_use);
    has_p = false;
    has_s = j < n_tiles && qk(j, kc);
    if (grp == 0 && has_s) {
      softmax(j);
      has_p = true;
      has_s = false;
    }
  };
  if (!G0_DMA || grp == 0) {
    issue_k(0, k0);
    issue_r(0, r0);
  }
  for (int j = 0; j <= n_tiles; j += 2) {
    step(j, k0, k1, r1, r0, v0, v1);
    if (j + 1 <= n_tiles) step(j + 1, k1, k0, r0, r1, v1, v0);
  }

  const float l_tot = sum_halves(l_run);
  if (myq < N) {
    const float inv = 1.f / l_tot;
    bf16* orow = (bf16*)p.o + ((size_t)wi.bh * N + myq) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int col = db * 32 + 8 * a + 4 * g;
        const uint32_t lo = pack_bf16(o[db][4 * a] * inv, o[db][4 * a + 1] * inv);
        const uint32_t hi = pack_bf16(o[db][4 * a + 2] * inv, o[db][4 * a + 3] * inv);
        *(i32x2*)(orow + col) = i32x2{(int)lo, (int)hi};
      }
    if (p.lse && g == 0) p.lse[(size_t)wi.bh * N + myq] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL, bool PERSIST>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_fp8_pp_kernel(FwdParams p) {
  if constexpr (PERSIST) {
    const PersistentMap pm = persistent_map(blockIdx.x, gridDim.x, p.total, p.remap, p.group_items);
    for (int r = 0;; ++r) {
      const int w = persistent_item(pm, r);
      if (w < 0) break;
      if (r > 0) __syncthreads();
      pp8_item<D, CAUSAL>(p, item_of(w, p.n_qt));
    }
  } else {
    pp8_item<D, CAUSAL>(p, map_work(blockIdx.x, p.total, p.n_qt, p.remap, p.group_items));
  }
}

// ====================================================== bf16, d = 256 =====
// Head dim 256: a 32-row block of O alone takes 128 fp32 registers a lane, so
// one wave per 32 rows cannot run two waves a SIMD.  Here the two waves that
// share a SIMD (w and w + 4) own the same 32 rows and split O by columns
// (role r holds columns 128r .. 128r + 127).  Key tiles alternate between
// them: the owner of tile t (role t & 1) computes S_t = K_t Q^T over the whole
// head dim and the softmax, and publishes P_t (bf16), the max it used and the
// row sums through LDS; both waves then add P_t V_t into their half of O.
// One phase per tile, between workgroup barriers:
//   owner of t:  P_{t-1} from LDS -> O += P_{t-1} V_{t-1};  softmax of S_t -> LDS
//   the other:   O += P_{t-1} V_{t-1} (its own P);          S_{t+1} = K_{t+1} Q^T
// so on each SIMD one wave's softmax (VALU) runs under the other's products.
// The running max is shared: P_t is formed against the max published with
// P_{t-1} (moved only on the slow path), and before adding P_t V_t each wave
// rescales its half of O (and the row sum) to P_t's max, so both halves and
// both copies of the row sum follow the same sequence of maxima exactly.
template <int D>
struct PairCfg {
  static constexpr int NW = 8, NT = 512, NPAIR = 4, BR = NPAIR * 32, BC = 64;
  static constexpr int RB = D * 2;               // bytes per K/V row
  static constexpr int TILE = BC * RB;           // one K (or V) tile
  static constexpr int IPW = TILE / 1024 / NW;   // 1 KB DMA issues per wave per tensor
  static constexpr int DH = D / 2;               // columns of O per wave
  static constexpr int PBYTES = 2 * 2 * 64 * 16; // one P tile of a pair (B-operand fragments)
  static_assert(IPW >= 1, "tile too small for the DMA split");
};

template <int D, bool CAUSAL, bool MASK>
__device__ __forceinline__ void fwd_bf16_pairs_kernel_item(const FwdParams& p, const WorkItem wi) {
  using C = PairCfg<D>;
  constexpr int BR = C::BR, BC = C::BC, RB = C::RB, IPW = C::IPW, DH = C::DH;
  constexpr int NKB = BC / 32;
  __shared__ __attribute__((aligned(1024))) unsigned char k0[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v0[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v1[C::TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char pbuf[C::NPAIR * C::PBYTES];
  __shared__ float mbuf[C::NPAIR * 64];
  __shared__ float sbuf[C::NPAIR * 64];

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pr = wid & 3, role = wid >> 2;
  const int lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int N = p.N;
  const int b = wi.bh / p.H, h = wi.bh - b * p.H;
  const int bkv = b * p.H_kv + h / (p.H / p.H_kv);
  const unsigned char* qg = (const unsigned char*)p.q + (size_t)wi.bh * N * RB;
  const unsigned char* kg = (const unsigned char*)p.k + (size_t)bkv * N * RB;
  const unsigned char* vg = (const unsigned char*)p.v + (size_t)bkv * N * RB;
  const int q_first = wi.qt * BR;
  const int q0 = q_first + pr * 32;              // first row of the pair
  const int myq = q0 + lr;
  const ItemMask mk = mask_of<MASK>(p, b, q_first, BC);
  const int L = mk.len;
  if (MASK && q_first >= L) {                    // every row of the item is padding
    if (role == 0) write_empty_rows(p, wi.bh, myq, g, D);
    return;
  }
  const int kv_end = CAUSAL ? min(L, q_first + BR) : L;
  const int t0 = mk.t_begin;                     // tiles t = 0.. stand for t0 + t
  const int n_tiles = (kv_end + BC - 1) / BC - t0;
  // tiles the pair takes part in: t_beg .. t_end - 1
  const int t_end = CAUSAL ? min(n_tiles, (q0 + 31) / BC + 1 - t0) : n_tiles;
  const int t_beg = MASK && mk.window >= 0 ? max(0, q0 - mk.window) / BC - t0 : 0;

  bf16x8 qr[D / 16];
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb) {
    bf16x8 x = {};
    if (myq < N) x = *(const bf16x8*)(qg + (size_t)myq * RB + (kb * 16 + 8 * g) * 2);
    qr[kb] = x;
  }
  const int dma_k0 = dma_base<RB, kSwzK>(wid * IPW, lane);
  const int dma_v0 = dma_base<RB, kSwzV>(wid * IPW, lane);
  // The swizzles touch only the low 4 bits of a 16-byte unit index, so units
  // 16 apart share one per-lane offset (+256 bytes, an immediate).
  constexpr int NKO = 8, NVO = DH / 32;
  static_assert(DH == 128, "the column split assumes 16 units of 16 bytes per half row");
  int koff[NKO];
#pragma unroll
  for (int kb = 0; kb < NKO; ++kb) koff[kb] = lr * RB + k_swz<RB>(lr, 2 * kb + g) * 16;
  const int s16 = lane & 15, G = lane >> 4;
  const int vrow = 4 * (G >> 1) + (s16 >> 2);
  int voff[NVO];   // this wave's half of the columns starts 16 units (256 bytes) in for role 1
#pragma unroll
  for (int db = 0; db < NVO; ++db)
    voff[db] = vrow * RB + v_swz<RB>(vrow, db * 4 + 2 * (G & 1) + ((s16 & 3) >> 1)) * 16 + (s16 & 1) * 8 +
               role * 256;

  const float c = p.scale_log2;
  f32x16 o[DH / 32];
#pragma unroll
  for (int i = 0; i < DH / 32; ++i) o[i] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.f;   // the max O and l are scaled to
  float m_own = -INFINITY, ts_own = 0.f;  // stats of the last tile this wave owned
  f32x16 s[NKB];
  bf16x8 pk[NKB][2];
  unsigned char* pb = pbuf + pr * C::PBYTES + lane * 16;
  float* mb = mbuf + pr * 64 + lane;
  float* sb = sbuf + pr * 64 + lane;

  auto issue = [&](const unsigned char* src, bool is_k, int t, unsigned char* st) {
    const int key0 = (t0 + t) * BC;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src + (size_t)key0 * RB, min(L - key0, BC) * RB);
#pragma unroll
    for (int i = 0; i < IPW; ++i)
      dma16_buf<0>(r, is_k ? dma_off<RB, kSwzK>(dma_k0, i) : dma_off<RB, kSwzV>(dma_v0, i),
                   st + (wid * IPW + i) * 1024);
  };
  auto qk = [&](const unsigned char* kl) {
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32) s[kb32] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb)
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32) {
        const bf16x8 a = *(const bf16x8*)(kl + kb32 * 32 * RB + (kb / NKO) * 256 + koff[kb % NKO]);
        s[kb32] = mfma_bf16(a, qr[kb], s[kb32]);
      }
    {
      constexpr int NM = NKB * (D / 16);
      __builtin_amdgcn_sched_group_barrier(0x100, kQkPrefetch, 0);
#pragma unroll
      for (int i = 0; i < NM - kQkPrefetch; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kQkPrefetch, 0);
    }
  };
  // Bring O and l to the max of the tile about to be added, then add its sums.
  auto rebase = [&](float m_t, float ts_t) {
    if (__any(m_t > m_ref)) {
      const float m_new = fmaxf(m_ref, m_t);
      // (with MASK a row may still have seen no key: both maxima -inf)
      const float alpha = MASK && m_new == -INFINITY ? 1.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DH / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    }
    l_run += ts_t;
  };
  // O += P V for this wave's columns; P fragments from registers or LDS.
  auto pv = [&](const unsigned char* vl, bool from_lds) {
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 pf = from_lds ? *(const bf16x8*)(pb + (kb32 * 2 + half) * 1024) : pk[kb32][half];
        const unsigned char* vb = vl + (kb32 * 32 + 16 * half) * RB;
#pragma unroll
        for (int db = 0; db < DH / 32; ++db) {
          const unsigned char* vr = vb + voff[db];
          const bf16x4 lo = lds_read_tr16(vr);
          const bf16x4 hi = lds_read_tr16(vr + 8 * RB);
          o[db] = mfma_bf16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pf, o[db]);
        }
      }
  };
  // Softmax of S_t against m_prev; leaves P_t in pk and publishes it.
  auto softmax = [&](int t, float m_prev) {
    const int key0 = (t0 + t) * BC;
    if ((key0 + BC > L) || (CAUSAL && key0 + BC - 1 > q0)) {
      const int lim = min(CAUSAL ? myq : L - 1, L - 1) - key0 - 4 * g;
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rel = kb32 * 32 + 8 * (r >> 2) + (r & 3);
          if (rel > lim) s[kb32][r] = -INFINITY;
        }
    }
    if (MASK && mk.window >= 0 && key0 < q0 + 31 - mk.window) {
      const int lo = myq - mk.window - key0 - 4 * g;
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rel = kb32 * 32 + 8 * (r >> 2) + (r & 3);
          if (rel < lo) s[kb32][r] = -INFINITY;
        }
    }
    auto expo = [&](float m) -> float {
      float acc = 0.f;
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint32_t w4[4];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float e0 = fast_exp2(fmaf(s[kb32][half * 8 + 2 * w], c, -m));
            const float e1 = fast_exp2(fmaf(s[kb32][half * 8 + 2 * w + 1], c, -m));
            w4[w] = pack_bf16(e0, e1);
            acc += e0 + e1;
          }
          pk[kb32][half] = __builtin_bit_cast(bf16x8, i32x4{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]});
        }
      return acc;
    };
    float m = m_prev;
    float ts = expo(m);
    if (__any(!(ts <= kSumBound))) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb32][r]);
      mx = max_halves(mx);
      m = fmaxf(m, mx * c);
      // (with MASK a row may have seen no key yet: m stays -inf and the
      // exponentials are taken against 0, so masked scores give 0)
      ts = expo(MASK && m == -INFINITY ? 0.f : m);
    }
    m_own = m;
    ts_own = sum_halves(ts);
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
      for (int half = 0; half < 2; ++half) *(bf16x8*)(pb + (kb32 * 2 + half) * 1024) = pk[kb32][half];
    *mb = m_own;
    *sb = ts_own;
  };

  // Phase ph: K_{ph+1} and V_{ph-1} are read; K_{ph+2} and V_ph are loaded.
  // K_t lives in stage t & 1 of k, V_t in stage t & 1 of v.  Role 0 owns the
  // even tiles, role 1 the odd ones; each role runs its own copy of the loop
  // (same barriers, same order), so the compiler sees which values live
  // across a phase: P after an owner phase, S after the other one.
  auto begin = [&](int ph, unsigned char* k_load, unsigned char* v_load) {
    wait_vmem();
    __syncthreads();
    if (ph + 2 < n_tiles) issue(kg, true, ph + 2, k_load);
    if (ph >= 0 && ph < n_tiles) issue(vg, false, ph, v_load);
  };
  auto as_owner = [&](int ph, const unsigned char* v_use) {
    // the partner's tile ph - 1: its max, row sums and P come from LDS
    const float m_prev = ph > t_beg ? *mb : -INFINITY;
    if (ph - 1 >= t_beg && ph - 1 < t_end) {
      rebase(m_prev, *sb);
      pv(v_use, true);
    }
    if (ph >= t_beg && ph < t_end) softmax(ph, m_prev);
  };
  auto as_other = [&](int ph, const unsigned char* k_use, const unsigned char* v_use) {
    if (ph - 1 >= t_beg && ph - 1 < t_end) {
      rebase(m_own, ts_own);
      pv(v_use, false);
    }
    if (ph + 1 >= t_beg && ph + 1 < t_end) qk(k_use);
  };

  issue(kg, true, 0, k0);
  if (role == 0) {
    for (int ph = -1; ph <= n_tiles; ph += 2) {
      begin(ph, k1, v1);                  // ph odd: K_{ph+1} in k0, V_{ph-1} in v0
      as_other(ph, k0, v0);
      if (ph + 1 <= n_tiles) {
        begin(ph + 1, k0, v0);            // ph + 1 even: K in k1, V in v1
        as_owner(ph + 1, v1);
      }
    }
  } else {
    for (int ph = -1; ph <= n_tiles; ph += 2) {
      begin(ph, k1, v1);
      as_owner(ph, v0);
      if (ph + 1 <= n_tiles) {
        begin(ph + 1, k0, v0);
        as_other(ph + 1, k1, v1);
      }
    }
  }

  // l_run already holds whole-row sums (the published sums were combined
  // across the two halves of the wave).
  if (MASK && myq >= L) {
    if (role == 0) write_empty_rows(p, wi.bh, myq, g, D);
  } else if (myq < N) {
    const float inv = 1.f / l_run;
    bf16* orow = (bf16*)p.o + ((size_t)wi.bh * N + myq) * D + role * DH;
#pragma unroll
    for (int db = 0; db < DH / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int col = db * 32 + 8 * a + 4 * g;
        const uint32_t lo = pack_bf16(o[db][4 * a] * inv, o[db][4 * a + 1] * inv);
        const uint32_t hi = pack_bf16(o[db][4 * a + 2] * inv, o[db][4 * a + 3] * inv);
        *(i32x2*)(orow + col) = i32x2{(int)lo, (int)hi};
      }
    if (p.lse && g == 0 && role == 0) p.lse[(size_t)wi.bh * N + myq] = (m_ref + fast_log2(l_run)) * kLn2;
  }
}

template <int D, bool CAUSAL, bool PERSIST, bool MASK>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_pairs_kernel(FwdParams p) {
  if constexpr (PERSIST) {
    const PersistentMap pm = persistent_map(blockIdx.x, gridDim.x, p.total, p.remap, p.group_items);
    for (int r = 0;; ++r) {
      const int w = persistent_item(pm, r);
      if (w < 0) break;
      if (r > 0) __syncthreads();
      fwd_bf16_pairs_kernel_item<D, CAUSAL, MASK>(p, item_of(w, p.n_qt));
    }
  } else {
    fwd_bf16_pairs_kernel_item<D, CAUSAL, MASK>(p, map_work(blockIdx.x, p.total, p.n_qt, p.remap, p.group_items));
  }
}

// ========================================================== fp32 ==========
// fp32 inputs on the fp32 MFMA (32x32x2); probabilities stay fp32.  The fp32
// matrix rate is a sixteenth of bf16's, so one wave walking every key of its
// rows is slow: NW waves share one block of 32 rows and split its key tiles
// (wave w takes tiles w, w + NW, ...), each keeping its own running max, sum
// and O; at the end the partial states are merged through LDS (the same
// rescaling as between tiles).  A wave stages its tiles in its own LDS region
// (K as rows, V transposed), loading the next tile into registers while it
// computes on the current one, so no barrier couples the waves until the
// merge.  Eight waves (two a SIMD, one workgroup a CU) when the items fit on
// the GPU at once, so the longest rows finish sooner; four (two workgroups a
// CU) otherwise.
__device__ __forceinline__ f32x4 ld_f32x4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <int D, int NW_>
struct F32Cfg {
  static constexpr int NW = NW_, NT = NW * 64;
  static constexpr int BR = 32;
  static constexpr int BC = 32;
  static constexpr int KS = D + 4;          // K row stride (floats)
  static constexpr int VS = BC + 4;         // V^T row stride (floats)
  static constexpr int KBUF = BC * KS;      // floats
  static constexpr int VBUF = D * VS;
  static constexpr int WBUF = KBUF + VBUF;  // one wave's region
  static constexpr int CPR = D / 4;         // 16-byte chunks per row
  static constexpr int KCH = BC * CPR / 64; // K chunks per lane
  static constexpr int VBT = (BC / 4) * (D / 4) / 64;   // 4x4 V blocks per lane
  static constexpr int MOFF = (D / 32) * 16 * 64;                 // merge record: O, then m and l
  static constexpr int PART = MOFF + 2 * 64;
  static_assert(BC * CPR % 64 == 0 && (BC / 4) * (D / 4) % 64 == 0, "tile must split evenly");
  static_assert(PART <= WBUF, "merge record must fit the wave's region");
};

template <int D, bool CAUSAL, int NW_>
__global__ __launch_bounds__(NW_ * 64) void fwd_f32_kernel(FwdParams p) {
  using C = F32Cfg<D, NW_>;
  constexpr int BC = C::BC, NW = C::NW;
  __shared__ __attribute__((aligned(16))) float smem[NW * C::WBUF];

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const WorkItem wi = map_work(blockIdx.x, p.total, p.n_qt, p.remap, p.group_items);
  const int N = p.N;
  const int b = wi.bh / p.H, h = wi.bh - b * p.H;
  const int bkv = b * p.H_kv + h / (p.H / p.H_kv);
  const float* qg = (const float*)p.q + (size_t)wi.bh * N * D;
  const float* kg = (const float*)p.k + (size_t)bkv * N * D;
  const float* vg = (const float*)p.v + (size_t)bkv * N * D;
  const int q0 = wi.qt * C::BR;
  const int myq = q0 + lr;
  const int kv_end = CAUSAL ? min(N, q0 + C::BR) : N;
  const int n_tiles = (kv_end + BC - 1) / BC;
  float* kl = smem + wid * C::WBUF;
  float* vt = kl + C::KBUF;

  // Loads go through buffer resources sized to the valid rows, so rows past
  // N read as zeros without a branch.
  // slot (kb4, e, g) <-> column kb4*8 + 4g + e
  f32x4 qr[D / 8];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qg + (size_t)q0 * D, min(N - q0, C::BR) * D * 4);
#pragma unroll
    for (int kb = 0; kb < D / 8; ++kb) qr[kb] = ld_f32x4(rq, (lr * D + kb * 8 + 4 * g) * 4);
  }
  const float c = p.scale_log2;
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  f32x4 kreg[C::KCH];
  f32x4 vreg[C::VBT][4];
  auto load_tile = [&](int j) {
    const int key0 = j * BC;
    const int bytes = min(N - key0, BC) * D * 4;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + (size_t)key0 * D, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + (size_t)key0 * D, bytes);
#pragma unroll
    for (int it = 0; it < C::KCH; ++it) {
      const int cidx = lane + it * 64;
      const int row = cidx / C::CPR, col = cidx - row * C::CPR;
      kreg[it] = ld_f32x4(rk, (row * D + col * 4) * 4);
    }
#pragma unroll
    for (int it = 0; it < C::VBT; ++it) {
      const int blk = lane + it * 64;
      const int kq = blk % (BC / 4), cc = blk / (BC / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) vreg[it][r] = ld_f32x4(rv, ((kq * 4 + r) * D + cc * 4) * 4);
    }
  };
  // (the wave's own LDS ops run in order, so these writes land after the
  // reads of the tile before)
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < C::KCH; ++it) {
      const int cidx = lane + it * 64;
      const int row = cidx / C::CPR, col = cidx - row * C::CPR;
      *(f32x4*)(kl + row * C::KS + col * 4) = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < C::VBT; ++it) {
      const int blk = lane + it * 64;
      const int kq = blk % (BC / 4), cc = blk / (BC / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *(f32x4*)(vt + (cc * 4 + e) * C::VS + kq * 4) =
            f32x4{vreg[it][0][e], vreg[it][1][e], vreg[it][2][e], vreg[it][3][e]};
    }
  };

  if (wid < n_tiles) {
    load_tile(wid);
    store_tile();
  }
  for (int j = wid; j < n_tiles; j += NW) {
    if (j + NW < n_tiles) load_tile(j + NW);
    const int key0 = j * BC;
    f32x16 s[BC / 32];
#pragma unroll
    for (int kb32 = 0; kb32 < BC / 32; ++kb32) {
      f32x16 acc = {};
      const float* krow = kl + (kb32 * 32 + lr) * C::KS + 4 * g;
#pragma unroll
      for (int kb = 0; kb < D / 8; ++kb) {
        const f32x4 a = *(const f32x4*)(krow + kb * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma_f32(a[e], qr[kb][e], acc);
      }
      s[kb32] = acc;
    }
    // Every row of the block sees key key0 of each tile it visits (causal
    // tiles start at or before the block's first row), so m stays finite.
    const bool need_mask = (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > q0);
    if (need_mask) {
#pragma unroll
      for (int kb32 = 0; kb32 < BC / 32; ++kb32)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb32 * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if ((CAUSAL && key > myq) || key >= N) s[kb32][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb32 = 0; kb32 < BC / 32; ++kb32)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb32][r]);
    mx = max_halves(mx);
    const float m_cand = mx * c;
    if (__any(m_cand > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, m_cand);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    }
    float ts = 0.f;
#pragma unroll
    for (int kb32 = 0; kb32 < BC / 32; ++kb32)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(fmaf(s[kb32][r], c, -m_run));
        s[kb32][r] = e;
        ts += e;
      }
    l_run += ts;
    // O^T += V^T P^T: MFMA (kb32, r) takes key kb32*32 + 8*(r/4) + 4g + r%4
#pragma unroll
    for (int kb32 = 0; kb32 < BC / 32; ++kb32)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const f32x4 va = *(const f32x4*)(vt + (db * 32 + lr) * C::VS + kb32 * 32 + 8 * a4 + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[db] = mfma_f32(va[e], s[kb32][4 * a4 + e], o[db]);
        }
    if (j + NW < n_tiles) store_tile();
  }

  // Merge: each wave leaves (m, l, O) in its region, lane by lane in register
  // order (a wave with no tile leaves m = -inf, l = 0, O = 0, weight 0); the
  // waves then share the groups of four register slots of every lane.
  constexpr int MOFF = C::MOFF;
  {
    float* rec = smem + wid * C::WBUF;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) rec[(db * 16 + r) * 64 + lane] = o[db][r];
    rec[MOFF + lane] = m_run;
    rec[MOFF + 64 + lane] = sum_halves(l_run);
  }
  __syncthreads();
  float m_w[NW], mt = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    m_w[w] = smem[w * C::WBUF + MOFF + lane];
    mt = fmaxf(mt, m_w[w]);
  }
  float f_w[NW], l_tot = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    f_w[w] = fast_exp2(m_w[w] - mt);
    l_tot += f_w[w] * smem[w * C::WBUF + MOFF + 64 + lane];
  }
  if (myq < N) {
    const float inv = 1.f / l_tot;
    float* orow = (float*)p.o + ((size_t)wi.bh * N + myq) * D;
    constexpr int NGRP = (D / 32) * 4;
    static_assert(NGRP % NW == 0, "slot groups must split evenly over the waves");
#pragma unroll
    for (int i = 0; i < NGRP / NW; ++i) {
      const int q = wid + NW * i, db = q >> 2, a = q & 3;
      f32x4 acc = {};
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += f_w[w] * smem[w * C::WBUF + (db * 16 + 4 * a + e) * 64 + lane];
      *(f32x4*)(orow + db * 32 + 8 * a + 4 * g) = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    }
    if (p.lse && g == 0 && wid == 0) p.lse[(size_t)wi.bh * N + myq] = (mt + fast_log2(l_tot)) * kLn2;
  }
}

// ========================================================= launchers ======
static void finish_grid(FwdParams& p, int br) {
  p.n_qt = (p.N + br - 1) / br;
  p.total = p.B * p.H * p.n_qt;
  // A contiguous eighth of the heads can be whole sequences; with a padding
  // mask their lengths differ, so the (batch, K/V head) groups are dealt to
  // the XCDs in turn instead.
  const int groups = p.B * p.H_kv;
  p.group_items = (p.H / p.H_kv) * p.n_qt;
  p.remap = p.seqlens ? (groups % 8 == 0 ? 2 : 0) : (p.total % 8 == 0 ? 1 : 0);
}

// Compute units of the current device, read once per device.
static int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Launch one workgroup per item, or, when the items outnumber what the GPU
// holds at once, a persistent grid of (resident workgroups per CU) x CUs
// that loops over them.  `persistent` and `direct` are the two instances of
// the same kernel; residency is read once per kernel and device.
template <typename KP, typename KD>
static hipError_t launch_items(KP persistent, KD direct, int threads, FwdParams& p, hipStream_t s,
                               std::atomic<int>* occ_cache) {
  const int cus = cu_count();
  int occ = 0;
  if (cus > 0) {
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
      occ = occ_cache[dev].load(std::memory_order_relaxed);
      if (occ == 0 &&
          hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, persistent, threads, 0) == hipSuccess && occ > 0)
        occ_cache[dev].store(occ, std::memory_order_relaxed);
    }
  }
  const int grid = occ > 0 ? occ * cus : 0;
  if (grid > 0 && p.total > grid) return launch_kernel(persistent, dim3(grid), dim3(threads), s, p);
  return launch_kernel(direct, dim3(p.total), dim3(threads), s, p);
}

template <int D, bool CAUSAL, int NW, int BC, int NST>
static hipError_t launch_bf16(FwdParams& p, hipStream_t s) {
  // one workgroup per item: with several workgroups resident per CU the
  // looping instance measured slower (C4 forward: 789 vs 937 TFLOP/s)
  using C = Bf16Cfg<D, NW, BC, NST>;
  finish_grid(p, C::BR);
  if (masked(p))
    return launch_kernel(fwd_bf16_kernel<D, CAUSAL, NW, BC, NST, false, true>, dim3(p.total), dim3(C::NT), s, p);
  else
    return launch_kernel(fwd_bf16_kernel<D, CAUSAL, NW, BC, NST, false, false>, dim3(p.total), dim3(C::NT), s, p);
}

template <int D, bool CAUSAL>
static hipError_t launch_sp(FwdParams& p, hipStream_t s) {
  // One workgroup per item (two resident per CU).  When the 128-row items
  // would all be resident at once, the split instance with 64-row items
  // (waves splitting the keys) halves the longest item.
  using C = Bf16Cfg<D, 4, 64, 2>;
  if ((long long)p.B * p.H * ((p.N + C::BR - 1) / C::BR) <= 2LL * cu_count()) {
    finish_grid(p, 64);
    return launch_kernel(fwd_bf16_sp_kernel<D, CAUSAL, true>, dim3(p.total), dim3(C::NT), s, p);
  }
  finish_grid(p, C::BR);
  return launch_kernel(fwd_bf16_sp_kernel<D, CAUSAL, false>, dim3(p.total), dim3(C::NT), s, p);
}

template <int D, bool CAUSAL>
static hipError_t launch_pairs(FwdParams& p, hipStream_t s) {
  // Causal: as many workgroups as fit, each looping over its share of the
  // items (C2b 0.348 vs 0.378 ms with one workgroup per item); non-causal:
  // one workgroup per item (the looping grid measured 1.5% slower).
  finish_grid(p, PairCfg<D>::BR);
  if constexpr (CAUSAL) {
    if (masked(p)) {
      static std::atomic<int> occ_m[64];
      return launch_items(fwd_bf16_pairs_kernel<D, CAUSAL, true, true>,
                          fwd_bf16_pairs_kernel<D, CAUSAL, false, true>, PairCfg<D>::NT, p, s, occ_m);
    }
    static std::atomic<int> occ[64];
    return launch_items(fwd_bf16_pairs_kernel<D, CAUSAL, true, false>,
                        fwd_bf16_pairs_kernel<D, CAUSAL, false, false>, PairCfg<D>::NT, p, s, occ);
  }
  if (masked(p))
    return launch_kernel(fwd_bf16_pairs_kernel<D, CAUSAL, false, true>, dim3(p.total), dim3(PairCfg<D>::NT), s, p);
  else
    return launch_kernel(fwd_bf16_pairs_kernel<D, CAUSAL, false, false>, dim3(p.total), dim3(PairCfg<D>::NT), s, p);
}

template <int D, bool CAUSAL, int BC, bool LATE>
static hipError_t launch_pp(FwdParams& p, hipStream_t s) {
  using C = PpCfg<D, BC, LATE>;
  finish_grid(p, C::BR);
  if (masked(p)) {
    static std::atomic<int> occ_m[64];
    return launch_items(fwd_bf16_pp_kernel<D, CAUSAL, BC, LATE, true, true>,
                        fwd_bf16_pp_kernel<D, CAUSAL, BC, LATE, false, true>, C::NT, p, s, occ_m);
  }
  static std::atomic<int> occ[64];
  return launch_items(fwd_bf16_pp_kernel<D, CAUSAL, BC, LATE, true, false>,
                      fwd_bf16_pp_kernel<D, CAUSAL, BC, LATE, false, false>, C::NT, p, s, occ);
}

// Kernel choice per (head dim, mask), from measurements on MI355X:
//  * d = 128: ping-pong, 8 waves, 64-key tiles, DMA at the start of a phase;
//  * d = 64 non-causal: ping-pong, 128-key tiles, DMA at the end of a phase;
//  * d = 64 causal: four independent waves per workgroup with 128-row tiles
//    (twice the workgroups of the ping-pong kernel: better balance for short
//    causal grids), each wave software-pipelined when there is no other mask
//    (C2a 0.103 vs 0.109 ms, C4 922 vs 893 TFLOP/s);
//  * d = 256: wave pairs splitting the columns of O (two waves a SIMD);
//  * block-sparse: four independent waves with 128-row tiles, one query
//    block per workgroup, so every step of its tile list is work for every
//    wave (the ping-pong kernel's two query blocks often need different
//    tiles; S1 forward 950 vs 784 TFLOP/s).
hipError_t launch_fwd_bf16(int d, bool causal, FwdParams& p, hipStream_t s) {
  switch (d) {
    case 64:
      if (causal && !masked(p)) return launch_sp<64, true>(p, s);
      if (p.block_mask && !causal) return launch_bf16<64, false, 4, 64, kNst64>(p, s);
      // non-causal: the pipelined kernel once its 128-row items exceed what
      // the GPU holds at once (2x16x4096: 899 vs 874 TFLOP/s), the ping-pong
      // kernel below that (C2a_nc, 512 items: 0.145 vs 0.150 ms)
      if (!masked(p) && (long long)p.B * p.H * ((p.N + 127) / 128) > 2LL * cu_count())
        return launch_sp<64, false>(p, s);
      return causal ? launch_bf16<64, true, 4, 64, kNst64>(p, s) : launch_pp<64, false, 128, true>(p, s);
    case 128:
      if (p.block_mask)
        return causal ? launch_bf16<128, true, 4, 64, 2>(p, s) : launch_bf16<128, false, 4, 64, 2>(p, s);
      return causal ? launch_pp<128, true, 64, false>(p, s) : launch_pp<128, false, 64, false>(p, s);
    case 256: return causal ? launch_pairs<256, true>(p, s) : launch_pairs<256, false>(p, s);
  }
  return hipErrorInvalidValue;
}

template <int D, bool CAUSAL>
static hipError_t launch_pp8(FwdParams& p, hipStream_t s) {
  finish_grid(p, 256);
  static std::atomic<int> occ[64];
  return launch_items(fwd_fp8_pp_kernel<D, CAUSAL, true>, fwd_fp8_pp_kernel<D, CAUSAL, false>, 512, p, s, occ);
}

hipError_t launch_fwd_fp8(int d, bool causal, FwdParams& p, hipStream_t s) {
  // the ping-pong schedule with fp8 K/V tiles (C5 1361 vs 1168 TFLOP/s for a
  // four-wave kernel that staged the tiles through registers)
  if (d == 128) return causal ? launch_pp8<128, true>(p, s) : launch_pp8<128, false>(p, s);
  return hipErrorInvalidValue;
}

template <int D, bool CAUSAL>
static hipError_t launch_f32(FwdParams& p, hipStream_t s) {
  finish_grid(p, 32);
  // (C1, 256 items on 256 CUs: 24 us with eight waves, 25 with four; with
  // several items a CU four waves measured 6-16% faster)
  if (p.total <= cu_count())
    return launch_kernel(fwd_f32_kernel<D, CAUSAL, 8>, dim3(p.total), dim3(512), s, p);
  else
    return launch_kernel(fwd_f32_kernel<D, CAUSAL, 4>, dim3(p.total), dim3(256), s, p);
}

hipError_t launch_fwd_f32(int d, bool causal, FwdParams& p, hipStream_t s) {
  if (d == 64) return causal ? launch_f32<64, true>(p, s) : launch_f32<64, false>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
