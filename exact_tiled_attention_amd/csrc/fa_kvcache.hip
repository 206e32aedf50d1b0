// Attention of a few new queries against a long KV cache (decode), gfx950.
//
// With one (or a few) queries per head the score matrix is a handful of rows
// and the kernel's cost is reading the cache: every K and V row is read once
// and used by the G * N_q query rows of its GQA group, a few flops per byte,
// far below the MFMA/HBM ridge.  So the work is split over the cache
// instead of over queries -- the split of the KV-cache read across thread
// blocks that "FlashAttentionとは？…" describes for decode (短い系列の効果と
// デコード向け最適化の違い) -- into enough independent pieces to keep every CU's
// memory pipe full, and a second kernel merges the pieces.
//
// Split kernel.  One wave owns all query rows of one GQA group (32 rows per
// row group: row r = g * N_q + i is query i of the group's head g) and one
// contiguous chunk of the cache.  It streams its chunk through its own LDS
// stages by DMA, 32 keys per tile, NST tiles deep, with no workgroup barrier:
// each wave waits only for its own loads, so a slow wave never holds up
// another.  Per tile it forms S^T = K Q^T with one MFMA chain (one query row
// per lane, as in the prefill kernels), masks, applies the online softmax and
// adds P V into an fp32 accumulator.  It writes its chunk's normalised output
// and base-2 logsumexp to the workspace.
//
// Combine kernel.  Per query row, the chunk results (O_s, lse_s) merge as
//   lse = log2 sum_s 2^lse_s,   O = sum_s 2^(lse_s - lse) O_s,
// the same rescaling the online softmax applies between tiles ("Flash
// Attentionとは？…", 最大値と正規化項を持ち回るオンラインsoftmaxの再スケール),
// here between chunks.
//
// Masking: batch b uses the first kv_len[b] cache rows (clamped to
// [0, N_kv]); the N_q queries are the last N_q positions, so under the causal
// mask query i sees keys 0 .. kv_len - N_q + i.  A row that sees no key gets
// O = 0 and LSE = -inf.
#include <stdint.h>

#include <type_traits>

#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {


template <int D>
struct KvTile {
  static constexpr int NW = KvCfg<D>::NW, NST = KvCfg<D>::NST;
  static constexpr int BC = 32;              // keys per tile
  static constexpr int RB = D * 2;           // bytes per K/V row
  static constexpr int TILE = BC * RB;       // bytes of one K (or V) tile
  static constexpr int IPT = TILE / 1024;    // 1 KB DMA issues per tile and tensor
  static constexpr int STAGE = 2 * TILE;     // K tile, then V tile
  static_assert(NST >= 2 && NST <= 4, "two to four stages");
  // vmcnt field: all later tiles plus this tile's V may be outstanding
  static_assert((NST - 1) * 2 * IPT + IPT < 64, "DMA count must fit the vmcnt field");
};

__device__ __forceinline__ int cache_len(const KvParams& p, int b) {
  return p.kv_len ? min(max(p.kv_len[b], 0), p.Nkv) : p.Nkv;
}

// ---------------------------------------------------------- work split -----
// A unit is (batch, K/V head, 32-row query group); batch b's units each hold
// t_b = ceil(len_b / 32) tiles of 32 keys, T tiles in all.  Of the W waves
// launched (at least one per unit), each unit gets one, and the E = W - U
// others are shared out in proportion to tiles: a unit of batch b is cut
// into n_b = 1 + floor(t_b E / T) near-equal pieces, one per wave.  The
// pieces of all units are then about T / E tiles whatever the mix of cache
// lengths, so a ragged batch keeps every CU busy.  The lengths live on the
// device; every wave and the combine derive the same partition from them.
__device__ __forceinline__ int batch_tiles(const KvParams& p, int b) {
  return (cache_len(p, b) + 31) >> 5;
}
// Wave-wide inclusive prefix sum of one int per lane.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off, 64);
    if (lane >= off) v += y;
  }
  return v;
}
struct KvSplit {
  int total;   // T: tiles of all units
  int extra;   // E: waves beyond one per unit
};
__device__ __forceinline__ KvSplit kv_split(const KvParams& p) {
  const int lane = threadIdx.x & 63;
  int total = 0;
  if (!p.kv_len) {                             // every cache full: no scan
    KvSplit sp;
    sp.total = p.B * p.upb * ((p.Nkv + 31) >> 5);
    sp.extra = min(p.W - p.B * p.upb, sp.total / kKvMinTiles);
    return sp;
  }
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int b = b0 + lane;
    int v = b < p.B ? batch_tiles(p, b) * p.upb : 0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    total += v;
  }
  // the same in every lane; readfirstlane lets the compiler keep it in an SGPR
  KvSplit sp;
  sp.total = __builtin_amdgcn_readfirstlane(total);
  sp.extra = min(p.W - p.B * p.upb, sp.total / kKvMinTiles);
  return sp;
}
__device__ __forceinline__ int pieces_of(const KvSplit& sp, int tiles) {
  return sp.total > 0 ? 1 + (int)((long long)tiles * sp.extra / sp.total) : 1;
}
// Batch of wave w and the first wave of that batch; bt = B when w is past
// the last batch's waves.
__device__ __forceinline__ void wave_batch(const KvParams& p, const KvSplit& sp, int w, int& bt, int& first) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  bt = p.B;
  first = 0;
  if (!p.kv_len) {
    const int per = pieces_of(sp, (p.Nkv + 31) >> 5) * p.upb;
    bt = min(w / per, p.B);
    first = bt * per;
    return;
  }
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int b = b0 + lane;
    const int v = b < p.B ? pieces_of(sp, batch_tiles(p, b)) * p.upb : 0;
    const int incl = wave_incl_scan(v);
    const unsigned long long hit = __ballot(b < p.B && base + incl - v <= w && w < base + incl);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      bt = b0 + l;
      first = base + __shfl(incl - v, l, 64);
      return;
    }
    base += __shfl(incl, 63, 64);
  }
}
// First wave of batch bt.
__device__ __forceinline__ int batch_first_wave(const KvParams& p, const KvSplit& sp, int bt) {
  const int lane = threadIdx.x & 63;
  int base = 0, first = 0;
  if (!p.kv_len) return bt * pieces_of(sp, (p.Nkv + 31) >> 5) * p.upb;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int b = b0 + lane;
    const int v = b < p.B ? pieces_of(sp, batch_tiles(p, b)) * p.upb : 0;
    const int incl = wave_incl_scan(v);
    if (bt >= b0 && bt < b0 + 64) first = base + __shfl(incl - v, bt - b0, 64);
    base += __shfl(incl, 63, 64);
  }
  return first;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(KvCfg<D>::NW * 64) void kv_split_kernel(KvParams p) {
  using T = KvTile<D>;
  constexpr int NW = T::NW, NST = T::NST, BC = T::BC, RB = T::RB, IPT = T::IPT;
  // One array per stage: the compiler then sees that a DMA into one stage
  // never aliases the reads of another and waits only for what it must.
  __shared__ __attribute__((aligned(1024))) unsigned char st0[NW * T::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[NW * T::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[NST > 2 ? NW * T::STAGE : 1];
  __shared__ __attribute__((aligned(1024))) unsigned char st3[NST > 3 ? NW * T::STAGE : 1];

  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lr = lane & 31, g = lane >> 5;
  const int w = blockIdx.x * NW + wid;
  const KvSplit sp = kv_split(p);
  int b, first;
  wave_batch(p, sp, w, b, first);
  // wave-uniform values: in SGPRs the buffer descriptors built from them need
  // no per-lane (waterfall) handling
  b = __builtin_amdgcn_readfirstlane(b);
  first = __builtin_amdgcn_readfirstlane(first);
  if (b >= p.B) return;                      // a wave past the last piece
  const int L = cache_len(p, b);
  const int tb = (L + 31) >> 5;
  const int nb = pieces_of(sp, tb);
  const int j = (w - first) / nb;            // unit within the batch
  const int piece = w - first - j * nb;
  const int lo = (int)((long long)piece * tb / nb), hi = (int)((long long)(piece + 1) * tb / nb);
  if (lo >= hi) return;                      // an empty piece: the combine skips it

  // Per-lane LDS offsets, fixed for every tile.
  int dma_k[IPT], dma_v[IPT];
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int byte = i * 1024 + lane * 16;
    const int row = byte / RB, pu = (byte % RB) / 16;
    dma_k[i] = row * RB + k_swz<RB>(row, pu) * 16;   // the swizzles are involutions
    dma_v[i] = row * RB + v_swz<RB>(row, pu) * 16;
  }
  constexpr int NKO = D / 16 < 8 ? D / 16 : 8, NVO = D / 32 < 4 ? D / 32 : 4;
  int koff[NKO];
#pragma unroll
  for (int kb = 0; kb < NKO; ++kb) koff[kb] = lr * RB + k_swz<RB>(lr, 2 * kb + g) * 16;
  const int s16 = lane & 15, G4 = lane >> 4;
  const int vrow = 4 * (G4 >> 1) + (s16 >> 2);
  int voff[NVO];
#pragma unroll
  for (int db = 0; db < NVO; ++db)
    voff[db] = vrow * RB + v_swz<RB>(vrow, db * 4 + 2 * (G4 & 1) + ((s16 & 3) >> 1)) * 16 + (s16 & 1) * 8;
  auto stage = [&](int u) -> unsigned char* {
    unsigned char* base = u == 0 ? st0 : (NST == 2 || u == 1 ? st1 : (NST == 3 || u == 2 ? st2 : st3));
    return base + wid * T::STAGE;
  };
  const float c = p.scale_log2;

  // This wave's piece: tiles [lo, hi) of unit j (= kv head * n_rg + row
  // group) of batch b; its result goes to partial slot w.
  {
    const int kvh = j / p.n_rg, rg = j - kvh * p.n_rg;
    const int bkv = b * p.H_kv + kvh;
    const int k_begin = lo * BC;
    const int n_t = hi - lo;

    // This lane's query row; lanes past the group's rows compute on zeros.
    const int r = rg * 32 + lr;
    const bool row_ok = r < p.R;
    const int gi = row_ok ? r / p.Nq : 0;
    const int qi = row_ok ? r - gi * p.Nq : p.Nq - 1;
    const int h = kvh * p.G + gi;
    // last visible key of the row, and the smallest one over the group
    const int lim = CAUSAL ? min(L - p.Nq + qi, L - 1) : L - 1;
    const int lim_lo = CAUSAL ? L - p.Nq : L - 1;

    bf16x8 qr[D / 16];
    {
      const unsigned char* qrow = (const unsigned char*)p.q + (((size_t)b * p.H + h) * p.Nq + qi) * RB;
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) {
        bf16x8 x = {};
        if (row_ok) x = *(const bf16x8*)(qrow + (kb * 16 + 8 * g) * 2);
        qr[kb] = x;
      }
    }
    const unsigned char* kg = (const unsigned char*)p.k + (size_t)bkv * p.Nkv * RB;
    const unsigned char* vg = (const unsigned char*)p.v + (size_t)bkv * p.Nkv * RB;
    auto issue = [&](int t, unsigned char* st) {
      const int key0 = k_begin + t * BC;
      const int bytes = min(L - key0, BC) * RB;   // rows past the cache length read as zero
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + (size_t)key0 * RB, bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + (size_t)key0 * RB, bytes);
#pragma unroll
      for (int i = 0; i < IPT; ++i) dma16_buf_nt(rk, dma_k[i], st + i * 1024);
#pragma unroll
      for (int i = 0; i < IPT; ++i) dma16_buf_nt(rv, dma_v[i], st + T::TILE + i * 1024);
    };

    f32x16 o[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    // LATER = tiles issued after this one; their DMAs may stay in flight.
    auto consume = [&](int t, const unsigned char* kl, auto later_c) __attribute__((always_inline)) {
      constexpr int LATER = decltype(later_c)::value;
      const unsigned char* vl = kl + T::TILE;
      const int key0 = k_begin + t * BC;
      wait_vmem_upto<LATER * 2 * IPT + IPT>();          // this tile's K has landed
      f32x16 sc = {};
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) {
        const bf16x8 a = *(const bf16x8*)(kl + (kb / NKO) * 256 + koff[kb % NKO]);
        sc = mfma_bf16(a, qr[kb], sc);
      }
      if (key0 + BC - 1 > lim_lo) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int key = key0 + 8 * (q >> 2) + 4 * g + (q & 3);
          if (key > lim) sc[q] = -INFINITY;
        }
      }
      // P against the running max; the max is taken (and the output
      // rescaled) only when some lane's partial sum leaves [0, kSumBound],
      // which also catches rows that have not seen a key yet (max -inf).
      bf16x8 pk[2];
      auto expo = [&](float m) __attribute__((always_inline)) -> float {
        float tsum = 0.f;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint32_t w4[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const float e0 = fast_exp2(fmaf(sc[half * 8 + 2 * x], c, -m));
            const float e1 = fast_exp2(fmaf(sc[half * 8 + 2 * x + 1], c, -m));
            w4[x] = pack_bf16(e0, e1);
            tsum += e0 + e1;
          }
          pk[half] = __builtin_bit_cast(bf16x8, i32x4{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]});
        }
        return tsum;
      };
      float ts = expo(m_run);
      if (__any(!(ts <= kSumBound))) {
        float mx = -INFINITY;
#pragma unroll
        for (int q = 0; q < 16; ++q) mx = fmaxf(mx, sc[q]);
        mx = max_halves(mx);
        const float m_new = fmaxf(m_run, mx * c);
        // A row with no visible key so far keeps m = -inf, l = 0, O = 0; its
        // exponentials are then taken against 0 so that masked scores give 0.
        const bool none = m_new == -INFINITY;
        const float alpha = none ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
          for (int q = 0; q < 16; ++q) o[i][q] *= alpha;
        ts = expo(none ? 0.f : m_new);
      }
      l_run += ts;
      wait_vmem_upto<LATER * 2 * IPT>();                // this tile's V has landed
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const unsigned char* vb = vl + 16 * half * RB;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const unsigned char* vr = vb + (db / NVO) * 256 + voff[db % NVO];
          const bf16x4 lo4 = lds_read_tr16(vr);
          const bf16x4 hi4 = lds_read_tr16(vr + 8 * RB);
          o[db] = mfma_bf16(__builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7), pk[half], o[db]);
        }
      }
    };

    // Tile t lives in stage t % NST.  Before tile t is consumed, tile
    // t + NST - 1 is issued into the stage tile t - 1 used (its reads are
    // done: their values fed the MFMAs of tile t - 1), so NST - 1 tiles stay
    // in flight behind the one being consumed.  The last NST - 1 tiles, with
    // nothing left to issue, wait for everything.
#pragma unroll
    for (int u = 0; u < NST - 1; ++u)
      if (u < n_t) issue(u, stage(u));
    const int n_main = max(0, n_t - (NST - 1));
    for (int t0 = 0; t0 < n_main; t0 += NST) {
#pragma unroll
      for (int u = 0; u < NST; ++u) {
        const int t = t0 + u;
        if (t < n_main) {
          issue(t + NST - 1, stage((u + NST - 1) % NST));
          consume(t, stage(u), std::integral_constant<int, NST - 1>{});
        }
      }
    }
    for (int t = n_main; t < n_t; ++t) {
      wait_vmem();
      consume(t, stage(t % NST), std::integral_constant<int, 0>{});
    }

    const float l_tot = sum_halves(l_run);
    if (row_ok) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      const size_t prow = (size_t)w * p.R_pad + lr;
      float* po = p.part_o + prow * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int col = db * 32 + 8 * a + 4 * g;
          *(f32x4*)(po + col) = f32x4{o[db][4 * a] * inv, o[db][4 * a + 1] * inv, o[db][4 * a + 2] * inv,
                                      o[db][4 * a + 3] * inv};
        }
      if (g == 0) p.part_lse[prow] = l_tot > 0.f ? m_run + fast_log2(l_tot) : -INFINITY;
    }
  }

}

// One workgroup per query row: merge the partials of the row's unit, which
// are the consecutive waves that took its pieces.
template <int D>
__global__ __launch_bounds__(256) void kv_combine_kernel(KvParams p) {
  constexpr int TPS = D / 4;      // threads per partial row (4 floats each)
  constexpr int SG = 256 / TPS;   // partials read side by side
  __shared__ float sacc[SG][D];
  __shared__ float stot[SG];
  __shared__ float smx[SG];
  const int tid = threadIdx.x, dc = tid % TPS, sg = tid / TPS;
  const int bkv = blockIdx.x / p.R, r = blockIdx.x - bkv * p.R;
  const int b = bkv / p.H_kv, kvh = bkv - b * p.H_kv;
  const int gi = r / p.Nq, qi = r - gi * p.Nq;
  const int rg = r >> 5, rr = r & 31;
  const int j = kvh * p.n_rg + rg;
  const size_t orow = ((size_t)b * p.H + kvh * p.G + gi) * p.Nq + qi;

  const KvSplit sp = kv_split(p);
  const int tb = batch_tiles(p, b);
  const int nb = pieces_of(sp, tb);
  // pieces [lo, hi) with lo < hi hold tiles; with nb <= tb every piece does
  const int n_part = tb == 0 ? 0 : min(nb, tb);
  const size_t slot0 = (size_t)batch_first_wave(p, sp, b) + (size_t)j * nb;
  const float* pl = p.part_lse + slot0 * p.R_pad + rr;
  const float* po = p.part_o + (slot0 * p.R_pad + rr) * D + dc * 4;
  const size_t stride = (size_t)p.R_pad;         // rows between consecutive slots

  // One pass: each thread merges its partials online (running max m, sum of
  // weights t, weighted output acc), then the SG groups merge through LDS.
  float m = -INFINITY, t = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // (a piece whose rows saw no key has l = -inf and x = 0; while every piece
  // so far is such, mn stays -inf and nothing accumulates)
#pragma unroll 4
  for (int s = sg; s < n_part; s += SG) {
    const float l = pl[s * stride];
    const f32x4 x = *(const f32x4*)(po + s * stride * D);
    const float mn = fmaxf(m, l);
    const bool none = mn == -INFINITY;
    const float a = none ? 1.f : fast_exp2(m - mn), wgt = none ? 0.f : fast_exp2(l - mn);
    acc = acc * a + x * wgt;
    t = t * a + wgt;
    m = mn;
  }
  *(f32x4*)&sacc[sg][dc * 4] = acc;
  if (dc == 0) {
    stot[sg] = t;
    smx[sg] = m;
  }
  __syncthreads();
  if (sg == 0) {
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < SG; ++q) mx = fmaxf(mx, smx[q]);
    float tt = 0.f;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    if (mx != -INFINITY) {
#pragma unroll
      for (int q = 0; q < SG; ++q) {
        const float a = fast_exp2(smx[q] - mx);
        tt += stot[q] * a;
        sum += *(const f32x4*)&sacc[q][dc * 4] * a;
      }
    }
    const float inv = tt > 0.f ? 1.f / tt : 0.f;
    bf16* out = (bf16*)p.o + orow * D + dc * 4;
    *(i32x2*)out = i32x2{(int)pack_bf16(sum[0] * inv, sum[1] * inv), (int)pack_bf16(sum[2] * inv, sum[3] * inv)};
    if (p.lse && dc == 0) p.lse[orow] = tt > 0.f ? (mx + fast_log2(tt)) * kLn2 : -INFINITY;
  }
}

// ------------------------------------------------------------- host -------
hipError_t launch_kvcache_bf16(int d, bool causal, KvParams& p, hipStream_t s) {
  const unsigned split_blocks = (unsigned)(p.W / p.nw);
  const unsigned rows = (unsigned)((size_t)p.B * p.H_kv * p.R);
  auto run = [&](auto dc, auto cc) -> hipError_t {
    constexpr int D = decltype(dc)::value;
    constexpr bool C = decltype(cc)::value;
    if (hipError_t e = launch_kernel(kv_split_kernel<D, C>, dim3(split_blocks), dim3(KvCfg<D>::NW * 64), s, p);
        e != hipSuccess)
      return e;
    return launch_kernel(kv_combine_kernel<D>, dim3(rows), dim3(256), s, p);
  };
  using T = std::true_type;
  using F = std::false_type;
  switch (d) {
    case 64: return causal ? run(std::integral_constant<int, 64>{}, T{}) : run(std::integral_constant<int, 64>{}, F{});
    case 128: return causal ? run(std::integral_constant<int, 128>{}, T{}) : run(std::integral_constant<int, 128>{}, F{});
    case 256: return causal ? run(std::integral_constant<int, 256>{}, T{}) : run(std::integral_constant<int, 256>{}, F{});
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
