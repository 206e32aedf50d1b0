// Device helpers shared by the gfx950 attention kernels: MFMA wrappers,
// bf16/fp8 packing, cross-half-wave exchange and the work-item map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The running max is only moved when a tile's max exceeds it by more than
// this many powers of two, so most tiles skip the rescale of the output;
// probabilities then stay below 2^kRescaleSlack, far inside fp32/bf16 range.
constexpr float kRescaleSlack = 8.0f;
// Bound on one lane's partial row sum of a tile's probabilities taken against
// a stale running max (each term is then at most 2^12).
constexpr float kSumBound = 4096.0f;

// ---------------------------------------------------------------- MFMA ----
// 32x32 output tile, fp32 accumulate.  Output layout (all 32x32 shapes):
// lane l holds column (l & 31); register r holds row 8*(r/4) + 4*(l/32) + r%4.
// Operand layout: lane l holds row/column (l & 31) and k-slots
// [(l/32)*KL, (l/32)*KL + KL) where KL is the per-lane k count; A and B use
// the same slot numbering, so any consistent slot->k map gives the same sum.
__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
// 32x32x64 fp8 (OCP e4m3) x fp8; 32 codes per lane per operand.
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// ---------------------------------------------------------- conversions ---
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v;
  v[0] = (bf16)lo;
  v[1] = (bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------- exchanges -----
// Combine a value across lane l and lane l^32 (the two halves of a wave hold
// different keys of the same query row).  v_permlane32_swap with the same
// register as both operands leaves, in every lane, its own value in one
// result and its partner's in the other, so one op combines the pair.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ------------------------------------------------------------ LDS I/O -----
typedef __attribute__((address_space(3))) void lds_void_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// Transposing LDS read of 16-bit elements.  Within each group of 16 lanes,
// lane s supplies the address of 4 consecutive elements; lane i receives
// element (i % 4) of the rows addressed by lanes 4j + i/4, j = 0..3.  With
// lanes 4j+q pointing at row r0+j, columns c0+4q.., lane i gets column c0+i
// of rows r0..r0+3: a 4 x 16 block arrives transposed.
__device__ __forceinline__ bf16x4 lds_read_tr16(const void* lds) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)lds);
  return __builtin_bit_cast(bf16x4, v);
}
// The same DMA through a buffer resource: base and byte range in SGPRs, a
// 32-bit per-lane offset; bytes past num_records read as zero, so a ragged
// last tile needs no clamping and the address math costs no VALU work.
// (The byte range is checked against the per-lane offset; the scalar offset
// is always passed as 0.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, num_bytes, 0x00020000);
}
template <int IMM>
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, int voff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_wave_base, 16, voff, 0, IMM, 0);
}
// The same with the non-temporal cache policy (nt): for data read exactly
// once, such as a KV cache in decode.  Measured on MI355X, streaming reads
// reach ~7.0 TB/s this way against ~6.1 TB/s with the default policy.
__device__ __forceinline__ void dma16_buf_nt(__amdgpu_buffer_rsrc_t r, int voff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_wave_base, 16, voff, 0, 0, 2);
}
// 4 bytes per lane into LDS (lds + 4*l), through a buffer resource.
__device__ __forceinline__ void dma4_buf(__amdgpu_buffer_rsrc_t r, int voff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_wave_base, 4, voff, 0, 0, 0);
}
// XOR swizzle for tiles read both as rows (16 bytes per lane, 16 consecutive
// rows per clock) and through the transposing read (4 rows x 32 bytes per 16
// lanes): row bits go to distinct unit bits so both patterns spread over all
// 64 banks.  Rows of 128 bytes alternate bank halves by themselves.
template <int RB>
__device__ __forceinline__ int rt_swz(int row, int u) {
  return RB == 128 ? (u ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3)))
                   : (u ^ (((row & 1) << 3) | ((row & 2) << 1) | ((row >> 2) & 3)));
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Workgroup barrier for LDS stages: each wave's own LDS reads and writes
// complete first, but its global loads (LDS-DMA prefetches of later tiles,
// waited for separately by count) stay in flight.  A memory fence would make
// the compiler wait for every LDS-DMA write as well, so the barrier is a bare
// s_barrier whose "memory" clobber keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N of this wave's vector-memory operations are in flight
// (they complete in issue order), N a compile-time constant < 64.
template <int N>
__device__ __forceinline__ void wait_vmem_upto() {
  // s_waitcnt encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | (((N >> 4) & 3) << 14));
}
// XOR swizzles of the 16-byte units of a K or V row in LDS (the DMA writes
// rows unpadded).  They were chosen by measuring the operand reads on MI355X
// (rocprof-free microbenchmarks of the exact access patterns):
//  * K operand reads (16 bytes per lane, lanes 0-15 on rows r..r+15 of one
//    logical unit): row bit 0 -> unit bit 3, row bits 1-3 -> unit bits 0-2
//    reaches the full LDS rate; XOR with (r & 15) loses ~25%.  Rows of 128
//    bytes already alternate bank halves, so there u ^ ((r >> 1) & 7).
//  * transposing V reads (4 rows x 32 bytes per 16 lanes): row bit 0 -> unit
//    bit 3, row bit 1 -> unit bit 2 (128-byte rows: row bit 1 -> unit bit 2).
template <int RB>
__device__ __forceinline__ int k_swz(int row, int u) {
  return RB == 128 ? (u ^ ((row >> 1) & 7)) : (u ^ ((row >> 1) & 7) ^ ((row & 1) << 3));
}
template <int RB>
__device__ __forceinline__ int v_swz(int row, int u) {
  return RB == 128 ? (u ^ (((row >> 1) & 1) << 2)) : (u ^ (((row & 1) << 3) | ((row & 2) << 1)));
}

// Global byte offsets of a wave's 16-byte LDS-DMA copies of a tile of rows
// of RB bytes stored row-swizzled (kind S: rt_swz, k_swz or v_swz).  The
// wave copies KBs k0 .. k0 + n - 1 (n a power of two dividing k0); each
// swizzle XORs row bits into unit bits, and the row bits that change with i
// (i * 1024 / RB) never overlap those from the lane or from k0, so copy i is
// at copy 0's offset XOR a constant, plus i KB: one register serves all of
// the wave's copies.  (The empty asm hides the base's value, so the compiler
// forms each offset where it is used instead of keeping all of them live.)
enum { kSwzRt = 0, kSwzK = 1, kSwzV = 2 };
template <int RB, int S>
__device__ __forceinline__ int swz_of(int row, int u) {
  if constexpr (S == kSwzRt) return rt_swz<RB>(row, u);
  else if constexpr (S == kSwzK) return k_swz<RB>(row, u);
  else return v_swz<RB>(row, u);
}
template <int RB, int S>
__device__ __forceinline__ int dma_base(int k0, int lane) {
  const int byte = k0 * 1024 + lane * 16;
  const int row = byte / RB, pu = (byte % RB) / 16;
  return row * RB + swz_of<RB, S>(row, pu) * 16;
}
template <int RB, int S>
__device__ __forceinline__ int dma_off(int base, int i) {
  asm volatile("" : "+v"(base));
  return (base ^ (swz_of<RB, S>(i * (1024 / RB), 0) * 16)) + i * 1024;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ----------------------------------------------------------- work map -----
// Work item -> (head, q-tile).  Workgroups are handed to the 8 XCDs round
// robin (id % 8), each XCD with its own L2.  Items are numbered head-major,
// and the heads of one (batch, K/V head) group -- group_items consecutive
// items -- share that group's K/V.  The map keeps whole groups on one XCD so
// they share its L2:
//   remap 1  each XCD takes a contiguous eighth of the items;
//   remap 2  XCD x takes groups x, x + 8, x + 16, ... (for sequences of
//            different lengths, so that every XCD gets a mix of them);
//   remap 3  as remap 1, with the XCD's units of group_items consecutive
//            items taken in turn (unit 0's first item, unit 1's first, ...,
//            then every unit's second): the units' heaviest causal tiles
//            all come first, so the dispatcher, which hands an XCD's
//            workgroups to its CUs in order as they free up, pairs heavy
//            with light (one unit after another left a CU that drew only
//            heavy tiles at the end: the GQA prefill backward's dK/dV pass
//            reached 68% of an even split in a dispatch model);
//   remap 0  no map (the counts do not divide by 8).
// Inside a head the heaviest causal tiles (largest q-tile index) come first.
struct WorkItem {
  int bh;
  int qt;
};
// The item at position s of XCD x's share (total % 8 == 0).
__device__ __forceinline__ int xcd_item(int x, int s, int total, int group_items, int remap) {
  if (remap == 2) {
    const int gl = s / group_items, within = s - gl * group_items;
    return (x + 8 * gl) * group_items + within;
  }
  if (remap == 3) {
    const int per = total >> 3, units = per / group_items;
    const int k = s / units;
    return x * per + (s - k * units) * group_items + k;
  }
  return x * (total >> 3) + s;
}
__device__ __forceinline__ WorkItem map_work(int block, int total, int n_qt, int remap, int group_items) {
  const int w = remap ? xcd_item(block & 7, block >> 3, total, group_items, remap) : block;
  WorkItem it;
  it.bh = w / n_qt;
  it.qt = n_qt - 1 - (w - it.bh * n_qt);
  return it;
}

// Persistent grid: `workers` workgroups (one per CU) each loop over several
// work items, so no workgroup ever waits for the dispatcher (which issues in
// order and, with causal tiles of uneven length, stalls on a busy XCD while
// other CUs idle).  With a map (remap != 0) each XCD's share of the items (as
// above) is worked by that XCD's workers (workgroup b runs on XCD b % 8);
// otherwise all workers share all items.  Worker c takes one item per round
// in snake order (c, then L-1-c, ...), which balances uneven causal work and
// keeps an XCD on one or two heads at a time.
struct PersistentMap {
  int x, per;      // XCD and size of this worker's share
  int L, c;        // workers sharing it, this worker's index among them
  int remap, group_items, total;
};
__device__ __forceinline__ PersistentMap persistent_map(int block, int workers, int total, int remap,
                                                        int group_items) {
  PersistentMap m;
  m.group_items = group_items;
  m.total = total;
  if (remap && total % 8 == 0 && workers % 8 == 0) {
    m.x = block & 7;
    m.per = total >> 3;
    m.L = workers >> 3;
    m.c = block >> 3;
    m.remap = remap;
  } else {
    m.x = 0;
    m.per = total;
    m.L = workers;
    m.c = block;
    m.remap = 0;
  }
  return m;
}
// Block-sparse attention (128 x 128 blocks, mask [H][nb][nb] of bytes): a
// workgroup runs its tile loop over a list of only the key tiles that some
// of its rows need, so a tile whose key block is off for all of them costs
// nothing (no load, no step, no barrier).  Wave 0 reads query blocks
// qb .. qb + ROWS - 1 of head h and writes, in key order, 4 t + f for each
// key tile t (BC keys) in [t_first, t_first + n_all) with f != 0, bit r of
// f set when query block qb + r has t's key block on; every wave of the
// workgroup gets the count.  kMaxTiles bounds the list (N <= 131072 with
// 64-key tiles).
constexpr int kMaxTiles = 2048;
template <int BC, int ROWS>
__device__ __forceinline__ int list_tiles(const unsigned char* block_mask, int nb, int h, int qb, int t_first,
                                          int n_all, unsigned short* list, int* count) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const unsigned char* row = block_mask + ((size_t)h * nb + qb) * nb;
    int n = 0;
    for (int base = 0; base < n_all; base += 64) {   // uniform trip count: every lane votes
      const int t = t_first + base + lane;
      int f = 0;
      if (base + lane < n_all) {
        const int kb = (t * BC) >> 7;
        f = row[kb] != 0;
        if (ROWS == 2 && qb + 1 < nb) f |= (row[nb + kb] != 0) << 1;
      }
      const unsigned long long bal = __ballot(f != 0);
      if (f) list[n + __popcll(bal & ((1ull << lane) - 1))] = (unsigned short)(4 * t + f);
      n += __popcll(bal);
    }
    if (lane == 0) *count = n;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*count);
}
// Item of round r for this worker, or -1 when its share is done.
__device__ __forceinline__ int persistent_item(const PersistentMap& m, int r) {
  const int j = r * m.L + ((r & 1) ? m.L - 1 - m.c : m.c);
  if (j >= m.per) return -1;
  return m.remap ? xcd_item(m.x, j, m.total, m.group_items, m.remap) : j;
}
__device__ __forceinline__ WorkItem item_of(int w, int n_qt) {
  WorkItem it;
  it.bh = w / n_qt;
  it.qt = n_qt - 1 - (w - it.bh * n_qt);
  return it;
}

}  // namespace fa
