// Host-side planning of the decode (KV-cache) split: how many waves share the
// cache read and how much workspace their partial results take.  Kept apart
// from the kernels so the C ABI's validation and sizing build and run on a
// machine without a GPU (and under host sanitizers).
#include <stddef.h>

#include "fa_kernels.hpp"

namespace fa {

// Waves: one pass of the chip (every resident wave slot of the 256 CUs of
// MI355X), and at least one per unit; one partial slot per wave.
KvPlan kv_plan(int B, int H, int H_kv, int Nq, int Nkv, int d) {
  KvPlan pl{};
  int nw = 0, nst = 0;
  switch (d) {
    case 64: nw = KvCfg<64>::NW; nst = KvCfg<64>::NST; break;
    case 128: nw = KvCfg<128>::NW; nst = KvCfg<128>::NST; break;
    case 256: nw = KvCfg<256>::NW; nst = KvCfg<256>::NST; break;
    default: return pl;
  }
  constexpr int kCUs = 256, kLds = 160 * 1024, kBC = 32;
  const long long wg_lds = (long long)nw * nst * 2 * kBC * d * 2;
  pl.nw = nw;
  pl.G = H / H_kv;
  pl.R = pl.G * Nq;
  pl.n_rg = (pl.R + 31) / 32;
  pl.R_pad = pl.R < 32 ? pl.R : 32;
  const long long units = (long long)B * H_kv * pl.n_rg;
  long long W = kCUs * (kLds / wg_lds) * nw;
  if (W < units) W = (units + nw - 1) / nw * nw;
  pl.W = W;
  pl.max_tiles = units * ((Nkv + kBC - 1) / kBC);
  const size_t rows = (size_t)W * pl.R_pad;
  pl.lse_bytes = (rows * sizeof(float) + 255) & ~(size_t)255;
  pl.ws_bytes = pl.lse_bytes + rows * d * sizeof(float);
  return pl;
}

}  // namespace fa
