// Key/value tiles of the concatenated rows (cartridge rows, then real
// tokens) for the query-major bf16 kernels: which rows a tile holds, and the
// direct global -> LDS copy of one 64-row tile of K and V.
#pragma once

#include "common.hpp"

namespace cartattn {

constexpr int kKvTile = 64;   // rows per key tile of the query-major kernels

// Tile t of one (batch, kv head): tiles [0, n_ct) hold cartridge rows, the
// rest hold real tokens; j0 is the tile's first row in its own source and
// abs0 its position in the concatenation (cartridge row j at j, token i at
// p + i).
struct KvTile {
  int j0, rows, abs0;
  bool cart;
};

__device__ __forceinline__ KvTile kv_tile(int t, int n_ct, int p, int n) {
  KvTile f;
  f.cart = t < n_ct;
  f.j0 = f.cart ? t * kKvTile : (t - n_ct) * kKvTile;
  f.rows = f.cart ? min(kKvTile, p - f.j0) : min(kKvTile, n - f.j0);
  f.abs0 = f.cart ? f.j0 : p + f.j0;
  return f;
}

// Sliding window (window > 0): the query at position p + i sees the rows at
// positions above p + i - window. First tile holding a row that the query at
// position p + i0 (the earliest of a workgroup) can see.
__device__ __forceinline__ int first_window_tile(int window, int i0, int p, int n_ct) {
  if (window <= 0) return 0;
  const int a = p + i0 - window + 1;   // first visible position
  if (a <= 0) return 0;
  return a < p ? a / kKvTile : n_ct + (a - p) / kKvTile;
}

// Bases of one (batch, kv head)'s rows; consecutive rows are Hkv*D apart.
template <int D>
struct KvSrc {
  const bf16 *kc, *vc, *kt, *vt;
  size_t row_stride;
  int p, n;
};

// base: the sequence's first token row; n: its length.
template <int D>
__device__ __forceinline__ KvSrc<D> kv_src(const void* k_cart, const void* v_cart,
                                           const void* k_tok, const void* v_tok, int base, int n,
                                           int p, int Hkv, int kv) {
  KvSrc<D> s;
  s.kc = reinterpret_cast<const bf16*>(k_cart) + (size_t)kv * D;
  s.vc = reinterpret_cast<const bf16*>(v_cart) + (size_t)kv * D;
  s.kt = reinterpret_cast<const bf16*>(k_tok) + ((size_t)base * Hkv + kv) * D;
  s.vt = reinterpret_cast<const bf16*>(v_tok) + ((size_t)base * Hkv + kv) * D;
  s.row_stride = (size_t)Hkv * D;
  s.p = p;
  s.n = n;
  return s;
}

template <int D>
using KvMap = TileMap<D, kKvTile>;

// Issue this wave's share of the copy of tile t's K and V rows.
template <int D>
__device__ __forceinline__ void kv_issue(const KvMap<D>& m, bf16* Kst, bf16* Vst, int t,
                                         int n_ct, const KvSrc<D>& s, int wave, int lane) {
  const KvTile f = kv_tile(t, n_ct, s.p, s.n);
  const bf16* kb = (f.cart ? s.kc : s.kt) + (size_t)f.j0 * s.row_stride;
  const bf16* vb = (f.cart ? s.vc : s.vt) + (size_t)f.j0 * s.row_stride;
  dma_tile<D, kKvTile>(m, Kst, kb, s.row_stride, f.rows, wave, lane);
  dma_tile<D, kKvTile>(m, Vst, vb, s.row_stride, f.rows, wave, lane);
}

}  // namespace cartattn
