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

// The copy map of a workgroup of NWAVE waves.
template <int D, int NWAVE = 4>
using KvMap = TileMap<D, kKvTile, NWAVE>;

// The copy map of one (batch, kv head)'s rows (Hkv*D elements apart).
template <int D, int NWAVE = 4>
__device__ __forceinline__ KvMap<D, NWAVE> kv_map(int Hkv, int wave, int lane) {
  return KvMap<D, NWAVE>(wave, lane, (uint32_t)(Hkv * D * 2));
}

// The copy of one tile's K and V rows as this wave's single copy
// instructions, so that a caller can place them inside its compute:
// issue<J>() (J < N) issues copy J, the first NK of them K's blocks, the
// rest V's.
// With `on` false (no tile left to copy) every issue is a no-op.
// The buffer descriptors are built at the copy from wave-uniform values read
// from lane 0 (a descriptor carried across the branch around a tile's
// compute was otherwise taken for divergent).
template <int D, int NWAVE = 4>
struct KvCopy {
  using Map = KvMap<D, NWAVE>;
  static constexpr int NK = Map::NK;
  static constexpr int N = 2 * NK;
  const bf16 *ks, *vs;   // the tile's first K and V rows
  uint32_t bytes;        // buffer range: through the tile's last row
  bf16 *kd, *vd;
  bool on;

  template <int J>
  __device__ __forceinline__ void issue(const Map& m, int wave, int lane) const {
    static_assert(J >= 0 && J < N, "copy index");
    if (!on) return;
    if constexpr (J < NK)
      dma_block<D, kKvTile, NWAVE>(m, J, kd, uniform_rsrc(ks, bytes), wave, lane);
    else
      dma_block<D, kKvTile, NWAVE>(m, J - NK, vd, uniform_rsrc(vs, bytes), wave, lane);
  }
  // Copies LO .. HI-1.
  template <int LO, int HI>
  __device__ __forceinline__ void range(const Map& m, int wave, int lane) const {
    static_assert(0 <= LO && LO <= HI && HI <= N, "copy range");
    static_for<HI - LO>([&](auto I) { this->template issue<LO + decltype(I)::value>(m, wave, lane); });
  }
  __device__ __forceinline__ void all(const Map& m, int wave, int lane) const {
    static_for<N>([&](auto J) { this->template issue<decltype(J)::value>(m, wave, lane); });
  }
};

// Consecutive key tiles of one (batch, kv head), walked one at a time: the
// current tile's first K and V rows move by one tile per step (and to the
// first token row when the walk leaves the cartridge), so a step costs a
// few scalar adds instead of a 64-bit product per tile.
template <int D>
struct KvWalk {
  KvSrc<D> s;
  int n_ct;
  int t;               // the current tile
  const bf16 *k, *v;   // its first K and V rows

  __device__ __forceinline__ KvWalk(const KvSrc<D>& src, int n_ct_, int t0)
      : s(src), n_ct(n_ct_), t(t0) {
    const KvTile f = kv_tile(t0, n_ct, s.p, s.n);
    k = (f.cart ? s.kc : s.kt) + (size_t)f.j0 * s.row_stride;
    v = (f.cart ? s.vc : s.vt) + (size_t)f.j0 * s.row_stride;
  }
  __device__ __forceinline__ void next() {
    ++t;
    if (t == n_ct) {
      k = s.kt;
      v = s.vt;
    } else {
      k += (size_t)kKvTile * s.row_stride;
      v += (size_t)kKvTile * s.row_stride;
    }
  }
  // rows of the current tile (1 .. kKvTile)
  __device__ __forceinline__ int rows() const {
    return t < n_ct ? min(kKvTile, s.p - t * kKvTile) : min(kKvTile, s.n - (t - n_ct) * kKvTile);
  }
};

// Prepare the copy of the walk's current tile into the stage (Kst, Vst);
// `on` false when there is no tile to copy (nothing is read then).
template <int D, int NWAVE = 4>
__device__ __forceinline__ KvCopy<D, NWAVE> kv_copy(const KvWalk<D>& w, bf16* Kst, bf16* Vst,
                                                    bool on) {
  KvCopy<D, NWAVE> c;
  c.bytes = (uint32_t)(w.rows() - 1) * (uint32_t)(w.s.row_stride * 2) + D * 2;
  c.ks = w.k;
  c.vs = w.v;
  c.kd = Kst;
  c.vd = Vst;
  c.on = on;
  return c;
}

}  // namespace cartattn
