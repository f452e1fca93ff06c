// Backward pass of cartridge attention: gradients through the concat into
// the token tensors and into the trainable cartridge rows.
//
// Source: "Cartridges: trained KV-prefix corpus compression", section
// "Semantics (pinned to the reference implementation)": the f32-KV backward
// routes gradients through the concat into the trainable rows, and row 0 is a
// frozen constant. The formulas are the softmax adjoint: with
// D_i = dO_i . O_i and P_ij = exp(scale q_i.k_j - LSE_i),
//   dV_j = sum_i P_ij dO_i,  dS_ij = P_ij (dO_i . v_j - D_i),
//   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i.
//
// Design (gfx950):
//  * preprocess: -D_i, lse_i log2(e) and (float32 mode) zeroing of the f32 dQ
//    accumulator in one pass; with bf16 tokens it also rounds the f32
//    cartridge rows to their bf16 shadow;
//  * float32 reference mode, one generic kernel: a workgroup per 128-key
//    tile (4 waves x 32 keys) keeps its K, V rows as MFMA operands and its
//    f32 dK, dV in registers over a loop of (batch, q-head of the group,
//    32-query tile) units, Q and dO staged in LDS; dS goes through LDS once
//    per unit for dQ = dS K, accumulated in f32 with global atomics;
//    cartridge tiles may be split over units (partial sums reduced by a
//    small kernel) to balance the grid;
//  * bf16 path: a dK/dV kernel (two wave roles per key group, pieces of a
//    tile summed by the tile's last piece) and a query-major dQ kernel that
//    recomputes S and dP, described below; the only atomics are one counter
//    per piece;
//  * block ids are remapped so one kv head's tiles share an XCD and its L2.
#include <math.h>

#include <algorithm>
#include <vector>

#include <type_traits>

#include "common.hpp"
#include "kvtiles.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace cartattn {

namespace {

typedef unsigned v4u32 __attribute__((ext_vector_type(4)));

constexpr int kBNB = 128;      // keys per workgroup tile
constexpr int kBQ = 32;        // queries per unit
constexpr int kThreads = 256;
constexpr int kKvThreads = 512;   // dK/dV kernel: 4 pairs of waves

struct BwdArgs {
  const void* q;
  const void* k_tok;
  const void* v_tok;
  const void* k_cart;
  const void* v_cart;
  const void* out;
  const void* dout;
  const float* lse;
  float* lse2;        // [B][Hq][n]: lse * log2(e), written by the preprocess
  float* delta;       // [B][Hq][n], -D (D = dO . O per row)
  float* dq_acc;      // [B][n][Hq][D]
  void* dq;           // tok dtype
  void* dk_tok;
  void* dv_tok;
  float* dk_cart;
  float* dv_cart;
  float* dk_part;     // [splits][p][Hkv][D]
  float* dv_part;
  float* dk_tpart;    // [kv_stmax][B][n][Hkv][D], token-tile pieces (bf16 path)
  float* dv_tpart;
  float* dq_part;     // [q_splits][B][n][Hq][D], dQ key-split pieces (bf16 path)
  int* kv_cnt;        // [Hkv][n_ct + B n_tt] finished pieces per key tile (bf16 path)
  int n_cnt;
  // f32 cartridge rows rounded to the bf16 shadow by the preprocess (bf16 path)
  const f32x4* cast_k;
  const f32x4* cast_v;
  bf16x4* cast_kb;
  bf16x4* cast_vb;
  size_t cast_n4;
  int kv_target, kv_ptok, kv_stmax, q_splits;
  int kv_cart_pieces;         // dK/dV pieces of the cartridge tiles of one kv head
  int D4;             // head_dim / 4
  int B, n, p, f, Hq, Hkv, g;
  int n_ct, n_tt, nqt, splits_c;
  int hpw, wph, n_hg, n_qb;   // query-major grid of the dQ kernel
  int zero_dq;                // preprocess clears the f32 dQ accumulator
  int accumulate;
  int window;                 // > 0: sliding window (positions above p + i - window)
  int kv_tok_pieces;          // dK/dV pieces of one kv head's token tiles (all sequences)
  Segs seg;                   // token rows of each sequence; n is the longest
  float scale, scale_log2;
  int q_pair;                 // dQ grid resident at once: blocks dealt in pairs
  int kv_ttok;                // dK/dV token tiles: pieces of at most this many units
};

template <typename T> struct BLds;
template <> struct BLds<bf16> {
  static constexpr int rpad = 8;   // row-major tiles: stride D+8 (b128 reads)
  static constexpr int tpad = 4;   // transposed q tiles: stride 36 (b64 reads)
};
template <> struct BLds<float> {
  static constexpr int rpad = 1;
  static constexpr int tpad = 1;
};

// Same access pattern as the forward's V^T fragment: item t of MFMA m holds
// column d_row(m*KPL + t, hl) of an LDS row.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag tr_frag(const T* row, int m, int hl);
template <>
__device__ __forceinline__ bf16x8 tr_frag<bf16>(const bf16* row, int m, int hl) {
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 16 * m + 4 * hl);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 16 * m + 8 + 4 * hl);
  bf16x8 f;
  f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
  f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
  return f;
}
template <>
__device__ __forceinline__ float tr_frag<float>(const float* row, int m, int hl) {
  return row[d_row(m, hl)];
}

// KPL consecutive elements of a TS row converted to an MFMA fragment of T.
template <typename T, typename TS>
__device__ __forceinline__ typename Mfma<T>::frag conv_frag(const TS* p);
template <> __device__ __forceinline__ bf16x8 conv_frag<bf16, bf16>(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <> __device__ __forceinline__ bf16x8 conv_frag<bf16, float>(const float* p) {
  float v[8];
  load8<float>(p, v);
  bf16x8 f;
#pragma unroll
  for (int t = 0; t < 8; ++t) f[t] = (bf16)v[t];
  return f;
}
template <> __device__ __forceinline__ float conv_frag<float, float>(const float* p) {
  return *p;
}

template <typename T> __device__ __forceinline__ typename Mfma<T>::frag zero_frag();
template <> __device__ __forceinline__ bf16x8 zero_frag<bf16>() {
  bf16x8 f;
#pragma unroll
  for (int t = 0; t < 8; ++t) f[t] = (bf16)0.f;
  return f;
}
template <> __device__ __forceinline__ float zero_frag<float>() { return 0.f; }

template <typename T, typename TR, int D>
__global__ __launch_bounds__(kThreads) void attn_bwd_kernel(BwdArgs a) {
  using M = Mfma<T>;
  constexpr int KPL = M::KPL;
  constexpr int KSTEP = M::KSTEP;
  constexpr int NKS = D / KSTEP;
  constexpr int NDB = D / 32;
  constexpr int NPV = 16 / KPL;          // MFMAs per 32-row contraction
  constexpr int RSTR = D + BLds<T>::rpad;        // Qs, dOs
  constexpr int TSTR = kBQ + BLds<T>::tpad;      // Qt, dOt
  constexpr int KTSTR = kBNB + BLds<T>::rpad;    // Kt, dSs
  __shared__ __align__(16) T Kt[D * KTSTR];
  __shared__ __align__(16) T Qs[kBQ * RSTR];
  __shared__ __align__(16) T dOs[kBQ * RSTR];
  __shared__ __align__(16) T Qt[D * TSTR];
  __shared__ __align__(16) T dOt[D * TSTR];
  __shared__ __align__(16) T dSs[kBQ * KTSTR];
  __shared__ __align__(16) float lse2s[kBQ];
  __shared__ __align__(16) float dls[kBQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // ---- decode the work item: per kv head, cartridge items then token items
  const int per_kv = a.n_ct * a.splits_c + a.B * a.n_tt;
  const int lg = xcd_remap(blockIdx.x, gridDim.x);
  const int kv = lg / per_kv;
  int r0 = lg % per_kv;
  const bool cart = r0 < a.n_ct * a.splits_c;
  int tile, split = 0, b = 0, u_begin, u_end;
  const int units_per_head = a.nqt;
  if (cart) {
    tile = r0 / a.splits_c;
    split = r0 % a.splits_c;
    const int U = a.B * a.g * a.nqt;
    u_begin = (int)((long long)split * U / a.splits_c);
    u_end = (int)((long long)(split + 1) * U / a.splits_c);
  } else {
    r0 -= a.n_ct * a.splits_c;
    b = r0 / a.n_tt;
    tile = r0 % a.n_tt;
    if (tile * kBNB >= a.seg.len(b, a.n)) return;     // past a packed segment's end
    u_begin = 0;
    u_end = a.g * ((a.seg.len(b, a.n) + kBQ - 1) / kBQ - tile * (kBNB / kBQ));
  }
  const int base = a.seg.base(b, a.n);                // token tiles: the sequence's rows
  const int j0 = tile * kBNB;                         // first row in its source
  const int limit = cart ? a.p : a.seg.len(b, a.n);   // rows that exist
  const int my_key = j0 + 32 * wave + l32;            // this lane's key row (B operand)
  const size_t row_stride = (size_t)a.Hkv * D;

  // ---- K, V rows of this wave as B operands; K^T of the tile into LDS
  typename M::frag kf[NKS], vf[NKS];
  {
    const bool ok = my_key < limit;
    if (cart) {
      const TR* kp = reinterpret_cast<const TR*>(a.k_cart) + ((size_t)my_key * a.Hkv + kv) * D;
      const TR* vp = reinterpret_cast<const TR*>(a.v_cart) + ((size_t)my_key * a.Hkv + kv) * D;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        kf[ks] = ok ? conv_frag<T, TR>(kp + ks * KSTEP + hl * KPL) : zero_frag<T>();
        vf[ks] = ok ? conv_frag<T, TR>(vp + ks * KSTEP + hl * KPL) : zero_frag<T>();
      }
    } else {
      const size_t off = (((size_t)base + my_key) * a.Hkv + kv) * D;
      const T* kp = reinterpret_cast<const T*>(a.k_tok) + off;
      const T* vp = reinterpret_cast<const T*>(a.v_tok) + off;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        kf[ks] = ok ? conv_frag<T, T>(kp + ks * KSTEP + hl * KPL) : zero_frag<T>();
        vf[ks] = ok ? conv_frag<T, T>(vp + ks * KSTEP + hl * KPL) : zero_frag<T>();
      }
    }
    constexpr int CPR = D / 8;
    constexpr int NCH = kBNB * CPR / kThreads;
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int c = tid + u * kThreads;
      const int r = c / CPR;
      const int col = (c % CPR) * 8;
      const int j = j0 + r;
      float v8[8];
      if (j < limit) {
        if (cart)
          load8<TR>(reinterpret_cast<const TR*>(a.k_cart) + ((size_t)j * a.Hkv + kv) * D + col, v8);
        else
          load8<T>(reinterpret_cast<const T*>(a.k_tok) + (((size_t)base + j) * a.Hkv + kv) * D + col, v8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v8[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) Kt[(col + e) * KTSTR + r] = from_f32<T>(v8[e]);
    }
  }

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dk[db][r] = 0.f; dv[db][r] = 0.f; }

  // dQ work split inside the workgroup: d-block and key range per wave.
  constexpr int NKP = 4 / NDB;                 // key parts (1 for D=128, 2 for D=64)
  const int q_db = wave % NDB;
  const int q_kp = wave / NDB;
  constexpr int KP_STEPS = (kBNB / NKP) / KSTEP;

  for (int u = u_begin; u < u_end; ++u) {
    int bb, hin, qt;
    if (cart) {
      bb = u / (a.g * units_per_head);
      hin = (u / units_per_head) % a.g;
      qt = u % units_per_head;
    } else {
      const int span = (a.seg.len(b, a.n) + kBQ - 1) / kBQ - tile * (kBNB / kBQ);
      bb = b;
      hin = u / span;
      qt = tile * (kBNB / kBQ) + u % span;
    }
    const int h = kv * a.g + hin;
    const int i0 = qt * kBQ;
    const int nbb = a.seg.len(bb, a.n);     // the unit's sequence: length and first row
    const int bbase = a.seg.base(bb, a.n);

    __syncthreads();   // previous unit is done with the staged tiles and dS
    {
      constexpr int CPR = D / 8;
      constexpr int NCH = kBQ * CPR / kThreads;
#pragma unroll
      for (int uu = 0; uu < NCH; ++uu) {
        const int c = tid + uu * kThreads;
        const int r = c / CPR;
        const int col = (c % CPR) * 8;
        const int i = i0 + r;
        float qv[8], ov[8];
        if (i < nbb) {
          const size_t off = (((size_t)bbase + i) * a.Hq + h) * D + col;
          load8<T>(reinterpret_cast<const T*>(a.q) + off, qv);
          load8<T>(reinterpret_cast<const T*>(a.dout) + off, ov);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) { qv[e] = 0.f; ov[e] = 0.f; }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const T qe = from_f32<T>(qv[e]);
          const T oe = from_f32<T>(ov[e]);
          Qs[r * RSTR + col + e] = qe;
          dOs[r * RSTR + col + e] = oe;
          Qt[(col + e) * TSTR + r] = qe;
          dOt[(col + e) * TSTR + r] = oe;
        }
      }
      if (tid < kBQ) {
        const int i = i0 + tid;
        const size_t li = ((size_t)bb * a.Hq + h) * a.n + i;
        lse2s[tid] = (i < nbb) ? a.lse[li] * kLog2e : INFINITY;
        dls[tid] = (i < nbb) ? a.delta[li] : 0.f;
      }
    }
    __syncthreads();

    // S = Q K^T and dP = dO V^T: rows = queries (A from LDS), cols = this
    // wave's keys (B in registers). Lane (key + 32 hl), reg r <-> query d_row(r, hl).
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
    {
      const T* qrow = Qs + l32 * RSTR + hl * KPL;
      const T* orow = dOs + l32 * RSTR + hl * KPL;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        s = M::mma(load_frag<T>(qrow + ks * KSTEP), kf[ks], s);
        dp = M::mma(load_frag<T>(orow + ks * KSTEP), vf[ks], dp);
      }
    }
    const bool key_ok = my_key < limit;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qq = d_row(r, hl);
      const int i = i0 + qq;
      bool vis = key_ok && (cart || my_key <= i);   // i >= n has lse2 = +inf
      if (a.window > 0) vis = vis && ((cart ? my_key : a.p + my_key) > i + a.p - a.window);
      const float pv = vis ? exp2f(s[r] * a.scale_log2 - lse2s[qq]) : 0.f;
      s[r] = pv;                                  // P
      dp[r] = pv * (dp[r] + dls[qq]);             // dS (unscaled)
    }

    // dV += P^T dO, dK += dS^T Q (A from registers, B = transposed tiles).
#pragma unroll
    for (int m = 0; m < NPV; ++m) {
      const typename M::frag pf = pack_regs<T>(s, m);
      const typename M::frag sf = pack_regs<T>(dp, m);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dv[db] = M::mma(pf, tr_frag<T>(dOt + (32 * db + l32) * TSTR, m, hl), dv[db]);
        dk[db] = M::mma(sf, tr_frag<T>(Qt + (32 * db + l32) * TSTR, m, hl), dk[db]);
      }
    }

    // dS to LDS as [query][key of the tile] for dQ = dS K.
#pragma unroll
    for (int r = 0; r < 16; ++r)
      dSs[d_row(r, hl) * KTSTR + 32 * wave + l32] = from_f32<T>(dp[r]);
    __syncthreads();

    {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      const int kbase = q_kp * (kBNB / NKP);
      const T* arow = dSs + l32 * KTSTR + kbase + hl * KPL;
      const T* brow = Kt + (32 * q_db + l32) * KTSTR + kbase + hl * KPL;
#pragma unroll
      for (int ks = 0; ks < KP_STEPS; ++ks)
        acc = M::mma(load_frag<T>(arow + ks * KSTEP), load_frag<T>(brow + ks * KSTEP), acc);
      // lane (d + 32 hl), reg r <-> query d_row(r, hl), column 32*q_db + d
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + d_row(r, hl);
        if (i < nbb)
          atomicAdd(a.dq_acc + (((size_t)bbase + i) * a.Hq + h) * D + 32 * q_db + l32,
                    acc[r] * a.scale);
      }
    }
  }

  // ---- write dK, dV: lane (d + 32 hl), reg r <-> key 32*wave + d_row(r, hl)
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int j = j0 + 32 * wave + d_row(r, hl);
    if (j >= limit) continue;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int col = 32 * db + l32;
      const float gk = dk[db][r] * a.scale;
      const float gv = dv[db][r];
      if (cart) {
        const size_t o = ((size_t)j * a.Hkv + kv) * D + col;
        if (a.splits_c > 1) {
          const size_t po = (size_t)split * a.p * row_stride + o;
          a.dk_part[po] = gk;
          a.dv_part[po] = gv;
        } else if (j < a.f) {
          a.dk_cart[o] = 0.f;
          a.dv_cart[o] = 0.f;
        } else if (a.accumulate) {
          a.dk_cart[o] += gk;
          a.dv_cart[o] += gv;
        } else {
          a.dk_cart[o] = gk;
          a.dv_cart[o] = gv;
        }
      } else {
        const size_t o = (((size_t)base + j) * a.Hkv + kv) * D + col;
        reinterpret_cast<T*>(a.dk_tok)[o] = from_f32<T>(gk);
        reinterpret_cast<T*>(a.dv_tok)[o] = from_f32<T>(gv);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 path: two kernels.
//
// attn_bwd_kv_kernel -- dK and dV. One workgroup (8 waves) per piece of a
//   128-key tile's list of (batch, q-head, 32-query) units. Waves k and k+4
//   (one SIMD) share keys 32k .. 32k+31 and split the work by role: wave k
//   computes S = Q K^T, the softmax P and dV += P^T dO; wave k+4 computes
//   dP = dO V^T, dS = P (dP - D) with P handed over through LDS, and
//   dK += dS^T Q. Each keeps one operand (K or V rows) and one f32
//   accumulator in registers, so two waves fit each SIMD and one's softmax
//   runs beside the other's MFMAs. Each unit's Q, dO, LSE*log2(e) and -D rows
//   are copied global -> LDS by direct loads into a ring of padded tiles
//   three units ahead; one LDS-only barrier per unit.
//
// attn_bwd_dq_kernel -- dQ, query-major like the forward: per key tile it
//   recomputes S^T = K Q^T and dP^T = V dO^T, forms dS^T, and accumulates
//   dQ^T += K^T dS^T in registers (K^T by transpose reads, dS^T straight from
//   the MFMA result layout). dQ is written once, in the token dtype.
// Cartridge rows arrive as bf16 (f32 master rows are cast first).


// Entry i of the segment offsets of the dK/dV kernel's argument. A run-time
// index into an array member of a by-value kernel argument makes the
// compiler copy the whole argument to per-lane scratch memory; reading it in
// place in the kernarg segment (where BwdArgs, the kernel's only argument,
// starts at offset 0) keeps every read a scalar load.
__device__ inline int bwd_seg_off(int i) {
  const auto* kb = (const __attribute__((address_space(4))) char*)(
      __builtin_amdgcn_kernarg_segment_ptr());
  return *(const __attribute__((address_space(4))) int*)(
      kb + offsetof(BwdArgs, seg) + offsetof(Segs, off) + sizeof(int) * i);
}
template <int D>
__global__ __launch_bounds__(kKvThreads, 1) void attn_bwd_kv_kernel(BwdArgs a) {
  using M = Mfma<bf16>;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  using TL = Tile<D>;
  // Q / dO tiles in whole 1 KiB blocks, 2 more than a multiple of 4, so that
  // the copy of a unit (2 QBLK blocks and the four 16-row halves of lse and
  // -D) splits evenly over the 8 waves
  constexpr int QBLK0 = (tile_elems<D, kBQ>() + 511) / 512;
  constexpr int QBLK = QBLK0 + ((2 - QBLK0 % 4) + 4) % 4;
  constexpr int QTILE = QBLK * 512;
  constexpr int NOPS = (2 * QBLK + 4) / 8;   // copies per wave per unit
  static_assert((2 * QBLK + 4) % 8 == 0, "copies per unit must split over 8 waves");
  // Ring of AHEAD + 2 unit stages: Q tile | dO tile | lse*log2(e) [32], -D [32].
  // Step j reads the stages of units j (row fragments, lse) and j-1
  // (transpose fragments, -D) and issues the copy of unit j + AHEAD before
  // its MFMAs (a copy issued between MFMAs holds the wave's next MFMAs up
  // until the memory pipeline takes it); stages are read while copies fill
  // others, so every LDS access of the unit loop is issued by the
  // inline-assembly helpers with explicit waits.
  constexpr int AHEAD = 3;
  constexpr int NST = AHEAD + 2;
  constexpr int STAGE = 2 * QTILE + 2 * 2 * kBQ;   // bf16 elements per stage
  constexpr int O_OFF = 2 * QTILE;                  // byte offset of dO in a stage
  constexpr int L_OFF = 4 * QTILE;                  // byte offset of lse / -D
  constexpr int XSLOT = 4 * 4096;                   // bytes of one P hand-over slot
  __shared__ __align__(16) bf16 ring[NST * STAGE];
  __shared__ __align__(16) float xchg[2 * XSLOT / 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int pair = wave & 3;       // keys 32 pair .. of the tile
  const bool grole = wave >= 4;    // G role (dP, dK) or P role (S, dV)
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // ---- work item: a piece of one key tile's unit list (pieces of cartridge
  // tiles first, then the pieces of the token tiles, tile-major)
  // Sequence b_: its length, first token row, and the query tiles below
  // qt_hi that hold a query seeing a row of key tile t_ (all of its query
  // tiles, or with a sliding window those below the window end of the
  // tile's last row).
  const bool packed = a.seg.packed != 0;
  auto len_of = [&](int b_) {
    b_ = min(b_, a.B - 1);
    return packed ? bwd_seg_off(b_ + 1) - bwd_seg_off(b_) : a.n;
  };
  auto base_of = [&](int b_) { return packed ? bwd_seg_off(min(b_, a.B - 1)) : b_ * a.n; };
  auto qt_hi_of = [&](bool c_, int t_, int b_) -> int {
    const int nq_ = (len_of(b_) + kBQ - 1) / kBQ;
    if (a.window <= 0) return nq_;
    const int last = min(t_ * kBNB + kBNB - 1, (c_ ? a.p : len_of(b_)) - 1);
    const int hi = (c_ ? last - a.p : last) + a.window;   // queries below hi see it
    return max(0, min(nq_, (hi + kBQ - 1) / kBQ));
  };
  // units (sequence, head, query tile) of cartridge tile t_
  auto cart_units = [&](int t_) {
    if (!packed) return a.B * a.g * qt_hi_of(true, t_, 0);
    int u_ = 0;
    for (int b_ = 0; b_ < a.B; ++b_) u_ += a.g * qt_hi_of(true, t_, b_);
    return u_;
  };
  const int per_kv = a.kv_cart_pieces + a.kv_tok_pieces;
  const int lg = xcd_remap(blockIdx.x, gridDim.x);
  const int kv = lg / per_kv;
  int r0 = lg % per_kv;
  const bool cart = r0 < a.kv_cart_pieces;
  int tile, split = 0, n_split = 1, b = 0, u_begin, u_end;
  if (cart && a.window <= 0) {
    // split-major: the workgroups that run together (consecutive ids on one
    // XCD) read the same window of units, so their Q / dO copies share the L2
    split = r0 / a.n_ct;
    tile = r0 % a.n_ct;
    n_split = a.splits_c;
    const int U = cart_units(0);    // every cartridge tile sees every query
    u_begin = (int)((long long)split * U / a.splits_c);
    u_end = (int)((long long)(split + 1) * U / a.splits_c);
  } else if (cart) {
    // sliding window: the cartridge tiles see different query ranges, so
    // their pieces are dealt tile-major (a tile no query sees: one piece
    // with no units, which writes its zero gradient)
    tile = 0;
    int U = cart_units(0);
    n_split = max(1, (U + a.kv_target - 1) / a.kv_target);
    while (r0 >= n_split && tile + 1 < a.n_ct) {
      r0 -= n_split;
      ++tile;
      U = cart_units(tile);
      n_split = max(1, (U + a.kv_target - 1) / a.kv_target);
    }
    if (r0 >= n_split) return;   // beyond the planned pieces (never, by construction)
    split = r0;
    u_begin = (int)((long long)split * U / n_split);
    u_end = (int)((long long)(split + 1) * U / n_split);
  } else {
    // token pieces tile-major (the larger tiles, nearer the start, first),
    // then by sequence (those long enough to have the tile), then by piece
    r0 -= a.kv_cart_pieces;
    int ut = 0;
    for (tile = 0; tile < a.n_tt; ++tile) {
      if (!packed) {
        ut = a.g * (qt_hi_of(false, tile, 0) - tile * (kBNB / kBQ));
        n_split = (ut + a.kv_ttok - 1) / a.kv_ttok;
        if (r0 < a.B * n_split) { b = r0 / n_split; r0 %= n_split; break; }
        r0 -= a.B * n_split;
        continue;
      }
      bool found = false;
      for (b = 0; b < a.B; ++b) {
        if (tile * kBNB >= len_of(b)) continue;
        ut = a.g * (qt_hi_of(false, tile, b) - tile * (kBNB / kBQ));
        n_split = (ut + a.kv_ttok - 1) / a.kv_ttok;
        if (r0 < n_split) { found = true; break; }
        r0 -= n_split;
      }
      if (found) break;
    }
    if (tile >= a.n_tt) return;  // beyond the planned pieces (never, by construction)
    split = r0;
    u_begin = (int)((long long)split * ut / n_split);
    u_end = (int)((long long)(split + 1) * ut / n_split);
  }
  const int j0 = tile * kBNB;
  const int nb = cart ? 0 : len_of(b);      // a token tile's sequence length
  const int limit = cart ? a.p : nb;
  const int my_key = j0 + 32 * pair + l32;
  const bool key_ok = my_key < limit;
  const size_t row_stride = (size_t)a.Hkv * D;
  const bf16* kbase = cart ? reinterpret_cast<const bf16*>(a.k_cart) + kv * D
                           : reinterpret_cast<const bf16*>(a.k_tok) + ((size_t)base_of(b) * a.Hkv + kv) * D;
  const bf16* vbase = cart ? reinterpret_cast<const bf16*>(a.v_cart) + kv * D
                           : reinterpret_cast<const bf16*>(a.v_tok) + ((size_t)base_of(b) * a.Hkv + kv) * D;
  // Queries i visible to this lane's key: lo <= i < hi (an empty range for a
  // key past the end of its rows); hi is the query's sequence length (a
  // cartridge key: per unit), or with a sliding window the key's window end
  // if that comes first.
  const int vis_lo = !key_ok ? (1 << 30) : (cart ? 0 : my_key);
  const int win_hi = a.window > 0 ? (cart ? my_key - a.p : my_key) + a.window : (1 << 30);
  auto vis_span_for = [&](int len_) { return (uint32_t)max(0, min(len_, win_hi) - vis_lo); };

  // ---- unit cursor: (sequence, q-head of the group, query tile), the end
  // of its query tiles, and the offsets of its Q / dO rows (bytes) and of
  // its lse / D (elements); within a head the next unit is one query tile
  // further, so only a change of head recomputes them
  const int qt0 = cart ? 0 : tile * (kBNB / kBQ);
  const uint32_t q_row_bytes = (uint32_t)(a.Hq * D * 2);
  struct Unit { int bb, hin, qt, qt_end, len; size_t qoff, loff; };
  auto locate_unit = [&](Unit& x) {
    const int h = kv * a.g + x.hin;
    x.len = len_of(x.bb);
    x.qoff = (((size_t)base_of(x.bb) + (size_t)x.qt * kBQ) * a.Hq + h) * (size_t)(D * 2);
    x.loff = ((size_t)x.bb * a.Hq + h) * a.n + (size_t)x.qt * kBQ;
  };
  // query tiles of the unit's sequence that this key tile serves
  auto qt_end_of = [&](int bb_) { return bb_ < a.B ? qt_hi_of(cart, tile, bb_) : qt0 + 1; };
  Unit cu;
  if (cart) {
    int u = u_begin, bb = 0, nq_ = qt_end_of(0);
    if (!packed) {
      const int nqu = max(1, nq_);   // the same for every sequence
      bb = u / (a.g * nqu);
      u -= bb * a.g * nqu;
      nq_ = nqu;
    } else {
      while (bb < a.B - 1 && u >= a.g * nq_) { u -= a.g * nq_; nq_ = qt_end_of(++bb); }
      nq_ = max(1, nq_);
    }
    cu.bb = bb;
    cu.hin = u / nq_;
    cu.qt = u % nq_;
    cu.qt_end = nq_;
  } else {
    const int nq_ = max(1, qt_end_of(b) - qt0);
    cu.bb = b;
    cu.hin = u_begin / nq_;
    cu.qt = qt0 + u_begin % nq_;
    cu.qt_end = qt0 + nq_;
  }
  locate_unit(cu);
  auto next = [&](Unit x) {
    if (++x.qt == x.qt_end) {
      x.qt = qt0;
      if (++x.hin == a.g) {
        x.hin = 0;
        ++x.bb;
        // a cartridge tile skips the sequences none of whose queries see it
        if (cart) while (x.bb < a.B && qt_end_of(x.bb) == 0) ++x.bb;
        x.qt_end = max(qt0 + 1, qt_end_of(x.bb));
      }
      locate_unit(x);
    } else {
      x.qoff += (size_t)kBQ * q_row_bytes;
      x.loff += kBQ;
    }
    return x;
  };
  // Units whose pairs are not all visible (some key of the tile missing, the
  // query tile ragged, or a token tile's diagonal) take the mask.
  const bool mask_all = j0 + kBNB > limit;
  const int q_diag = cart ? 0 : qt0 + kBNB / kBQ;        // first tile past the diagonal
  // with a sliding window, the first query past the window of the tile's
  // first row (later queries lose rows of the tile)
  const int q_win = a.window > 0 ? (cart ? j0 - a.p : j0) + a.window : (1 << 30);
  // (len: the unit's sequence length; its first ragged query tile is len / 32)
  auto needs_mask = [&](int qt, int len) {
    return mask_all || qt >= len / kBQ || qt < q_diag || qt * kBQ + kBQ > q_win;
  };

  // ---- this wave's copies of a unit: copy o = wave + 8 i of the list
  // (Q blocks, dO blocks, lse halves, -D halves). Rows past the unit's last
  // (ragged tile, or the rounding of the tile to whole blocks) fall outside
  // the copy's buffer range and read as zeros, which the mask discards.
  uint32_t c_off[NOPS], c_dst[NOPS];
  bool c_dout[NOPS];
#pragma unroll
  for (int i = 0; i < NOPS; ++i) {
    const int o = wave + 8 * i;
    if (o < 2 * QBLK) {
      const bool od = o >= QBLK;
      const int blk = od ? o - QBLK : o;
      int r, cc;
      TL::locate(blk * 64 + lane, r, cc);
      c_off[i] = (uint32_t)r * q_row_bytes + (uint32_t)(cc < D / 8 ? cc : 0) * 16;
      c_dst[i] = (od ? O_OFF : 0) + blk * 1024;
      c_dout[i] = od;
    } else {
      const int hh = o - 2 * QBLK;   // 0, 1: lse halves; 2, 3: -D halves
      c_off[i] = 4 * (lane + 16 * (hh & 1));
      c_dst[i] = L_OFF + 128 * (hh >> 1) + 64 * (hh & 1);
      c_dout[i] = false;
    }
  }
  // only the last copy of waves 4..7 is an lse / -D half
  const bool lcopy = wave >= 4;
  const float* lbase = wave >= 6 ? a.delta : a.lse2;
  const char* obase[NOPS];
#pragma unroll
  for (int i = 0; i < NOPS; ++i)
    obase[i] = reinterpret_cast<const char*>(c_dout[i] ? a.dout : a.q);
  // Every wave issues NOPS copies per unit, and a copy past the piece's last
  // unit (its buffer range empty) still issues its loads, which read
  // nothing: the wait counts of the ring are constants.
  struct Copy { buf_rsrc r[NOPS]; uint32_t st; };
  const uint32_t ring_base = lds_addr(ring);
  auto copy_setup = [&](const Unit& x, uint32_t st_addr, bool real) {
    Copy c;
    const int rows = min(kBQ, x.len - x.qt * kBQ);
    const uint32_t nq = real ? (uint32_t)(rows - 1) * q_row_bytes + D * 2 : 0u;
#pragma unroll
    for (int i = 0; i < NOPS - 1; ++i) c.r[i] = make_rsrc(obase[i] + x.qoff, nq);
    c.r[NOPS - 1] = lcopy ? make_rsrc(lbase + x.loff, real ? 4u * (uint32_t)rows : 0u)
                          : make_rsrc(obase[NOPS - 1] + x.qoff, nq);
    c.st = st_addr - ring_base;   // byte offset of the stage in the ring
    return c;
  };
  auto copy_part = [&](const Copy& c, int i) {
    if (i < NOPS - 1 || !lcopy) {
      dma16_at(c.r[i], c_off[i], ring, c.st + c_dst[i]);
    } else if (lane < 16) {
      dma4_at(c.r[i], c_off[i], ring, c.st + c_dst[i]);
    }
  };
  auto stage_addr = [&](int st) { return ring_base + (uint32_t)(2 * STAGE) * st; };
  auto issue = [&](const Unit& x, int st, bool real) {
    const Copy c = copy_setup(x, stage_addr(st), real);
#pragma unroll
    for (int i = 0; i < NOPS; ++i) copy_part(c, i);
  };

  // ---- the wave's operand rows (K for the P role, V for the G role) as B
  // operands; the copies of units 0 .. AHEAD-1 are issued around these loads
  const int nu = u_end - u_begin;
  if (nu > 0) issue(cu, 0, true);
  bf16x8 kvf[NKS];
  {
    const bf16* ob = grole ? vbase : kbase;
    const int kr = key_ok ? my_key : limit - 1;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kvf[ks] = *reinterpret_cast<const bf16x8*>(ob + (size_t)kr * row_stride + 16 * ks + 8 * hl);
  }
  if (nu > 0) {
    Unit x = cu;
    for (int u = 1; u < AHEAD; ++u) {
      x = next(x);
      issue(x, u, u < nu);
    }
  }

  // dV (P role) or dK (G role) of the wave's 32 keys
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  const float c = a.scale_log2;

  // Per-lane LDS byte offsets inside a stage: the row fragment (row l32,
  // 8 elements at 8 hl), the transpose strip (tr_col4's lane pattern for
  // rows 4 hl .., columns 16 ((lane >> 4) & 1) ..) and lse / -D (queries
  // 8 c4 + 4 hl .. of a lane's result registers 4 c4 ..); the lane's 16-byte
  // words of the P hand-over (4 words of 4 result registers, 1 KiB apart).
  const uint32_t row_lane = TL::off(l32, 8 * hl);
  const uint32_t tr_lane = TL::off(4 * hl + ((lane & 15) >> 2), 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  const uint32_t ld_lane = L_OFF + 16 * hl;
  const uint32_t x_lane = lds_addr(xchg) + 4096 * pair + 16 * lane;
  auto mask_rel = [&](int qt) { return (uint32_t)(qt * kBQ + 4 * hl - vis_lo); };
  // Transpose fragment f = m * NDB + db (queries 16 m .., columns 32 db ..)
  // of the dO (P role) or Q (G role) tile of a stage: 2 reads.
  auto tr_frag = [&](auto G, uint32_t stage, auto F) {
    constexpr int f = decltype(F)::value;
    constexpr int off = (decltype(G)::value ? 0 : O_OFF) + TL::rows(16 * (f / NDB)) + 2 * 32 * (f % NDB);
    const uint32_t base = stage + tr_lane;
    return cat8(lds_tr4<off>(base), lds_tr4<off + TL::rows(8)>(base));
  };
  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;

  // Step j of one wave. Phase A (unit j < nu): the 32 x 32 block X = R W^T
  // with R the unit's Q (P role) or dO (G role) row fragments and W the
  // wave's K or V rows, into xa (rows = queries, columns = keys; lane
  // (key + 32 hl), reg r <-> query d_row(r, hl)). Phase B (unit j-1): acc +=
  // Y^T T with Y the packed operand of unit j-1 (P or G) and T the transpose
  // fragments of its dO or Q tile. The two interleave per k-step, each
  // k-step's LDS reads issued one k-step ahead; with phase A, the copies of
  // unit j + AHEAD go out first.
  auto mfma_steps = [&](auto G, auto HA, auto HB, uint32_t stA, uint32_t stB, f32x16& xa,
                        const bf16x8 (&yb)[2], const Copy& cp) {
    constexpr bool A = decltype(HA)::value, B = decltype(HB)::value;
    constexpr int ROFF = decltype(G)::value ? O_OFF : 0;   // row fragments of dO or Q
    bf16x8 ra[2], tb[2];
    constexpr int NR = (A ? 1 : 0) + (B ? 2 : 0);
    auto batch = [&](auto KS, int slot) {
      constexpr int ks = decltype(KS)::value;
      if constexpr (A) ra[slot] = __builtin_bit_cast(bf16x8, lds_read16<ROFF + 32 * ks>(stA + row_lane));
      if constexpr (B) tb[slot] = tr_frag(G, stB, KS);
    };
    if constexpr (A) {
#pragma unroll
      for (int r = 0; r < 16; ++r) xa[r] = 0.f;
    }
    if constexpr (A) {
#pragma unroll
      for (int i = 0; i < NOPS; ++i) copy_part(cp, i);
    }
    batch(std::integral_constant<int, 0>{}, 0);
    static_for<NKS>([&](auto KS) {
      constexpr int ks = decltype(KS)::value;
      if constexpr (ks + 1 < NKS) {
        batch(std::integral_constant<int, ks + 1>{}, (ks + 1) & 1);
        lds_wait<NR>();
      } else {
        lds_wait<0>();
      }
      if constexpr (A) lds_tie(ra[ks & 1]);
      if constexpr (B) lds_tie(tb[ks & 1]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (A) xa = M::mma(ra[ks & 1], kvf[ks], xa);
      if constexpr (B) {
        constexpr int m = ks / NDB, db = ks % NDB;
        acc[db] = M::mma(yb[m], tb[ks & 1], acc[db]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // P role, step j: phase A = S of unit j, phase B = dV += P^T dO of unit
  // j-1; then the softmax of unit j: P = exp2(S c - lse2), cleared where the
  // key cannot see the query, handed to the G wave of the pair (slot j % 2)
  // and packed for the next step.
  auto p_step = [&](auto HA, auto HB, uint32_t stA, uint32_t stB, f32x16& s, bf16x8 (&pp)[2],
                    const Copy& cp, int qt, int len, uint32_t xw) {
    constexpr bool A = decltype(HA)::value;
    mfma_steps(No{}, HA, HB, stA, stB, s, pp, cp);
    if constexpr (A) {
      f32x4 lq[4];
      lq[0] = lds_read16<0>(stA + ld_lane);
      lq[1] = lds_read16<32>(stA + ld_lane);
      lq[2] = lds_read16<64>(stA + ld_lane);
      lq[3] = lds_read16<96>(stA + ld_lane);
      lds_wait<0>();
#pragma unroll
      for (int q = 0; q < 4; ++q) lds_tie(lq[q]);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lq[r >> 2][r & 3]));
      if (needs_mask(qt, len)) {
        const uint32_t rel = mask_rel(qt);
        const uint32_t vis_span = vis_span_for(len);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[r] = rel + (uint32_t)(8 * (r >> 2) + (r & 3)) < vis_span ? s[r] : 0.f;
      }
      lds_write16<0>(xw, f32x4{s[0], s[1], s[2], s[3]});
      lds_write16<1024>(xw, f32x4{s[4], s[5], s[6], s[7]});
      lds_write16<2048>(xw, f32x4{s[8], s[9], s[10], s[11]});
      lds_write16<3072>(xw, f32x4{s[12], s[13], s[14], s[15]});
      pp[0] = pack_regs<bf16>(s, 0);
      pp[1] = pack_regs<bf16>(s, 1);
      lds_wait<0>();
    }
  };
  // G role, step j: first G = P (dP - D) of unit j-1 from its P (slot
  // (j-1) % 2) and dP (computed by the previous step), packed; then phase A
  // = dP of unit j, phase B = dK += G^T Q of unit j-1.
  auto g_step = [&](auto HA, auto HB, uint32_t stA, uint32_t stB, f32x16& dp, bf16x8 (&gg)[2],
                    const Copy& cp, uint32_t xr) {
    constexpr bool B = decltype(HB)::value;
    if constexpr (B) {
      f32x4 pv[4], dn[4];
      pv[0] = lds_read16<0>(xr);
      pv[1] = lds_read16<1024>(xr);
      pv[2] = lds_read16<2048>(xr);
      pv[3] = lds_read16<3072>(xr);
      dn[0] = lds_read16<4 * kBQ>(stB + ld_lane);
      dn[1] = lds_read16<4 * kBQ + 32>(stB + ld_lane);
      dn[2] = lds_read16<4 * kBQ + 64>(stB + ld_lane);
      dn[3] = lds_read16<4 * kBQ + 96>(stB + ld_lane);
      lds_wait<0>();
#pragma unroll
      for (int q = 0; q < 4; ++q) { lds_tie(pv[q]); lds_tie(dn[q]); }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p_ = pv[r >> 2][r & 3];
        dp[r] = fmaf(p_, dp[r], p_ * dn[r >> 2][r & 3]);   // P dP + P (-D)
      }
      gg[0] = pack_regs<bf16>(dp, 0);
      gg[1] = pack_regs<bf16>(dp, 1);
    }
    // MFMAs at raised priority: the P wave's softmax VALU work runs beside
    // them without holding them back
    __builtin_amdgcn_s_setprio(2);
    mfma_steps(Yes{}, HA, HB, stA, stB, dp, gg, cp);
    __builtin_amdgcn_s_setprio(0);
  };

  // The unit loop of one role (compile-time, so that each role's loop has
  // its own register assignment).
  auto drive = [&](auto G) {
    constexpr bool GR = decltype(G)::value;
    f32x16 xa;          // S (P role) or dP (G role) of the newest unit
    bf16x8 yb[2];       // packed P (P role) or G (G role) of the unit before
    const Copy none{};
    // the unit copied at step j (j + AHEAD), and the query tiles and
    // sequence lengths of units j .. j + AHEAD - 1 (they set the mask of
    // unit j), shifted along as the copies advance
    static_assert(AHEAD == 3, "the mask shift register holds AHEAD units");
    Unit uc = cu;
    int mq[AHEAD], ml[AHEAD];
#pragma unroll
    for (int u = 0; u < AHEAD; ++u) {
      mq[u] = uc.qt;
      ml[u] = uc.len;
      uc = next(uc);
    }
    auto shift = [&]() {
#pragma unroll
      for (int u = 0; u + 1 < AHEAD; ++u) {
        mq[u] = mq[u + 1];
        ml[u] = ml[u + 1];
      }
      mq[AHEAD - 1] = uc.qt;
      ml[AHEAD - 1] = uc.len;
      uc = next(uc);
    };
    // LDS addresses of the stages of units j, j-1 and j+AHEAD (unit u lives
    // in stage u % NST; AHEAD + 2 == NST, so unit j+1+AHEAD takes the stage
    // of unit j-1)
    static_assert(AHEAD + 2 == NST, "stage rotation");
    const uint32_t st_last = stage_addr(NST - 1);
    uint32_t s0 = stage_addr(0), s1 = st_last, sc = stage_addr(AHEAD);
    uint32_t xs = 0;   // byte offset of slot j % 2
    auto rotate = [&]() {
      sc = s1;
      s1 = s0;
      s0 = s0 == st_last ? ring_base : s0 + (uint32_t)(2 * STAGE);
      xs ^= (uint32_t)XSLOT;
    };
    auto run = [&](auto HA, auto HB, const Copy& cp) {
      if constexpr (GR)
        g_step(HA, HB, s0, s1, xa, yb, cp, x_lane + (xs ^ (uint32_t)XSLOT));
      else
        p_step(HA, HB, s0, s1, xa, yb, cp, mq[0], ml[0], x_lane + xs);
    };
    // j = 0: phase A of unit 0
    CART_WAIT_VMCNT((AHEAD - 1) * NOPS);
    lds_barrier_waited();
    run(Yes{}, No{}, copy_setup(uc, sc, AHEAD < nu));
    shift();
    rotate();
    // j = 1 .. nu-1: unit j (phase A) and unit j-1 (phase B)
    for (int j = 1; j < nu; ++j) {
      CART_WAIT_VMCNT((AHEAD - 1) * NOPS);
      lds_barrier_waited();
      run(Yes{}, Yes{}, copy_setup(uc, sc, j + AHEAD < nu));
      shift();
      rotate();
    }
    // j = nu: phase B of unit nu-1 (its stage landed before step nu-1)
    lds_barrier_waited();
    run(No{}, Yes{}, none);
  };
  if (nu > 0) {
    if (grole) drive(Yes{});
    else drive(No{});
    // the copies past the piece's last unit read nothing but still write
    // their LDS stages: let them finish before the workgroup can end
    CART_WAIT_VMCNT(0);
  }
  static_assert(2 * NOPS < 64, "copies of two units must fit the wait count");

  // ---- dV (P role) or dK times the softmax scale (G role). A tile cut into
  // pieces: every piece stores its f32 partial sums, and the piece that
  // finishes last adds them up in piece order (the same sum whichever piece
  // that is) and writes the tile's result.
  const float oscale = grole ? a.scale : 1.f;
  const size_t tok_base = cart ? 0 : (size_t)base_of(b);
  auto out_off = [&](int j, int col) {
    return cart ? ((size_t)j * a.Hkv + kv) * D + col
                : ((tok_base + j) * a.Hkv + kv) * D + col;
  };
  float* const out_cart = grole ? a.dk_cart : a.dv_cart;
  bf16* const out_tok = reinterpret_cast<bf16*>(grole ? a.dk_tok : a.dv_tok);
  auto write = [&](int j, int col, float g) {
    const size_t o = out_off(j, col);
    if (cart) {
      if (j < a.f) out_cart[o] = 0.f;
      else if (a.accumulate) out_cart[o] += g;
      else out_cart[o] = g;
    } else {
      out_tok[o] = (bf16)g;
    }
  };
  if (n_split == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = j0 + 32 * pair + d_row(r, hl);
      if (j >= limit) continue;
#pragma unroll
      for (int db = 0; db < NDB; ++db) write(j, 32 * db + l32, acc[db][r] * oscale);
    }
    return;
  }
  // Partial sums are exchanged at device scope without cache maintenance:
  // each wave stores its accumulator registers lane-major (16-byte words,
  // 1 KiB per instruction) write-through past the XCD's L2 (device-scope
  // buffer stores), and the last piece reads them back around its L2
  // (device-scope buffer loads). A plain device-scope fence here would write
  // back and invalidate the whole L2 of the XCD for every piece.
  constexpr int NQ = 4 * NDB;                        // 16-byte words per lane
  const size_t region = (size_t)NQ * 1024;          // bytes per wave and piece
  const int tile_id = cart ? kv * a.n_ct + tile : (kv * a.B + b) * a.n_tt + tile;
  const int n_tiles = cart ? a.Hkv * a.n_ct : a.Hkv * a.B * a.n_tt;
  float* const part = grole ? (cart ? a.dk_part : a.dk_tpart) : (cart ? a.dv_part : a.dv_tpart);
  auto piece_rsrc = [&](int i) {
    const char* base = reinterpret_cast<const char*>(part) +
                       (((size_t)i * n_tiles + tile_id) * 4 + pair) * region;
    return make_rsrc(base, (uint32_t)region);
  };
  {
    const buf_rsrc rp = piece_rsrc(split);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const f32x4 v = {acc[db][4 * cc] * oscale, acc[db][4 * cc + 1] * oscale,
                         acc[db][4 * cc + 2] * oscale, acc[db][4 * cc + 3] * oscale};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, v), rp,
                                               (uint32_t)((db * 4 + cc) * 1024 + lane * 16), 0,
                                               kCpolDevice);
      }
  }
  // every store of the workgroup complete, then count this piece in
  __shared__ int last_piece;
  CART_WAIT_VMCNT(0);
  __syncthreads();
  if (tid == 0) {
    const int cid = cart ? kv * a.n_ct + tile : a.Hkv * a.n_ct + (kv * a.B + b) * a.n_tt + tile;
    last_piece = __hip_atomic_fetch_add(a.kv_cnt + cid, 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == n_split - 1;
  }
  __syncthreads();
  if (!last_piece) return;
  // The last piece adds the pieces in piece order (the same sum whichever
  // piece is last), its own from registers, the others' words HQ at a time
  // (two passes: the sums, the loads and the accumulator fit the registers).
  constexpr int HQ = NQ / 2;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x4 sg[HQ];
#pragma unroll
    for (int q = 0; q < HQ; ++q) sg[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < n_split; ++i) {
      if (i == split) {
#pragma unroll
        for (int q = 0; q < HQ; ++q) {
          const int w = h * HQ + q, db = w / 4, cc = w % 4;
#pragma unroll
          for (int e = 0; e < 4; ++e) sg[q][e] += acc[db][4 * cc + e] * oscale;
        }
        continue;
      }
      const buf_rsrc rp = piece_rsrc(i);
      v4u32 t[HQ];
#pragma unroll
      for (int q = 0; q < HQ; ++q)
        t[q] = __builtin_amdgcn_raw_buffer_load_b128(rp, (uint32_t)((h * HQ + q) * 1024 + lane * 16), 0,
                                                     kCpolDevice);
      // all of the pass's loads in flight before the first add
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < HQ; ++q) sg[q] += __builtin_bit_cast(f32x4, t[q]);
    }
    // words h HQ .. : db = w / 4, registers 4 (w % 4) .. of the accumulator
#pragma unroll
    for (int q = 0; q < HQ; ++q) {
      const int w = h * HQ + q, db = w / 4, cc = w % 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * cc + e;
        const int j = j0 + 32 * pair + d_row(r, hl);
        if (j < limit) write(j, 32 * db + l32, sg[q][e]);
      }
    }
  }
}

// Waves of a dQ workgroup; they share each K/V tile they copy.
constexpr int kDqWaves = 4;

// Where a tile's compute in the dQ kernel issues the copy of the next tile
// (all before the S, dP MFMAs measured fastest of the placements tried).
template <int D> constexpr int kDqCopyA = KvCopy<D, kDqWaves>::N;
template <int D> constexpr int kDqCopyB = KvCopy<D, kDqWaves>::N;

template <int D>
__global__ __launch_bounds__(64 * kDqWaves, 8 / kDqWaves) void attn_bwd_dq_kernel(BwdArgs a) {
  using M = Mfma<bf16>;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  using TL = Tile<D>;
  __shared__ __align__(16) bf16 K0[tile_elems<D, kKvTile>()];
  __shared__ __align__(16) bf16 V0[tile_elems<D, kKvTile>()];
  __shared__ __align__(16) bf16 K1[tile_elems<D, kKvTile>()];
  __shared__ __align__(16) bf16 V1[tile_elems<D, kKvTile>()];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  int lg = xcd_remap(blockIdx.x, gridDim.x);
  const int split = lg % a.q_splits; lg /= a.q_splits;
  // Longest query blocks first. When the whole grid is resident at once
  // (q_pair), the second half of the blocks is dealt shortest first, so a
  // CU's two workgroups tend to pair a long block with a short one.
  const int qr = lg % a.n_qb; lg /= a.n_qb;
  const int qhalf = (a.n_qb + 1) / 2;
  const int qb = (a.q_pair && qr >= qhalf) ? qr - qhalf : a.n_qb - 1 - qr;
  const int hg = lg % a.n_hg; lg /= a.n_hg;
  const int b = lg % a.B; lg /= a.B;
  const int kv = lg;
  const int hw = wave % a.hpw;
  const int pb = wave / a.hpw;
  const int h = kv * a.g + hg * a.hpw + hw;
  const int i0 = (qb * a.wph + pb) * 32;
  const int base = a.seg.base(b, a.n);   // the sequence's first token row
  const int nb = a.seg.len(b, a.n);      // and its length
  if (qb * a.wph * 32 >= nb) return;     // no query of this workgroup exists
  const bool wave_active = i0 < nb;
  const int my_i = i0 + l32;
  const int wg_last = min(nb, (qb + 1) * a.wph * 32) - 1;
  const int n_ct = (a.p + kKvTile - 1) / kKvTile;
  const int nt_all = n_ct + wg_last / kKvTile + 1;
  // this workgroup's contiguous range of key tiles (with a sliding window,
  // from the first tile its earliest query can see)
  const int t_lo = first_window_tile(a.window, qb * a.wph * 32, a.p, n_ct);
  const int t_begin = t_lo + (int)((long long)split * (nt_all - t_lo) / a.q_splits);
  const int t_end = t_lo + (int)((long long)(split + 1) * (nt_all - t_lo) / a.q_splits);
  // first position the wave's first query sees (no window: far below 0)
  const int win_lo = a.window > 0 ? a.p + i0 - a.window + 1 : -(1 << 30);

  const KvSrc<D> src = kv_src<D>(a.k_cart, a.v_cart, a.k_tok, a.v_tok, base, nb, a.p, a.Hkv, kv);
  const KvMap<D, kDqWaves> kmap = kv_map<D, kDqWaves>(a.Hkv, wave, lane);
  KvWalk<D> walk(src, n_ct, t_begin);
  if (t_begin < t_end) kv_copy<D, kDqWaves>(walk, K0, V0, true).all(kmap, wave, lane);

  // Q^T and dO^T as B operands: lane (q + 32 hl) holds row q, 8 columns per k-step.
  bf16x8 qf[NKS], of[NKS];
  const int qi = min(my_i, nb - 1);
  {
    const size_t off = (((size_t)base + qi) * a.Hq + h) * D + 8 * hl;
    const bf16* qp = reinterpret_cast<const bf16*>(a.q) + off;
    const bf16* op = reinterpret_cast<const bf16*>(a.dout) + off;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
      of[ks] = *reinterpret_cast<const bf16x8*>(op + 16 * ks);
    }
  }
  const size_t li = ((size_t)b * a.Hq + h) * a.n + qi;
  const float lse2 = a.lse2[li];
  const float dl = a.delta[li];
  const float c = a.scale_log2;
  const float scale = a.scale;

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  // One 64-key tile at LDS byte addresses kst, vst. All LDS reads are issued
  // by the inline-assembly helpers with explicit waits (the copy of the next
  // tile into the other stage is in flight meanwhile), one step ahead of the
  // MFMAs that use them.
  const uint32_t row_lane = TL::off(l32, 8 * hl);
  const uint32_t tr_lane = TL::off(4 * hl + ((lane & 15) >> 2), 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  // The copy of the next tile (cp): copies [0, kDqCopyA) are issued before
  // the S, dP MFMAs, [kDqCopyA, kDqCopyB) after them, the rest before the dQ
  // MFMAs.
  auto compute = [&](uint32_t kst, uint32_t vst, const KvTile& f, const KvCopy<D, kDqWaves>& cp) {
    // S^T = K Q^T and dP^T = V dO^T for the two 32-key halves: K and V row
    // fragments (row 32 kh + l32, 8 elements at 16 ks + 8 hl), four reads
    // per k-step.
    f32x16 s[2], dp[2];
    {
      bf16x8 kr[2][2], vr[2][2];
      auto rd = [&](auto KS, int slot) {
        constexpr int ks = decltype(KS)::value;
        kr[slot][0] = __builtin_bit_cast(bf16x8, lds_read16<32 * ks>(kst + row_lane));
        kr[slot][1] = __builtin_bit_cast(bf16x8, lds_read16<TL::rows(32) + 32 * ks>(kst + row_lane));
        vr[slot][0] = __builtin_bit_cast(bf16x8, lds_read16<32 * ks>(vst + row_lane));
        vr[slot][1] = __builtin_bit_cast(bf16x8, lds_read16<TL::rows(32) + 32 * ks>(vst + row_lane));
      };
      cp.template range<0, kDqCopyA<D>>(kmap, wave, lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) { s[0][r] = 0.f; s[1][r] = 0.f; dp[0][r] = 0.f; dp[1][r] = 0.f; }
      rd(std::integral_constant<int, 0>{}, 0);
      // MFMA phases run at a raised wave priority, so that the other wave of
      // the SIMD fills the VALU slots with its softmax meanwhile
      __builtin_amdgcn_s_setprio(1);
      static_for<NKS>([&](auto KS) {
        constexpr int ks = decltype(KS)::value;
        if constexpr (ks + 1 < NKS) {
          rd(std::integral_constant<int, ks + 1>{}, (ks + 1) & 1);
          lds_wait<4>();
        } else {
          lds_wait<0>();
        }
        lds_tie(kr[ks & 1][0]);
        lds_tie(kr[ks & 1][1]);
        lds_tie(vr[ks & 1][0]);
        lds_tie(vr[ks & 1][1]);
        __builtin_amdgcn_sched_barrier(0);
        s[0] = M::mma(kr[ks & 1][0], qf[ks], s[0]);
        s[1] = M::mma(kr[ks & 1][1], qf[ks], s[1]);
        dp[0] = M::mma(vr[ks & 1][0], of[ks], dp[0]);
        dp[1] = M::mma(vr[ks & 1][1], of[ks], dp[1]);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    __builtin_amdgcn_s_setprio(0);
    cp.template range<kDqCopyA<D>, kDqCopyB<D>>(kmap, wave, lane);
    // dS^T / scale = P (dP - D) (the scale is applied to dQ at the end);
    // key k = 32 kh + d_row(r, hl) is visible iff lo <= k < lim (its row
    // exists and, for a token tile, it is not after the query; with a
    // sliding window, it is not before the query's window).
    // (one branch for the whole tile: tiles that need no mask skip it)
    if (f.rows < kKvTile || (!f.cart && f.j0 + kKvTile - 1 > i0) || f.abs0 < win_lo + 31) {
      const int lim = f.cart ? f.rows : min(f.rows, my_i - f.j0 + 1);
      const int lim_l = lim - 4 * hl;
      const int lo_l = win_lo + (my_i - i0) - f.abs0 - 4 * hl;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kc = 32 * kh + (r & 3) + 8 * (r >> 2);   // key minus 4 hl
          s[kh][r] = (kc < lim_l && kc >= lo_l) ? s[kh][r] : -INFINITY;
        }
    }
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p_ = __builtin_amdgcn_exp2f(fmaf(s[kh][r], c, -lse2));
        dp[kh][r] = p_ * (dp[kh][r] + dl);
      }
    cp.template range<kDqCopyB<D>, KvCopy<D, kDqWaves>::N>(kmap, wave, lane);
    // dQ^T += K^T dS^T in four steps j = (kh, m): K^T fragments by transpose
    // reads of rows 32 kh + 16 m .. (8 reads per step, one step ahead).
    {
      const uint32_t kb = kst + tr_lane;
      bf16x8 ka[2][NDB];
      auto rdk = [&](auto J, int slot) {
        constexpr int j = decltype(J)::value;
        static_for<NDB>([&](auto DB) {
          constexpr int db = decltype(DB)::value;
          constexpr int off = TL::rows(16 * j) + 2 * 32 * db;
          ka[slot][db] = cat8(lds_tr4<off>(kb), lds_tr4<off + TL::rows(8)>(kb));
        });
      };
      rdk(std::integral_constant<int, 0>{}, 0);
      __builtin_amdgcn_s_setprio(1);
      static_for<4>([&](auto J) {
        constexpr int j = decltype(J)::value;
        constexpr int kh = j / 2, m = j % 2;
        if constexpr (j + 1 < 4) {
          rdk(std::integral_constant<int, j + 1>{}, (j + 1) & 1);
          lds_wait<2 * NDB>();
        } else {
          lds_wait<0>();
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) lds_tie(ka[j & 1][db]);
        const bf16x8 sfr = pack_regs<bf16>(dp[kh], m);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = M::mma(ka[j & 1][db], sfr, acc[db]);
        __builtin_amdgcn_sched_barrier(0);
      });
      __builtin_amdgcn_s_setprio(0);
    }
  };

  // After each barrier no wave reads the other stage any more; the copy of
  // the next tile into it is issued by this tile's compute (all at once by a
  // wave that skips the tile).
  for (int t = t_begin; t < t_end; t += 2) {
    CART_WAIT_VMCNT(0);
    lds_barrier();
    {
      if (t + 1 < t_end) walk.next();
      const KvCopy<D, kDqWaves> cp = kv_copy<D, kDqWaves>(walk, K1, V1, t + 1 < t_end);
      const KvTile f = kv_tile(t, n_ct, a.p, nb);
      if (wave_active && (f.cart || f.j0 <= i0 + 31) && f.abs0 + kKvTile > win_lo)
        compute(lds_addr(K0), lds_addr(V0), f, cp);
      else
        cp.all(kmap, wave, lane);
    }
    if (t + 1 >= t_end) break;
    CART_WAIT_VMCNT(0);
    lds_barrier();
    {
      if (t + 2 < t_end) walk.next();
      const KvCopy<D, kDqWaves> cp = kv_copy<D, kDqWaves>(walk, K0, V0, t + 2 < t_end);
      const KvTile f = kv_tile(t + 1, n_ct, a.p, nb);
      if (wave_active && (f.cart || f.j0 <= i0 + 31) && f.abs0 + kKvTile > win_lo)
        compute(lds_addr(K1), lds_addr(V1), f, cp);
      else
        cp.all(kmap, wave, lane);
    }
  }

  if (!wave_active || my_i >= nb) return;
  if (a.q_splits > 1) {
    // f32 piece of this key range (a split with no tiles writes zeros), in
    // the padded [split][b][i][h] layout
    const size_t prow = ((size_t)b * a.n + my_i) * a.Hq + h;
    float* pp = a.dq_part + ((size_t)split * a.B * a.n * a.Hq + prow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        *reinterpret_cast<float4*>(pp + 32 * db + 8 * cc + 4 * hl) =
            make_float4(acc[db][4 * cc] * scale, acc[db][4 * cc + 1] * scale,
                        acc[db][4 * cc + 2] * scale, acc[db][4 * cc + 3] * scale);
    return;
  }
  const size_t row = ((size_t)base + my_i) * a.Hq + h;
  bf16* dqp = reinterpret_cast<bf16*>(a.dq) + row * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      bf16x4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (bf16)(acc[db][4 * cc + e] * scale);
      *reinterpret_cast<bf16x4*>(dqp + 32 * db + 8 * cc + 4 * hl) = o4;
    }
}

// dQ = sum of the key-split pieces, in bf16 (4 elements per thread).
__global__ __launch_bounds__(256) void bwd_dq_combine(BwdArgs a) {
  const size_t n4 = (size_t)a.B * a.n * a.Hq * (a.D4);
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n4) return;
  // e walks the padded [b][i][h][D/4] pieces; dQ is written at the row of
  // (b, i), and nothing past a packed segment's end
  const size_t r = e / a.D4;
  const int bi = (int)(r / a.Hq);
  const int i = bi % a.n;
  const int b = bi / a.n;
  if (i >= a.seg.len(b, a.n)) return;
  const size_t out = (((size_t)a.seg.base(b, a.n) + i) * a.Hq + r % a.Hq) * a.D4 + e % a.D4;
  const float4* pp = reinterpret_cast<const float4*>(a.dq_part);
  float4 t = pp[e];
#pragma unroll 4
  for (int s = 1; s < a.q_splits; ++s) {
    const float4 u = pp[(size_t)s * n4 + e];
    t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
  }
  bf16x4 o;
  o[0] = (bf16)t.x; o[1] = (bf16)t.y; o[2] = (bf16)t.z; o[3] = (bf16)t.w;
  reinterpret_cast<bf16x4*>(a.dq)[out] = o;
}

// -D_i = -(dO_i . O_i) (stored negated: G = P dP + P (-D) is one multiply
// and one FMA) and lse_i * log2(e) for every (b, h, i), (f32 tokens) dQ
// accumulator := 0, and (bf16) the key tiles' piece counters := 0 and the
// bf16 shadow of f32 cartridge rows (grid-stride, 4 elements a thread). Sixteen
// lanes per row (D/16 elements each), 16 rows per workgroup; the row sum is
// taken with DPP adds.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_preprocess(BwdArgs a) {
  constexpr int EPL = D / 16;
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);   // token row * Hq + h
  const int sub = threadIdx.x & 15;
  const int total = a.seg.rows(a.B, a.n) * a.Hq;
  const bool ok = row < total;
  const int rr = ok ? row : total - 1;
  const T* o = reinterpret_cast<const T*>(a.out) + (size_t)rr * D + sub * EPL;
  const T* g = reinterpret_cast<const T*>(a.dout) + (size_t)rr * D + sub * EPL;
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc += to_f32(o[e]) * to_f32(g[e]);
  acc = row_sum<16>(acc);
  for (int c = blockIdx.x * 256 + threadIdx.x; c < a.n_cnt; c += gridDim.x * 256) a.kv_cnt[c] = 0;
  for (size_t c = (size_t)blockIdx.x * 256 + threadIdx.x; c < a.cast_n4; c += (size_t)gridDim.x * 256) {
    const f32x4 x = a.cast_k[c], y = a.cast_v[c];
    bf16x4 xb, yb;
#pragma unroll
    for (int e = 0; e < 4; ++e) { xb[e] = (bf16)x[e]; yb[e] = (bf16)y[e]; }
    a.cast_kb[c] = xb;
    a.cast_vb[c] = yb;
  }
  if (!ok) return;
  if (sub == 0) {
    const int h = row % a.Hq;
    const int t = row / a.Hq;
    int b = t / a.n, i = t % a.n;
    if (a.seg.packed) {
      // the packed segment holding row t
      int lo = 0, hi = a.seg.packed;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.seg.off[mid] <= t) lo = mid; else hi = mid;
      }
      b = lo;
      i = t - a.seg.off[lo];
    }
    const size_t li = ((size_t)b * a.Hq + h) * a.n + i;
    a.delta[li] = -acc;
    a.lse2[li] = a.lse[li] * kLog2e;
  }
  if (a.zero_dq) {
    float* dq = a.dq_acc + (size_t)row * D + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dq[e] = 0.f;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void bwd_dq_finalize(const float* __restrict__ acc,
                                                       T* __restrict__ dq, size_t n4) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const float4 v = reinterpret_cast<const float4*>(acc)[i];
  T* d = dq + 4 * i;
  d[0] = from_f32<T>(v.x);
  d[1] = from_f32<T>(v.y);
  d[2] = from_f32<T>(v.z);
  d[3] = from_f32<T>(v.w);
}

// Sum the split partials of the cartridge gradients; frozen rows -> 0.
template <int D>
__global__ __launch_bounds__(256) void bwd_cart_reduce_t(BwdArgs a) {
  const size_t total = (size_t)a.p * a.Hkv * D;
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const int j = (int)(e / ((size_t)a.Hkv * D));
  if (j < a.f) {
    a.dk_cart[e] = 0.f;
    a.dv_cart[e] = 0.f;
    return;
  }
  float sk = 0.f, sv = 0.f;
  for (int s = 0; s < a.splits_c; ++s) {
    sk += a.dk_part[(size_t)s * total + e];
    sv += a.dv_part[(size_t)s * total + e];
  }
  if (a.accumulate) {
    a.dk_cart[e] += sk;
    a.dv_cart[e] += sv;
  } else {
    a.dk_cart[e] = sk;
    a.dv_cart[e] = sv;
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

static BwdPlan make_plan_bwd(const AttnDims& d);

// Plans are cached per thread by shape: the work split is chosen by a small
// simulation that costs up to a few milliseconds on large shapes.
BwdPlan plan_bwd(const AttnDims& d) {
  struct Entry { AttnDims d; BwdPlan pl; bool used; };
  thread_local Entry cache[8] = {};
  thread_local int next_slot = 0;
  auto same = [](const AttnDims& x, const AttnDims& y) {
    return x.B == y.B && x.n == y.n && x.p == y.p && x.f == y.f && x.Hq == y.Hq &&
           x.Hkv == y.Hkv && x.D == y.D && x.tok_bf16 == y.tok_bf16 && x.row_bf16 == y.row_bf16 &&
           x.window == y.window && x.seg.packed == y.seg.packed &&
           (!x.seg.packed ||
            std::equal(x.seg.off, x.seg.off + x.seg.packed + 1, y.seg.off));
  };
  for (const Entry& e : cache)
    if (e.used && same(e.d, d)) return e.pl;
  const BwdPlan pl = make_plan_bwd(d);
  cache[next_slot] = Entry{d, pl, true};
  next_slot = (next_slot + 1) % 8;
  return pl;
}

static BwdPlan make_plan_bwd(const AttnDims& d) {
  BwdPlan pl{};
  const int g = d.Hq / d.Hkv;
  pl.n_ct = (d.p + kBNB - 1) / kBNB;
  pl.n_tt = (d.n + kBNB - 1) / kBNB;
  pl.nqt = (d.n + kBQ - 1) / kBQ;
  const long long U = (long long)d.B * g * pl.nqt;       // units of a cartridge tile
  auto tok_units = [&](int t) { return (long long)g * (pl.nqt - t * (kBNB / kBQ)); };
  // float32 path: cartridge tiles only are split
  int s = 1;
  while (pl.n_ct > 0 && U / (2 * s) >= 8 &&
         ((long long)d.Hkv * (pl.n_ct * s + d.B * pl.n_tt) < 512 || U / s > 2 * tok_units(0)))
    s *= 2;
  pl.splits_c = s;
  pl.grid_c = d.Hkv * pl.n_ct * s;
  pl.grid_t = d.Hkv * d.B * pl.n_tt;
  // bf16 path: every key tile's units cut into pieces of at most kv_target
  // units (a tile of u units into ceil(u / T) nearly equal pieces), T chosen
  // by a model of the dispatch: the grid's pieces, in order, are dealt to the
  // 8 XCDs in contiguous ranges (the kernel's block id remap), and each XCD
  // starts its pieces in order on its first free workgroup slot (32 CUs, one
  // dK/dV workgroup each). A piece costs its units plus a fixed overhead, in
  // units, from measured per-workgroup timelines: ~7 uncut (operand rows,
  // pipeline fill and drain, result store), ~12 cut (with its partial store)
  // plus its share of the tile's reduction by the last piece (~10). The
  // candidate with the smallest modelled finish time wins, the largest T
  // among equals.
  {
    // query tiles below qt_hi(t, b) of sequence b see a row of key tile t
    // (all of them, or with a sliding window those below the window end of
    // the tile's last row); token tile t exists for sequences longer than
    // t * 128
    auto len_of = [&](int b) { return d.seg.len(b, d.n); };
    auto qt_hi = [&](bool c, int t, int b) -> long long {
      const long long nq = (len_of(b) + kBQ - 1) / kBQ;
      if (d.window <= 0) return nq;
      const long long last =
          std::min<long long>((long long)t * kBNB + kBNB - 1, (c ? d.p : len_of(b)) - 1);
      const long long hi = (c ? last - d.p : last) + d.window;
      return std::max(0LL, std::min<long long>(nq, (hi + kBQ - 1) / kBQ));
    };
    auto cart_units = [&](int t) {
      long long u = 0;
      for (int b = 0; b < d.B; ++b) u += (long long)g * qt_hi(true, t, b);
      return u;
    };
    auto tok_units_w = [&](int t, int b) {
      return (long long)g * (qt_hi(false, t, b) - t * (kBNB / kBQ));
    };
    auto has_tile = [&](int t, int b) { return (long long)t * kBNB < len_of(b); };
    const bool windowed = d.window > 0;
    const long long Uc = pl.n_ct > 0 ? cart_units(0) : 0;   // every tile's, without a window
    long long t_max = 0;   // every tile one piece
    for (int t = 0; t < pl.n_ct; ++t) t_max = std::max(t_max, windowed ? cart_units(t) : Uc);
    for (int t = 0; t < pl.n_tt; ++t)
      for (int b = 0; b < d.B; ++b)
        if (has_tile(t, b)) t_max = std::max(t_max, tok_units_w(t, b));
    t_max = std::max(t_max, 1LL);
    const int slots = 32;   // one dK/dV workgroup per CU
    auto finish = [&](long long T, long long Tt) {
      std::vector<std::pair<long long, long long>> pieces;   // (units, pieces of its tile)
      auto tile = [&](long long u, bool at_least_one, long long T) {
        long long ns = (u + T - 1) / T;
        if (at_least_one && ns < 1) ns = 1;
        for (long long i = 0; i < ns; ++i) pieces.emplace_back((i + 1) * u / ns - i * u / ns, ns);
      };
      for (int kv = 0; kv < d.Hkv; ++kv) {
        if (!windowed) {
          // cartridge tiles split-major (every tile has the same pieces)
          const long long ns = (Uc + T - 1) / T;
          for (long long i = 0; i < ns; ++i)
            for (int c = 0; c < pl.n_ct; ++c)
              pieces.emplace_back((i + 1) * Uc / ns - i * Uc / ns, ns);
        } else {
          for (int c = 0; c < pl.n_ct; ++c) tile(cart_units(c), true, T);
        }
        for (int t = 0; t < pl.n_tt; ++t)
          for (int b = 0; b < d.B; ++b)
            if (has_tile(t, b)) tile(tok_units_w(t, b), false, Tt);
      }
      const size_t G = pieces.size(), q = G / 8, r = G % 8;
      double worst = 0.0;
      size_t first = 0;
      std::vector<double> slot(slots);   // min-heap of slot free times
      for (size_t x = 0; x < 8; ++x) {
        const size_t cnt = x < r ? q + 1 : q;
        std::fill(slot.begin(), slot.end(), 0.0);
        for (size_t i = first; i < first + cnt; ++i) {
          std::pop_heap(slot.begin(), slot.end(), std::greater<double>());
          slot.back() += (double)pieces[i].first +
                         (pieces[i].second > 1 ? 12.0 + 10.0 / (double)pieces[i].second : 7.0);
          std::push_heap(slot.begin(), slot.end(), std::greater<double>());
        }
        worst = std::max(worst, *std::max_element(slot.begin(), slot.end()));
        first += cnt;
      }
      return worst;
    };
    // Token tiles may be cut finer than cartridge tiles (Tt <= T): the
    // causal token tiles come last in each XCD's range, and smaller pieces
    // there even out the finish when the cartridge tiles are dealt whole.
    long long T = t_max, Tt = t_max;
    double best = finish(T, Tt);
    for (int k = 1; k <= 8; ++k) {
      const long long c = k == 1 ? t_max : std::max(4LL, (t_max + k - 1) / k);
      for (int kt = k; kt <= 8; ++kt) {
        const long long ct = kt == 1 ? t_max : std::max(4LL, (t_max + kt - 1) / kt);
        if (ct > c || (c == T && ct == Tt)) continue;
        const double f = finish(c, ct);
        if (f < best - 1e-9) { best = f; T = c; Tt = ct; }
      }
    }
    pl.kv_target = (int)T;
    pl.kv_ttok = (int)Tt;
    if (!windowed) {
      pl.kv_splits_c = pl.n_ct > 0 ? (int)((Uc + T - 1) / T) : 1;
      pl.kv_cart_pieces = pl.n_ct * pl.kv_splits_c;
    } else {
      pl.kv_splits_c = 1;
      pl.kv_cart_pieces = 0;
      for (int t = 0; t < pl.n_ct; ++t) {
        const int ns = std::max(1, (int)((cart_units(t) + T - 1) / T));
        pl.kv_splits_c = std::max(pl.kv_splits_c, ns);
        pl.kv_cart_pieces += ns;
      }
    }
    int ptok = 0, stmax = 1;
    for (int t = 0; t < pl.n_tt; ++t)
      for (int b = 0; b < d.B; ++b) {
        if (!has_tile(t, b)) continue;
        const int ns = (int)((tok_units_w(t, b) + Tt - 1) / Tt);
        ptok += ns;
        stmax = std::max(stmax, ns);
      }
    pl.kv_tok_pieces = ptok;
    pl.kv_ptok = d.B > 0 ? ptok / d.B : 0;   // per sequence, uniform batches only
    pl.kv_stmax = pl.n_tt > 0 ? stmax : 1;
    pl.grid_kv = d.Hkv * (pl.kv_cart_pieces + ptok);
    if (d.tok_bf16 && pl.kv_stmax > 1)
      pl.tok_part_bytes =
          (size_t)pl.kv_stmax * d.B * pl.n_tt * kBNB * d.Hkv * d.D * sizeof(float);
    if (d.tok_bf16) pl.cnt_bytes = (size_t)d.Hkv * (pl.n_ct + d.B * pl.n_tt) * sizeof(int);
  }
  pl.dq_bytes = d.tok_bf16 ? 0 : (size_t)d.B * d.n * d.Hq * d.D * sizeof(float);
  {
    // dQ workgroups of kDqWaves waves x 32 query rows, the q-heads of a GQA
    // group packed as extra rows (up to 4 per workgroup); key tiles split
    // while the grid is small (under two rounds of 4-wave workgroups)
    const int g = d.Hq / d.Hkv;
    pl.hpw = (g % 4 == 0) ? 4 : ((g % 2 == 0) ? 2 : 1);
    pl.wph = kDqWaves / pl.hpw;
    pl.n_hg = g / pl.hpw;
    pl.n_qb = (d.n + 32 * pl.wph - 1) / (32 * pl.wph);
    const long long base = (long long)d.Hkv * d.B * pl.n_hg * pl.n_qb;
    const int min_tiles = (d.p + kKvTile - 1) / kKvTile + 1;
    int qs = 1;
    if (d.tok_bf16)
      while (base * qs < 512 * 4 / kDqWaves && (qs * 2) * 4 <= min_tiles) qs *= 2;
    pl.q_splits = qs;
    pl.grid_q = (int)(base * qs);
    // two workgroups per CU: a grid of at most 512 runs in one round
    // (long-cartridge layer: dQ 1-2% faster with the blocks paired; grids of
    // several rounds ran faster longest-first, and key-split grids no faster)
    pl.q_pair = pl.grid_q <= 256 * (8 / kDqWaves) && qs == 1;
    if (qs > 1) pl.dq_part_bytes = (size_t)qs * d.B * d.n * d.Hq * d.D * sizeof(float);
  }
  pl.delta_bytes = (size_t)d.B * d.Hq * d.n * sizeof(float);   // and as much for lse2
  const int sc = d.tok_bf16 ? pl.kv_splits_c : s;
  // (bf16: whole 128-key tiles of lane-major words; float32: rows)
  pl.part_bytes =
      sc > 1 ? (size_t)sc * (d.tok_bf16 ? pl.n_ct * kBNB : d.p) * d.Hkv * d.D * sizeof(float) : 0;
  if (d.tok_bf16 && !d.row_bf16 && d.p > 0)
    pl.shadow_bytes = 2 * (size_t)d.p * d.Hkv * d.D * sizeof(uint16_t);
  return pl;
}

size_t bwd_workspace_bytes(const AttnDims& d) {
  const BwdPlan pl = plan_bwd(d);
  return align256(pl.shadow_bytes) + align256(pl.dq_bytes) + 2 * align256(pl.delta_bytes) +
         2 * align256(pl.part_bytes) + 2 * align256(pl.tok_part_bytes) +
         align256(pl.dq_part_bytes) + align256(pl.cnt_bytes);
}

// float32 reference mode: preprocess, generic kernel (dQ by atomics), dQ
// conversion, split reduction.
template <int D>
static hipError_t launch_bwd_f32(const BwdArgs& a, const BwdPlan& pl, hipStream_t st) {
  const int rows = a.B * a.n * a.Hq;
  const int tok_rows = a.seg.rows(a.B, a.n) * a.Hq;   // packed: the rows that exist
  CART_LAUNCH("bwd_preprocess", (bwd_preprocess<float, D>), (rows + 15) / 16, 256, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  CART_LAUNCH("attn_bwd", (attn_bwd_kernel<float, float, D>), pl.grid_c + pl.grid_t, kThreads, 0,
              st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t n4 = (size_t)tok_rows * D / 4;
  CART_LAUNCH("bwd_dq_finalize", (bwd_dq_finalize<float>), (unsigned)((n4 + 255) / 256), 256, 0, st,
              a.dq_acc, reinterpret_cast<float*>(a.dq), n4);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (pl.splits_c > 1) {
    const size_t total = (size_t)a.p * a.Hkv * D;
    CART_LAUNCH("bwd_cart_reduce", (bwd_cart_reduce_t<D>), (unsigned)((total + 255) / 256), 256, 0,
                st, a);
    e = hipGetLastError();
  }
  return e;
}

// bf16: preprocess, dK/dV kernel (its pieces reduced in the kernel), dQ
// kernel, dQ split reduction.
template <int D>
static hipError_t launch_bwd_bf16(const BwdArgs& a, const BwdPlan& pl, hipStream_t st) {
  const int rows = a.B * a.n * a.Hq;
  CART_LAUNCH("bwd_preprocess", (bwd_preprocess<bf16, D>), (rows + 15) / 16, 256, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  CART_LAUNCH("attn_bwd", (attn_bwd_kv_kernel<D>), pl.grid_kv, kKvThreads, 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  CART_LAUNCH("attn_bwd_dq", (attn_bwd_dq_kernel<D>), pl.grid_q, 64 * kDqWaves, 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (pl.q_splits > 1) {
    const size_t n4 = (size_t)a.B * a.n * a.Hq * (D / 4);
    CART_LAUNCH("bwd_dq_combine", (bwd_dq_combine), (unsigned)((n4 + 255) / 256), 256, 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return e;
}

hipError_t launch_bwd(const AttnDims& d, const void* q, const void* k_tok, const void* v_tok,
                      const void* k_cart, const void* v_cart, const void* out,
                      const float* lse, const void* dout, void* dq, void* dk_tok,
                      void* dv_tok, float* dk_cart, float* dv_cart, bool accumulate,
                      void* ws, hipStream_t st) {
  const BwdPlan pl = plan_bwd(d);
  BwdArgs a{};
  char* w = reinterpret_cast<char*>(ws);
  if (pl.shadow_bytes) {
    // the preprocess kernel (bf16 path, which is the only one with a shadow)
    // rounds the rows before the kernels that read them
    const size_t n = (size_t)d.p * d.Hkv * d.D;
    bf16* kb = reinterpret_cast<bf16*>(w);
    bf16* vb = kb + n;
    a.cast_k = reinterpret_cast<const f32x4*>(k_cart);
    a.cast_v = reinterpret_cast<const f32x4*>(v_cart);
    a.cast_kb = reinterpret_cast<bf16x4*>(kb);
    a.cast_vb = reinterpret_cast<bf16x4*>(vb);
    a.cast_n4 = n / 4;
    k_cart = kb;
    v_cart = vb;
    w += align256(pl.shadow_bytes);
  }
  a.q = q; a.k_tok = k_tok; a.v_tok = v_tok; a.k_cart = k_cart; a.v_cart = v_cart;
  a.out = out; a.dout = dout; a.lse = lse;
  a.dq_acc = reinterpret_cast<float*>(w);
  w += align256(pl.dq_bytes);
  a.delta = reinterpret_cast<float*>(w);
  w += align256(pl.delta_bytes);
  a.lse2 = reinterpret_cast<float*>(w);
  w += align256(pl.delta_bytes);
  a.dk_part = pl.part_bytes ? reinterpret_cast<float*>(w) : nullptr;
  w += align256(pl.part_bytes);
  a.dv_part = pl.part_bytes ? reinterpret_cast<float*>(w) : nullptr;
  w += align256(pl.part_bytes);
  a.dk_tpart = pl.tok_part_bytes ? reinterpret_cast<float*>(w) : nullptr;
  w += align256(pl.tok_part_bytes);
  a.dv_tpart = pl.tok_part_bytes ? reinterpret_cast<float*>(w) : nullptr;
  w += align256(pl.tok_part_bytes);
  a.dq_part = pl.dq_part_bytes ? reinterpret_cast<float*>(w) : nullptr;
  w += align256(pl.dq_part_bytes);
  a.kv_cnt = pl.cnt_bytes ? reinterpret_cast<int*>(w) : nullptr;
  a.n_cnt = (int)(pl.cnt_bytes / sizeof(int));
  a.dq = dq; a.dk_tok = dk_tok; a.dv_tok = dv_tok; a.dk_cart = dk_cart; a.dv_cart = dv_cart;
  a.B = d.B; a.n = d.n; a.p = d.p; a.f = d.f; a.Hq = d.Hq; a.Hkv = d.Hkv; a.g = d.Hq / d.Hkv;
  a.n_ct = pl.n_ct; a.n_tt = pl.n_tt; a.nqt = pl.nqt;
  a.splits_c = d.tok_bf16 ? pl.kv_splits_c : pl.splits_c;
  a.kv_target = pl.kv_target; a.kv_ptok = pl.kv_ptok; a.kv_stmax = pl.kv_stmax;
  a.kv_ttok = pl.kv_ttok;
  a.q_splits = pl.q_splits;
  a.kv_cart_pieces = pl.kv_cart_pieces;
  a.kv_tok_pieces = pl.kv_tok_pieces;
  a.window = d.window;
  a.seg = d.seg;
  a.D4 = d.D / 4;
  a.accumulate = accumulate ? 1 : 0;
  a.scale = d.scale;
  a.scale_log2 = d.scale * kLog2e;
  a.hpw = pl.hpw; a.wph = pl.wph; a.n_hg = pl.n_hg; a.n_qb = pl.n_qb; a.q_pair = pl.q_pair;
  a.zero_dq = d.tok_bf16 ? 0 : 1;
  if (d.tok_bf16) return d.D == 128 ? launch_bwd_bf16<128>(a, pl, st) : launch_bwd_bf16<64>(a, pl, st);
  return d.D == 128 ? launch_bwd_f32<128>(a, pl, st) : launch_bwd_f32<64>(a, pl, st);
}

}  // namespace cartattn
