// Forward pass of end-aligned causal grouped-query attention over
// concat(cartridge rows, real tokens).
//
// Source: "Cartridges: trained KV-prefix corpus compression", section
// "Semantics (pinned to the reference implementation)": the sequence axis
// holds concat(sink, trainable, tokens); the grouped attention's causal mask
// is aligned to the end (source_offset = kv_seq - q_seq), so each query has
// all prefix rows in view and, among the tokens, itself and those before it.
//
// Design (gfx950):
//  * one workgroup = 4 waves = 128 query rows of ONE kv-head group: the GQA
//    q-heads of the group are packed as extra rows, so every K/V tile staged
//    in LDS serves all of them;
//  * each wave owns 32 query rows of one q-head; its Q^T fragments stay in
//    registers for the whole key loop;
//  * S^T = K Q^T on the 32x32 MFMA (bf16 32x32x16, or f32 32x32x2 in the
//    float32 reference mode): rows are keys, columns are queries, so the
//    softmax statistics of a query live in one lane pair and the f32 result,
//    cast to bf16, is directly the B operand of O^T += V^T P^T;
//  * online softmax in f32 in the exp2 domain (scale * log2 e folded in);
//  * the key loop streams cartridge tiles (no mask) and then token tiles
//    (mask only on the diagonal tiles); the concat is never materialized;
//  * when the grid would be too small to fill 256 CUs the key range is split
//    and a combine kernel merges the partial (O, LSE) pairs by log-sum-exp;
//  * block ids are remapped so each XCD works on one contiguous range of kv
//    heads, keeping that head's cartridge tiles in its own L2.
#include <math.h>

#include "common.hpp"
#include "kvtiles.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace cartattn {

namespace {

constexpr int kBN = 64;        // keys per LDS tile
constexpr int kThreads = 256;  // 4 waves

struct FwdArgs {
  const void* q;
  const void* k_tok;
  const void* v_tok;
  const void* k_cart;
  const void* v_cart;
  void* out;
  float* lse;
  float* o_part;
  float* lse_part;
  int B, n, p, Hq, Hkv, g;
  int hpw, wph, n_hg, n_qb, n_splits;
  int window;          // > 0: sliding window (positions above p + i - window)
  float scale_log2;
  Segs seg;            // token rows of each sequence; n is the longest
};

template <typename T> struct Lds;
template <> struct Lds<bf16> {
  static constexpr int kpad = 8;   // K row stride D+8 bf16: conflict-free b128 reads
  static constexpr int vpad = 4;   // V^T row stride 68 bf16: conflict-free b64 reads
};
template <> struct Lds<float> {
  static constexpr int kpad = 1;   // odd strides: conflict-free b32 reads
  static constexpr int vpad = 1;
};

// A-operand fragment of V^T for MFMA m over a 32-key group whose LDS row
// (one head_dim column of V) starts at `row`: item t holds key d_row(m*KPL+t).
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag vt_frag(const T* row, int m, int hl);
template <>
__device__ __forceinline__ bf16x8 vt_frag<bf16>(const bf16* row, int m, int hl) {
  // keys 16m + 4hl + {0..3} and 16m + 8 + 4hl + {0..3}
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 16 * m + 4 * hl);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 16 * m + 8 + 4 * hl);
  bf16x8 f;
  f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
  f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
  return f;
}
template <>
__device__ __forceinline__ float vt_frag<float>(const float* row, int m, int hl) {
  return row[d_row(m, hl)];
}

template <typename T>
__device__ __forceinline__ void lds_store8(T* p, const float (&v)[8]);
template <> __device__ __forceinline__ void lds_store8<bf16>(bf16* p, const float (&v)[8]) {
  store8<bf16>(p, v);
}
template <> __device__ __forceinline__ void lds_store8<float>(float* p, const float (&v)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = v[e];
}

// Stage one tile of `rows` key/value rows into LDS: K row-major [BN][KSTR],
// V transposed [D][VSTR]. Rows at or beyond `rows` are zero-filled.
template <typename T, typename TS, int D>
__device__ __forceinline__ void stage_tile(T* Ks, T* Vt, const TS* kbase, const TS* vbase,
                                           size_t row_stride, int rows, int tid) {
  constexpr int KSTR = D + Lds<T>::kpad;
  constexpr int VSTR = kBN + Lds<T>::vpad;
  constexpr int CPR = D / 8;               // 8-element chunks per row
  constexpr int NCH = kBN * CPR / kThreads;
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int c = tid + u * kThreads;
    const int r = c / CPR;
    const int col = (c % CPR) * 8;
    float kv8[8], vv8[8];
    if (r < rows) {
      load8<TS>(kbase + (size_t)r * row_stride + col, kv8);
      load8<TS>(vbase + (size_t)r * row_stride + col, vv8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) { kv8[e] = 0.f; vv8[e] = 0.f; }
    }
    lds_store8<T>(Ks + r * KSTR + col, kv8);
#pragma unroll
    for (int e = 0; e < 8; ++e) Vt[(col + e) * VSTR + r] = from_f32<T>(vv8[e]);
  }
}

template <typename T, typename TR, int D>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(FwdArgs a) {
  using M = Mfma<T>;
  constexpr int KPL = M::KPL;
  constexpr int KSTEP = M::KSTEP;
  constexpr int NKS = D / KSTEP;
  constexpr int NDB = D / 32;
  constexpr int NKH = kBN / 32;
  constexpr int NPV = 16 / KPL;   // PV MFMAs per 32-key group
  constexpr int KSTR = D + Lds<T>::kpad;
  constexpr int VSTR = kBN + Lds<T>::vpad;
  __shared__ __align__(16) T Ks[kBN * KSTR];
  __shared__ __align__(16) T Vt[D * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  int lg = xcd_remap(blockIdx.x, gridDim.x);
  const int split = lg % a.n_splits; lg /= a.n_splits;
  const int qb = a.n_qb - 1 - (lg % a.n_qb); lg /= a.n_qb;   // longest blocks first
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
  const int n_ct = (a.p + kBN - 1) / kBN;
  const int nt = n_ct + wg_last / kBN + 1;
  const int t_begin = (int)((long long)split * nt / a.n_splits);
  const int t_end = (int)((long long)(split + 1) * nt / a.n_splits);

  // Q^T fragments (B operand): lane (q + 32 hl) holds Q[q][ks*KSTEP + hl*KPL ..].
  typename M::frag qf[NKS];
  {
    const int qi = min(my_i, nb - 1);
    const T* qp = reinterpret_cast<const T*>(a.q) + (((size_t)base + qi) * a.Hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = load_frag<T>(qp + ks * KSTEP + hl * KPL);
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  const size_t tok_stride = (size_t)a.Hkv * D;   // between consecutive rows
  for (int t = t_begin; t < t_end; ++t) {
    const bool cart = t < n_ct;
    const int j0 = cart ? t * kBN : (t - n_ct) * kBN;
    const int rows = cart ? min(kBN, a.p - j0) : min(kBN, nb - j0);
    __syncthreads();
    if (cart) {
      const TR* kb = reinterpret_cast<const TR*>(a.k_cart) + ((size_t)j0 * a.Hkv + kv) * D;
      const TR* vb = reinterpret_cast<const TR*>(a.v_cart) + ((size_t)j0 * a.Hkv + kv) * D;
      stage_tile<T, TR, D>(Ks, Vt, kb, vb, tok_stride, rows, tid);
    } else {
      const size_t off = (((size_t)base + j0) * a.Hkv + kv) * D;
      stage_tile<T, T, D>(Ks, Vt, reinterpret_cast<const T*>(a.k_tok) + off,
                          reinterpret_cast<const T*>(a.v_tok) + off, tok_stride, rows, tid);
    }
    __syncthreads();
    if (!wave_active) continue;
    if (!cart && j0 > i0 + 31) continue;   // whole tile above this wave's diagonal

    // S^T = K Q^T for the tile's 32-key groups.
    f32x16 s[NKH];
#pragma unroll
    for (int kh = 0; kh < NKH; ++kh) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kh][r] = 0.f;
      const T* krow = Ks + (32 * kh + l32) * KSTR + hl * KPL;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        s[kh] = M::mma(load_frag<T>(krow + ks * KSTEP), qf[ks], s[kh]);
    }

    // Mask, scale into the exp2 domain, running max.
    const bool diag = !cart && (j0 + kBN - 1 > i0);
    float mx = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < NKH; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kh + d_row(r, hl);
        bool vis = key < rows;
        if (diag) vis = vis && (j0 + key <= my_i);
        if (a.window > 0) vis = vis && ((cart ? j0 : a.p + j0) + key > my_i + a.p - a.window);
        const float v = vis ? s[kh][r] * a.scale_log2 : -INFINITY;
        s[kh][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = wave_max_halves(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float ls = 0.f;
#pragma unroll
    for (int kh = 0; kh < NKH; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = exp2f(s[kh][r] - m_use);
        s[kh][r] = pv;
        ls += pv;
      }
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;

    // O^T += V^T P^T: P^T (cast to T) is the B operand straight from s.
#pragma unroll
    for (int kh = 0; kh < NKH; ++kh)
#pragma unroll
      for (int m = 0; m < NPV; ++m) {
        const typename M::frag pf = pack_regs<T>(s[kh], m);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const T* vrow = Vt + (32 * db + l32) * VSTR + 32 * kh;
          acc[db] = M::mma(vt_frag<T>(vrow, m, hl), pf, acc[db]);
        }
      }
  }

  if (!wave_active || my_i >= nb) return;
  l_run = wave_sum_halves(l_run);
  const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  if (a.n_splits == 1) {
    T* op = reinterpret_cast<T*>(a.out) + (((size_t)base + my_i) * a.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          op[32 * db + 8 * c + 4 * hl + e] = from_f32<T>(acc[db][4 * c + e] * inv_l);
    if (hl == 0) a.lse[((size_t)b * a.Hq + h) * a.n + my_i] = lse;
  } else {
    float* op = a.o_part + ((((size_t)split * a.B + b) * a.n + my_i) * a.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float4 v4 = make_float4(acc[db][4 * c] * inv_l, acc[db][4 * c + 1] * inv_l,
                                acc[db][4 * c + 2] * inv_l, acc[db][4 * c + 3] * inv_l);
        *reinterpret_cast<float4*>(op + 32 * db + 8 * c + 4 * hl) = v4;
      }
    if (hl == 0)
      a.lse_part[(((size_t)split * a.B + b) * a.Hq + h) * a.n + my_i] = lse;
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel. Same work decomposition and softmax as attn_fwd_kernel, with:
//  * K and V tiles copied global -> LDS by direct (VGPR-free) loads into
//    padded, double-buffered tiles: the copy of tile t+1 runs while tile t
//    is multiplied, and the loop has one barrier per tile;
//  * the V^T operand of O^T += V^T P^T read with LDS transpose reads, so no
//    transposed copy of V is ever written;
//  * the running max is taken on raw scores and each probability costs one
//    FMA and one exp2; the O accumulator is rescaled only when some query's
//    max has grown by more than 2^8 since its last rescale (exact: the
//    probabilities are then at most 256, well inside f32 and bf16 range).
// Cartridge rows arrive as bf16 (f32 master rows are cast first).
// One key tile of the online softmax for one wave (32 queries x 64 keys).
// The K and V tiles are at LDS byte addresses kst, vst. All LDS reads are
// issued by the inline-assembly helpers with explicit waits (the copy of the
// next tile into the other stage is in flight meanwhile), one k-step ahead
// of the MFMAs that use them.
// Where a tile's compute issues the copy of the next tile: copies
// [0, kFwdCopyA) before the S MFMAs, [kFwdCopyA, kFwdCopyB) after them,
// the rest before the PV MFMAs. All before the S MFMAs measured fastest; a
// copy issued between MFMAs stalls the MFMAs behind it until the memory
// pipeline takes it.
template <int D> constexpr int kFwdCopyA = KvCopy<D>::N;
template <int D> constexpr int kFwdCopyB = KvCopy<D>::N;

template <int D>
__device__ __forceinline__ void fwd_compute(uint32_t kst, uint32_t vst, const KvTile& f,
                                            const bf16x8 (&qf)[D / 16], f32x16 (&acc)[D / 32],
                                            float& m_ref, float& l_run, float c, int i0,
                                            int my_i, int lane, int win_lo, const KvCopy<D>& cp,
                                            const KvMap<D>& kmap, int wave) {
  using M = Mfma<bf16>;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  using TL = Tile<D>;
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  // S^T = K Q^T for the two 32-key halves: K row fragments (row 32 kh + l32,
  // 8 elements at 16 ks + 8 hl), two reads per k-step.
  f32x16 s[2];
  {
    const uint32_t kb = kst + TL::off(l32, 8 * hl);
    bf16x8 kfr[3][2];
    auto rd = [&](auto KS) {
      constexpr int ks = decltype(KS)::value;
      kfr[ks % 3][0] = __builtin_bit_cast(bf16x8, lds_read16<32 * ks>(kb));
      kfr[ks % 3][1] = __builtin_bit_cast(bf16x8, lds_read16<TL::rows(32) + 32 * ks>(kb));
    };
    cp.template range<0, kFwdCopyA<D>>(kmap, wave, lane);
#pragma unroll
    for (int r = 0; r < 16; ++r) { s[0][r] = 0.f; s[1][r] = 0.f; }
    rd(std::integral_constant<int, 0>{});
    rd(std::integral_constant<int, 1>{});
    // MFMA phases run at a raised wave priority, so that the other wave of
    // the SIMD fills the VALU slots with its softmax meanwhile
    __builtin_amdgcn_s_setprio(1);
    static_for<NKS>([&](auto KS) {
      constexpr int ks = decltype(KS)::value;
      if constexpr (ks + 2 < NKS) {
        rd(std::integral_constant<int, ks + 2>{});
        lds_wait<4>();
      } else if constexpr (ks + 1 < NKS) {
        lds_wait<2>();
      } else {
        lds_wait<0>();
      }
      lds_tie(kfr[ks % 3][0]);
      lds_tie(kfr[ks % 3][1]);
      __builtin_amdgcn_sched_barrier(0);
      s[0] = M::mma(kfr[ks % 3][0], qf[ks], s[0]);
      s[1] = M::mma(kfr[ks % 3][1], qf[ks], s[1]);
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  __builtin_amdgcn_s_setprio(0);
  cp.template range<kFwdCopyA<D>, kFwdCopyB<D>>(kmap, wave, lane);
  // V^T fragments for O^T += V^T P^T, by transpose reads of rows 32 kh + 16 m
  // .. for step j = (kh, m); the first step's reads are issued here, so that
  // they land while the softmax runs.
  const uint32_t vb = vst + TL::off(4 * hl + ((lane & 15) >> 2), 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  bf16x8 va[2][NDB];
  auto rdv = [&](auto J, int slot) {
    constexpr int j = decltype(J)::value;
    static_for<NDB>([&](auto DB) {
      constexpr int db = decltype(DB)::value;
      constexpr int off = TL::rows(16 * j) + 2 * 32 * db;
      va[slot][db] = cat8(lds_tr4<off>(vb), lds_tr4<off + TL::rows(8)>(vb));
    });
  };
  rdv(std::integral_constant<int, 0>{}, 0);
  // Mask: key k = 32 kh + d_row(r, hl) of the tile is visible iff lo <= k <
  // lim (its row exists and, for a token tile, it is not after the query;
  // with a sliding window, it is not before the window of the query, whose
  // first visible position is win_lo + my_i - i0 for this lane).
  if (f.rows < kBN || (!f.cart && f.j0 + kBN - 1 > i0) || f.abs0 < win_lo + 31) {
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
  float mx = -INFINITY;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kh][r]);
  const float mxs = wave_max_halves(mx) * c;
  const bool grow = mxs > m_ref + 8.f;
  if (__any(grow)) {
    const float m_new = grow ? mxs : m_ref;
    const float alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    m_ref = m_new;
  }
  const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
  float ls = 0.f;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pv_ = __builtin_amdgcn_exp2f(fmaf(s[kh][r], c, -m_use));
      s[kh][r] = pv_;
      ls += pv_;
    }
  l_run += ls;
  cp.template range<kFwdCopyB<D>, KvCopy<D>::N>(kmap, wave, lane);
  // O^T += V^T P^T in four steps j = (kh, m), each step's V^T reads (8 per
  // step) issued one step ahead.
  {
    __builtin_amdgcn_s_setprio(1);
    static_for<4>([&](auto J) {
      constexpr int j = decltype(J)::value;
      constexpr int kh = j / 2, m = j % 2;
      if constexpr (j + 1 < 4) {
        rdv(std::integral_constant<int, j + 1>{}, (j + 1) & 1);
        lds_wait<2 * NDB>();
      } else {
        lds_wait<0>();
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) lds_tie(va[j & 1][db]);
      const bf16x8 pf = pack_regs<bf16>(s[kh], m);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] = M::mma(va[j & 1][db], pf, acc[db]);
      __builtin_amdgcn_sched_barrier(0);
    });
    __builtin_amdgcn_s_setprio(0);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(FwdArgs a) {
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __align__(16) bf16 K0[tile_elems<D, kBN>()];
  __shared__ __align__(16) bf16 V0[tile_elems<D, kBN>()];
  __shared__ __align__(16) bf16 K1[tile_elems<D, kBN>()];
  __shared__ __align__(16) bf16 V1[tile_elems<D, kBN>()];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  int lg = xcd_remap(blockIdx.x, gridDim.x);
  const int split = lg % a.n_splits; lg /= a.n_splits;
  const int qb = a.n_qb - 1 - (lg % a.n_qb); lg /= a.n_qb;
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
  const int n_ct = (a.p + kBN - 1) / kBN;
  const int nt = n_ct + wg_last / kBN + 1;
  // with a sliding window the tiles before the workgroup's first window are
  // skipped; the rest are split between the key-split workgroups
  const int t_lo = first_window_tile(a.window, qb * a.wph * 32, a.p, n_ct);
  const int t_begin = t_lo + (int)((long long)split * (nt - t_lo) / a.n_splits);
  const int t_end = t_lo + (int)((long long)(split + 1) * (nt - t_lo) / a.n_splits);
  // first position the wave's first query sees (no window: far below 0)
  const int win_lo = a.window > 0 ? a.p + i0 - a.window + 1 : -(1 << 30);

  const KvSrc<D> src = kv_src<D>(a.k_cart, a.v_cart, a.k_tok, a.v_tok, base, nb, a.p, a.Hkv, kv);
  const KvMap<D> kmap = kv_map<D>(a.Hkv, wave, lane);
  KvWalk<D> walk(src, n_ct, t_begin);
  if (t_begin < t_end) kv_copy<D>(walk, K0, V0, true).all(kmap, wave, lane);

  bf16x8 qf[NKS];
  {
    const int qi = min(my_i, nb - 1);
    const bf16* qp = reinterpret_cast<const bf16*>(a.q) + (((size_t)base + qi) * a.Hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16 + hl * 8);
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m_ref = -INFINITY;   // scaled (log2-domain) reference max of this query
  float l_run = 0.f;
  const float c = a.scale_log2;

  // Two tiles per trip, stage 0 then stage 1, so every LDS address is static.
  // After the barrier no wave reads the other stage any more; the copy of
  // the next tile into it is issued by this tile's compute (all at once by a
  // wave that skips the tile).
  for (int t = t_begin; t < t_end; t += 2) {
    CART_WAIT_VMCNT(0);
    lds_barrier();
    {
      if (t + 1 < t_end) walk.next();
      const KvCopy<D> cp = kv_copy<D>(walk, K1, V1, t + 1 < t_end);
      const KvTile f = kv_tile(t, n_ct, a.p, nb);
      if (wave_active && (f.cart || f.j0 <= i0 + 31) && f.abs0 + kBN > win_lo)
        fwd_compute<D>(lds_addr(K0), lds_addr(V0), f, qf, acc, m_ref, l_run, c, i0, my_i, lane,
                       win_lo, cp, kmap, wave);
      else
        cp.all(kmap, wave, lane);
    }
    if (t + 1 >= t_end) break;
    CART_WAIT_VMCNT(0);
    lds_barrier();
    {
      if (t + 2 < t_end) walk.next();
      const KvCopy<D> cp = kv_copy<D>(walk, K0, V0, t + 2 < t_end);
      const KvTile f = kv_tile(t + 1, n_ct, a.p, nb);
      if (wave_active && (f.cart || f.j0 <= i0 + 31) && f.abs0 + kBN > win_lo)
        fwd_compute<D>(lds_addr(K1), lds_addr(V1), f, qf, acc, m_ref, l_run, c, i0, my_i, lane,
                       win_lo, cp, kmap, wave);
      else
        cp.all(kmap, wave, lane);
    }
  }

  if (!wave_active || my_i >= nb) return;
  l_run = wave_sum_halves(l_run);
  const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse = l_run > 0.f ? (m_ref + log2f(l_run)) * kLn2 : -INFINITY;
  if (a.n_splits == 1) {
    bf16* op = reinterpret_cast<bf16*>(a.out) + (((size_t)base + my_i) * a.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (bf16)(acc[db][4 * cc + e] * inv_l);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * cc + 4 * hl) = o4;
      }
    if (hl == 0) a.lse[((size_t)b * a.Hq + h) * a.n + my_i] = lse;
  } else {
    float* op = a.o_part + ((((size_t)split * a.B + b) * a.n + my_i) * a.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        float4 v4 = make_float4(acc[db][4 * cc] * inv_l, acc[db][4 * cc + 1] * inv_l,
                                acc[db][4 * cc + 2] * inv_l, acc[db][4 * cc + 3] * inv_l);
        *reinterpret_cast<float4*>(op + 32 * db + 8 * cc + 4 * hl) = v4;
      }
    if (hl == 0)
      a.lse_part[(((size_t)split * a.B + b) * a.Hq + h) * a.n + my_i] = lse;
  }
}

// Merge split partials: lse = log sum_s exp(lse_s); O = sum_s exp(lse_s - lse) O_s.
// Merge the split-KV partials of each (b, i, h) row by their LSE. Sixteen
// lanes per row (D/16 output elements each), 16 rows per workgroup.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_fwd_combine(FwdArgs a) {
  constexpr int EPL = D / 16;
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);   // (b, i, h), h fastest
  const int sub = threadIdx.x & 15;
  if (row >= a.B * a.n * a.Hq) return;
  const int h = row % a.Hq;
  const int bi = row / a.Hq;
  const int i = bi % a.n;
  const int b = bi / a.n;
  if (i >= a.seg.len(b, a.n)) return;     // past a packed segment's end
  const size_t lrow = ((size_t)b * a.Hq + h) * a.n + i;
  const size_t lstride = (size_t)a.B * a.Hq * a.n;
  const size_t ostride = (size_t)a.B * a.n * a.Hq * D;
  float mx = -INFINITY;
#pragma unroll 4
  for (int s = 0; s < a.n_splits; ++s) mx = fmaxf(mx, a.lse_part[s * lstride + lrow]);
  float tot = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  const float* op = a.o_part + (size_t)row * D + sub * EPL;
#pragma unroll 4
  for (int s = 0; s < a.n_splits; ++s) {
    const float ls = a.lse_part[s * lstride + lrow];
    const float w = (ls == -INFINITY) ? 0.f : expf(ls - mx);
    tot += w;
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(op + s * ostride + e);
      o[e] += w * v.x; o[e + 1] += w * v.y; o[e + 2] += w * v.z; o[e + 3] += w * v.w;
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  T* out = reinterpret_cast<T*>(a.out) + (((size_t)a.seg.base(b, a.n) + i) * a.Hq + h) * D +
           sub * EPL;
#pragma unroll
  for (int e = 0; e < EPL; ++e) out[e] = from_f32<T>(o[e] * inv);
  if (sub == 0) a.lse[lrow] = mx + logf(tot);
}

}  // namespace

FwdPlan plan_fwd(const AttnDims& d) {
  FwdPlan pl{};
  const int g = d.Hq / d.Hkv;
  pl.hpw = (g % 4 == 0) ? 4 : ((g % 2 == 0) ? 2 : 1);
  pl.wph = 4 / pl.hpw;
  pl.n_hg = g / pl.hpw;
  pl.n_qb = (d.n + 32 * pl.wph - 1) / (32 * pl.wph);
  const long long base = (long long)d.Hkv * d.B * pl.n_hg * pl.n_qb;
  // Fewest key tiles any workgroup sees; never split below 4 tiles each.
  const int min_tiles = (d.p + kBN - 1) / kBN + 1;
  int splits = 1;
  while (base * splits < 512 && (splits * 2) * 4 <= min_tiles) splits *= 2;
  pl.n_splits = splits;
  pl.grid = (int)(base * splits);
  if (d.tok_bf16 && !d.row_bf16 && d.p > 0)
    pl.shadow_bytes = 2 * (size_t)d.p * d.Hkv * d.D * sizeof(uint16_t);
  if (splits > 1) {
    pl.o_part_bytes = (size_t)splits * d.B * d.n * d.Hq * d.D * sizeof(float);
    pl.lse_part_bytes = (size_t)splits * d.B * d.Hq * d.n * sizeof(float);
  }
  return pl;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t fwd_workspace_bytes(const AttnDims& d) {
  const FwdPlan pl = plan_fwd(d);
  return align256(pl.shadow_bytes) + align256(pl.o_part_bytes) + align256(pl.lse_part_bytes);
}

template <typename T, typename TR, int D>
static hipError_t launch_fwd_t(const FwdArgs& a, const FwdPlan& pl, hipStream_t st) {
  CART_LAUNCH("attn_fwd", (attn_fwd_kernel<T, TR, D>), pl.grid, kThreads, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.n_splits == 1) return e;
  CART_LAUNCH("attn_fwd_combine", (attn_fwd_combine<T, D>), (a.B * a.n * a.Hq + 15) / 16, 256, 0,
              st, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_fwd_bf16(const FwdArgs& a, const FwdPlan& pl, hipStream_t st) {
  CART_LAUNCH("attn_fwd", (attn_fwd_bf16_kernel<D>), pl.grid, kThreads, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.n_splits == 1) return e;
  CART_LAUNCH("attn_fwd_combine", (attn_fwd_combine<bf16, D>), (a.B * a.n * a.Hq + 15) / 16, 256, 0,
              st, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const AttnDims& d, const void* q, const void* k_tok, const void* v_tok,
                      const void* k_cart, const void* v_cart, void* out, float* lse,
                      void* ws, hipStream_t st) {
  const FwdPlan pl = plan_fwd(d);
  FwdArgs a{};
  char* w = reinterpret_cast<char*>(ws);
  if (pl.shadow_bytes) {
    // bf16 shadow of the f32 cartridge rows
    const size_t n = (size_t)d.p * d.Hkv * d.D;
    bf16* kb = reinterpret_cast<bf16*>(w);
    bf16* vb = kb + n;
    hipError_t e = launch_rows_to_bf16(reinterpret_cast<const float*>(k_cart),
                                       reinterpret_cast<const float*>(v_cart), kb, vb, n, st);
    if (e != hipSuccess) return e;
    k_cart = kb;
    v_cart = vb;
    w += align256(pl.shadow_bytes);
  }
  a.q = q; a.k_tok = k_tok; a.v_tok = v_tok; a.k_cart = k_cart; a.v_cart = v_cart;
  a.out = out; a.lse = lse;
  a.o_part = reinterpret_cast<float*>(w);
  a.lse_part = reinterpret_cast<float*>(w + align256(pl.o_part_bytes));
  a.B = d.B; a.n = d.n; a.p = d.p; a.Hq = d.Hq; a.Hkv = d.Hkv; a.g = d.Hq / d.Hkv;
  a.hpw = pl.hpw; a.wph = pl.wph; a.n_hg = pl.n_hg; a.n_qb = pl.n_qb; a.n_splits = pl.n_splits;
  a.window = d.window;
  a.seg = d.seg;
  a.scale_log2 = d.scale * kLog2e;
  if (d.tok_bf16)
    return d.D == 128 ? launch_fwd_bf16<128>(a, pl, st) : launch_fwd_bf16<64>(a, pl, st);
  if (d.D == 128) return launch_fwd_t<float, float, 128>(a, pl, st);
  return launch_fwd_t<float, float, 64>(a, pl, st);
}

}  // namespace cartattn
