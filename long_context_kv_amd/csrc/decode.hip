// Serving behind a cartridge: writing the prefix into a paged bf16 KV cache,
// appending rows, and the single-token decode step.
//
// Source: "Cartridges: trained KV-prefix corpus compression", section
// "Semantics (pinned to the reference implementation)", serving: an empty KV
// cache receives all p prefix rows in its own dtype, its length becomes p,
// and ordinary decoding resumes at position p; section
// "Composition": appending to the cache is the primitive; section "Evidence":
// decode behind the written prefix matches the trainer's cartridge eval.
//
// Cache layout: k_pages/v_pages are [n_pages][Hkv][16][D] bf16, so one
// (page, kv-head) is a contiguous 16*D*2-byte run (4 KiB at D = 128) and a
// decode workgroup streams whole runs. block_table maps (seq, logical page)
// to a physical page id.
//
// Decode is HBM-bound (4 flop per byte of K/V at a GQA group of 4): one
// one-wave workgroup per (sequence, kv head, split of the pages, chunk of up
// to 32 query rows); a sequence's pages are cut into ns = ceil(pages /
// pages-per-split) nearly equal splits, so the workgroups of a step run
// about equally long, and the splits are sized so that a step's workgroups
// are about as many as the GPU holds at once. The query rows of one kv head
// (its GQA q-heads, times the draft tokens of a verify step) are the columns
// of bf16 MFMAs, so each K/V byte is read once for all of them; the MFMA
// work is idle most of the time, but it costs the wave almost no issue slots,
// where per-row dot products on the VALU did (an earlier VALU kernel reached
// 5.3 TB/s at 4 rows per kv head and a third less at 8). The splits of a
// sequence are merged by log-sum-exp: on chip, when a launch has at most 8
// splits per sequence (one workgroup per (sequence, kv head, chunk), one
// wave per split, the partials exchanged through LDS), else by a second
// kernel over partials in the workspace.
#include <math.h>

#include <mutex>

#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace cartattn {

namespace {

constexpr int kPage = 16;
constexpr int kMaxPps = 256; // pages per split at most
constexpr int kPartHead = 4; // floats before a split partial's accumulator (m, l, 2 unused)

template <typename TS>
__global__ __launch_bounds__(256) void cache_append_kernel(CacheDims c, int seq, int start,
                                                           const TS* __restrict__ k,
                                                           const TS* __restrict__ v,
                                                           int n_rows) {
  const int cpr = c.D / 8;
  const size_t total = (size_t)n_rows * c.Hkv * cpr;
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e == 0) c.seq_lens[seq] = start + n_rows;
  if (e >= total) return;
  const int chunk = (int)(e % cpr);
  const int h = (int)((e / cpr) % c.Hkv);
  const int r = (int)(e / ((size_t)cpr * c.Hkv));
  const int row = start + r;
  const int lp = row / kPage;
  if (lp >= c.max_pages) return;
  const int page = c.block_table[(size_t)seq * c.max_pages + lp];
  if (page < 0 || page >= c.n_pages) return;
  const size_t src = ((size_t)r * c.Hkv + h) * c.D + chunk * 8;
  const size_t dst = (((size_t)page * c.Hkv + h) * kPage + row % kPage) * c.D + chunk * 8;
  float v8[8];
  load8<TS>(k + src, v8);
  store8<bf16>(reinterpret_cast<bf16*>(c.k_pages) + dst, v8);
  load8<TS>(v + src, v8);
  store8<bf16>(reinterpret_cast<bf16*>(c.v_pages) + dst, v8);
}

__global__ void cache_set_len_kernel(int32_t* seq_lens, int seq, int len) {
  if (threadIdx.x == 0 && blockIdx.x == 0) seq_lens[seq] = len;
}

// Append kq new rows per sequence at positions seq_len[s] .. seq_len[s] +
// kq - 1 (rows [s, t, Hkv, D] of k_new/v_new), then seq_len += kq.
__global__ __launch_bounds__(256) void decode_append_kernel(CacheDims c,
                                                            const bf16* __restrict__ k_new,
                                                            const bf16* __restrict__ v_new,
                                                            int kq) {
  const int s = blockIdx.x;
  const int cpr = c.D / 8;
  const int len = c.seq_lens[s];
  __syncthreads();   // every thread has read the old length
  for (int e = threadIdx.x; e < kq * c.Hkv * cpr; e += blockDim.x) {
    const int t = e / (c.Hkv * cpr);
    const int h = (e / cpr) % c.Hkv;
    const int chunk = e % cpr;
    const int row = len + t;
    const int lp = row / kPage;
    if (lp >= c.max_pages) continue;
    const int page = c.block_table[(size_t)s * c.max_pages + lp];
    if (page < 0 || page >= c.n_pages) continue;
    const size_t src = (((size_t)s * kq + t) * c.Hkv + h) * c.D + chunk * 8;
    const size_t dst = (((size_t)page * c.Hkv + h) * kPage + row % kPage) * c.D + chunk * 8;
    *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(c.k_pages) + dst) =
        *reinterpret_cast<const bf16x8*>(k_new + src);
    *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(c.v_pages) + dst) =
        *reinterpret_cast<const bf16x8*>(v_new + src);
  }
  __syncthreads();   // the old length is read by every thread before it moves
  if (threadIdx.x == 0) c.seq_lens[s] = len + kq;
}

struct DecArgs {
  CacheDims c;
  const bf16* q;       // [n_seqs][kq][Hq][D]
  bf16* out;           // [n_seqs][kq][Hq][D]
  float* part;         // [n_seqs][kq * Hq][max_splits][kPartHead + D]: m, l, -, -, acc[D]
  int Hq, g, pps, max_splits;
  int kq;              // query tokens per sequence (1: decode; > 1: verify)
  int n_chunks;        // workgroups per (sequence, kv head, split): query rows / R
  float scale_log2;
};

// out[s, h] = sum over the sequence's splits, weighted by exp2(m_split - M),
// for launches of more than 8 splits per sequence (fewer are merged inside
// the decode kernel). Every split of the decode grid writes its partial (one
// with no pages of its sequence: m = -inf, l = 0, O = 0, which weighs
// nothing), so the merge reads all max_splits of them without looking up the
// sequence's length.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecArgs a) {
  const int sh = blockIdx.x;          // (s * kq + t) * Hq + h
  const int lane = threadIdx.x;
  constexpr int PS = kPartHead + D;   // floats per partial
  constexpr int NE = D / 64;
  const float* pp = a.part + (size_t)sh * a.max_splits * PS;
  const int ns = a.max_splits;
  float o[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) o[e] = 0.f;
  float lt = 0.f;
  float mx = -INFINITY;
  for (int t = 0; t < ns; ++t) mx = fmaxf(mx, pp[t * PS]);
  const float mu = (mx == -INFINITY) ? 0.f : mx;
  for (int t = 0; t < ns; ++t) {
    const float w = exp2f(pp[t * PS] - mu);
    lt += w * pp[t * PS + 1];
#pragma unroll
    for (int e = 0; e < NE; ++e) o[e] += w * pp[t * PS + kPartHead + lane + 64 * e];
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
  for (int e = 0; e < NE; ++e) a.out[(size_t)sh * D + lane + 64 * e] = (bf16)(o[e] * inv);
}

// ---- the decode / verify kernel --------------------------------------------
// Up to 32 query rows (tokens x q-heads of one kv head) are the columns of
// 32x32x16 bf16 MFMAs: over tiles of two pages (32 keys), S^T = K Q^T, an
// online softmax per row (the forward's, lazily rescaled), then
// O^T += V^T P^T with V^T taken by LDS transpose reads. One wave per split
// streams the split's tiles through its own LDS tile (19 KiB at D = 128)
// filled by direct global->LDS loads, a 16-row tile per page, so no barrier
// orders the page stream. With 188 registers or fewer (two waves per SIMD)
// a CU holds eight of these waves, and the splits of a step (kResidentWgs)
// stream at once: measured on the 64-sequence serving cache, HBM streams at
// full rate only while most of the step's splits are resident. A second
// tile in flight per wave, which needs twice the LDS and so halves the
// resident splits, was 13% slower; one-page tiles with two stages, or three
// waves per SIMD, were no faster.
// W = 0: one wave per workgroup and split, its partial written to a.part for
// decode_merge_kernel. W > 0 (a power of two, at least max_splits): W waves
// per workgroup, wave w streams split w; each wave then leaves its partial
// in its own LDS tile and, after one barrier, the waves merge the chunk's
// rows and write the output (a wave past max_splits has no pages and a
// partial that weighs nothing). The LDS per workgroup is W tiles, so a CU
// still holds eight waves for every W.
template <int D, bool MASKED, int W>
__global__ __launch_bounds__(64 * (W > 0 ? W : 1)) __attribute__((amdgpu_waves_per_eu(2)))
void decode_mma_kernel(DecArgs a) {
  using M = Mfma<bf16>;
  using TL = Tile<D>;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int PT = tile_elems<D, kPage>();   // bf16 elements of one page's LDS tile
  constexpr int CH = PT / 8;                    // its 16-byte chunk positions
  constexpr int NB = (CH + 63) / 64;            // 1 KiB copies per page tile
  constexpr int LASTL = CH - 64 * (NB - 1);     // lanes of the last, partial copy
  static_assert(2 * PT == tile_elems<D, 2 * kPage>(), "two page tiles form one 32-row tile");
  constexpr int NW = W > 0 ? W : 1;   // waves per workgroup
  constexpr int PS = kPartHead + D;   // floats of one row's split partial
  // per wave: [K, V][two page tiles]
  __shared__ __align__(16) bf16 tiles[NW][2][2 * PT];
  static_assert(32 * PS * sizeof(float) <= sizeof(tiles[0]), "a wave's partials fit its tile");

  const int lane = threadIdx.x & 63;
  const int wave = NW > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  bf16 (&tile)[2][2 * PT] = tiles[wave];

  const int nb = a.max_splits;
  const int lg = xcd_remap(blockIdx.x, gridDim.x);
  const int split = W > 0 ? wave : lg % nb;
  const int rest = W > 0 ? lg : lg / nb;   // (sequence, kv head, chunk)
  const int chunk_id = rest % a.n_chunks;
  const int kv = (rest / a.n_chunks) % a.c.Hkv;
  const int s = rest / (a.n_chunks * a.c.Hkv);
  const int len = a.c.seq_lens[s];
  const int n_rows = a.kq * a.g;
  const int len_c = min(len, a.c.max_pages * kPage);
  const int pages = (len_c + kPage - 1) / kPage;
  const int ns = min(nb, (pages + a.pps - 1) / a.pps);
  const int pb = split < ns ? (int)((long long)split * pages / ns) : pages;
  const int pe = split < ns ? (int)((long long)(split + 1) * pages / ns) : pages;
  const int row_begin = pb * kPage;
  const int row_end = min(len_c, pe * kPage);
  const int n_pg = pe - pb;
  const int32_t* bt = a.c.block_table + (size_t)s * a.c.max_pages + pb;

  // This lane's query row (column l32 of every MFMA): Q^T fragments, and the
  // rows it may see (a verify token t sees rows below len - kq + t + 1).
  const int my_row = chunk_id * 32 + l32;
  const bool row_ok = my_row < n_rows;
  bf16x8 qf[NKS];
  int hi_row = row_end;
  {
    const int r = min(my_row, n_rows - 1);
    const int tok = r / a.g;
    const bf16* qp = a.q + (((size_t)s * a.kq + tok) * a.Hq + kv * a.g + r % a.g) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16 + hl * 8);
      if (!row_ok) qf[ks] = bf16x8{};
    }
    if constexpr (MASKED) hi_row = min(hi_row, len - a.kq + tok + 1);
    if (!row_ok) hi_row = 0;
  }

  // Copy map of a page tile: lane l of copy k writes chunk position 64 k + l,
  // which holds (row, column chunk) of the page's 16 x D run; padding
  // positions re-read chunk 0 of their row.
  uint32_t src_off[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    int rr, cc;
    TL::locate(64 * k + lane, rr, cc);
    src_off[k] = (uint32_t)(rr * D + (cc < D / 8 ? cc : 0) * 8) * 2;
  }
  const bf16* kpool = reinterpret_cast<const bf16*>(a.c.k_pages);
  const bf16* vpool = reinterpret_cast<const bf16*>(a.c.v_pages);
  // Tile t of the split: pages 2t and 2t + 1 (ids outside the pool read as
  // zeros and are masked). Rows at or past row_end read as zeros too (the
  // buffer range ends there), so no stale or non-finite bytes enter the
  // products. Returns the tile's page-validity bits.
  const int n_tiles = (n_pg + 1) / 2;
  // The page ids of tile t (its two table entries, -1 past the split), as
  // loaded values: the ids of tile t + 1 are loaded while tile t's copies
  // are in flight, so the table read adds no latency of its own.
  auto ids_of = [&](int t, int (&ids)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) ids[h] = 2 * t + h < n_pg ? bt[2 * t + h] : -1;
  };
  auto issue = [&](int t, const int (&ids)[2]) {
    int okb = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = 2 * t + h;
      int page = __builtin_amdgcn_readfirstlane(ids[h]);
      if (page >= a.c.n_pages) page = -1;
      okb |= (page >= 0) << h;
      const int rows = page >= 0 ? min(kPage, max(0, row_end - (row_begin + i * kPage))) : 0;
      const size_t base = ((size_t)max(page, 0) * a.c.Hkv + kv) * kPage * D;
      const buf_rsrc rk = uniform_rsrc(kpool + base, (uint32_t)(rows * D * 2));
      const buf_rsrc rv = uniform_rsrc(vpool + base, (uint32_t)(rows * D * 2));
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        if (k < NB - 1 || lane < LASTL) {
          dma16_at(rk, src_off[k], tile[0], (uint32_t)(h * PT * 2 + k * 1024));
          dma16_at(rv, src_off[k], tile[1], (uint32_t)(h * PT * 2 + k * 1024));
        }
      }
    }
    return okb;
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m_ref = -INFINITY;   // log2-domain reference max of this lane's row
  float l_run = 0.f;
  const float c = a.scale_log2;

  auto compute = [&](int t, int okb) {
    const uint32_t kst = lds_addr(tile[0]);
    const uint32_t vst = lds_addr(tile[1]);
    // S^T = K Q^T: K row fragments (row l32, 8 elements at 16 ks + 8 hl)
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
    const uint32_t kb = kst + TL::off(l32, 8 * hl);
    // (in two halves of the k-steps, so that half the fragments are live)
    static_for<2>([&](auto H) {
      constexpr int h0 = decltype(H)::value * (NKS / 2);
      bf16x8 kf[NKS / 2];
      static_for<NKS / 2>([&](auto KS) {
        constexpr int ks = decltype(KS)::value;
        kf[ks] = __builtin_bit_cast(bf16x8, lds_read16<32 * (h0 + ks)>(kb));
      });
      lds_wait<0>();
#pragma unroll
      for (int ks = 0; ks < NKS / 2; ++ks) lds_tie(kf[ks]);
#pragma unroll
      for (int ks = 0; ks < NKS / 2; ++ks) sc = M::mma(kf[ks], qf[h0 + ks], sc);
    });
    // V^T fragments of the two 16-key steps, by transpose reads
    const uint32_t vb =
        vst + TL::off(4 * hl + ((lane & 15) >> 2), 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    bf16x8 va[2][NDB];
    static_for<2>([&](auto J) {
      constexpr int j = decltype(J)::value;
      static_for<NDB>([&](auto DB) {
        constexpr int db = decltype(DB)::value;
        constexpr int off = TL::rows(16 * j) + 2 * 32 * db;
        va[j][db] = cat8(lds_tr4<off>(vb), lds_tr4<off + TL::rows(8)>(vb));
      });
    });
    // keys lo <= k < hi of the tile are visible to this lane's row
    const int row0 = row_begin + 2 * kPage * t;
    const int lo = (okb & 1) ? 0 : kPage;
    const int hi = (okb & 2) ? min(32, hi_row - row0) : min(kPage, hi_row - row0);
    if (lo > 0 || hi < 32) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int k = d_row(r, hl);
        sc[r] = (k >= lo && k < hi) ? sc[r] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
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
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pv = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -m_use));
      sc[r] = pv;
      l_run += pv;
    }
    lds_wait<0>();
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int db = 0; db < NDB; ++db) lds_tie(va[j][db]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bf16x8 pf = pack_regs<bf16>(sc, j);
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] = M::mma(va[j][db], pf, acc[db]);
    }
  };

  // one tile at a time: the other resident workgroups' copies keep HBM busy
  // while this one computes
  int ids[2], nxt[2];
  ids_of(0, ids);
  for (int t = 0; t < n_tiles; ++t) {
    const int okb = issue(t, ids);
    ids_of(t + 1, nxt);
    CART_WAIT_VMCNT(0);
    compute(t, okb);
    ids[0] = nxt[0];
    ids[1] = nxt[1];
  }
  CART_WAIT_VMCNT(0);
  l_run = wave_sum_halves(l_run);

  // The split partial of this lane's row: m, l (lane half 0) and the
  // unnormalised O, whose d = 32 db + d_row(r, hl) elements the lane holds
  // in 4-element runs.
  if constexpr (W == 0) {
    if (!row_ok) return;
    const int tok = my_row / a.g;
    float* pp = a.part + ((((size_t)s * a.kq + tok) * a.Hq + kv * a.g + my_row % a.g) *
                              a.max_splits + split) * PS;
    if (hl == 0) { pp[0] = m_ref; pp[1] = l_run; }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        *reinterpret_cast<f32x4*>(pp + kPartHead + 32 * db + 8 * cc + 4 * hl) =
            f32x4{acc[db][4 * cc], acc[db][4 * cc + 1], acc[db][4 * cc + 2], acc[db][4 * cc + 3]};
  } else {
    // Into this wave's own tile, [32 rows][PS]: its copies have landed and
    // its reads have returned (the last tile's waits), and no other wave
    // touches it before the barrier.
    asm volatile("" ::: "memory");
    float* mine = reinterpret_cast<float*>(&tile[0][0]) + l32 * PS;
    if (hl == 0) { mine[0] = m_ref; mine[1] = l_run; }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        *reinterpret_cast<f32x4*>(mine + kPartHead + 32 * db + 8 * cc + 4 * hl) =
            f32x4{acc[db][4 * cc], acc[db][4 * cc + 1], acc[db][4 * cc + 2], acc[db][4 * cc + 3]};
    __syncthreads();
    // Row r of the chunk is merged by wave r % W, lane l holding elements
    // l + 64 e, as decode_merge_kernel merges a row (waves past max_splits
    // add exact zeros).
    constexpr int NE = D / 64;
    constexpr int TS = sizeof(tiles[0]) / sizeof(float);   // floats between waves' tiles
    const float* p0 = reinterpret_cast<const float*>(&tiles[0][0][0]);
    const int rows_here = min(32, n_rows - chunk_id * 32);
    for (int r = wave; r < rows_here; r += W) {
      float m[W], l[W], x[W][NE];
#pragma unroll
      for (int t = 0; t < W; ++t) {
        const float* q = p0 + t * TS + r * PS;
        m[t] = q[0];
        l[t] = q[1];
#pragma unroll
        for (int e = 0; e < NE; ++e) x[t][e] = q[kPartHead + lane + 64 * e];
      }
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < W; ++t) mx = fmaxf(mx, m[t]);
      const float mu = (mx == -INFINITY) ? 0.f : mx;
      float lt = 0.f, o[NE];
#pragma unroll
      for (int e = 0; e < NE; ++e) o[e] = 0.f;
#pragma unroll
      for (int t = 0; t < W; ++t) {
        const float w = exp2f(m[t] - mu);
        lt += w * l[t];
#pragma unroll
        for (int e = 0; e < NE; ++e) o[e] += w * x[t][e];
      }
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int row = chunk_id * 32 + r;
      const size_t sh = ((size_t)s * a.kq + row / a.g) * a.Hq + kv * a.g + row % a.g;
#pragma unroll
      for (int e = 0; e < NE; ++e) a.out[sh * D + lane + 64 * e] = (bf16)(o[e] * inv);
    }
  }
}

template <int D, bool MASKED, int W>
hipError_t launch_dec_mma(DecArgs a, const DecodePlan& pl, hipStream_t st) {
  if constexpr (W > 0) {
    CART_LAUNCH("decode", (decode_mma_kernel<D, MASKED, W>), (unsigned)pl.grid, 64 * W, 0, st, a);
    return hipGetLastError();
  } else {
    CART_LAUNCH("decode", (decode_mma_kernel<D, MASKED, 0>), (unsigned)pl.grid, 64, 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    CART_LAUNCH("decode_merge", (decode_merge_kernel<D>), a.c.n_seqs * a.kq * a.Hq, 64, 0, st, a);
    return hipGetLastError();
  }
}

template <int D, bool MASKED>
hipError_t launch_dec_w(DecArgs a, const DecodePlan& pl, hipStream_t st) {
  switch (pl.waves) {
    case 1: return launch_dec_mma<D, MASKED, 1>(a, pl, st);
    case 2: return launch_dec_mma<D, MASKED, 2>(a, pl, st);
    case 4: return launch_dec_mma<D, MASKED, 4>(a, pl, st);
    case 8: return launch_dec_mma<D, MASKED, 8>(a, pl, st);
    default: return launch_dec_mma<D, MASKED, 0>(a, pl, st);
  }
}

template <int D>
hipError_t launch_dec_d(DecArgs a, const DecodePlan& pl, hipStream_t st) {
  return a.kq == 1 ? launch_dec_w<D, false>(a, pl, st) : launch_dec_w<D, true>(a, pl, st);
}

}  // namespace

// Device memory of the allocation-free decode entry point: the split
// partials live in this file-scope array instead of a caller's workspace.
// Every GPU the library runs on holds one copy until the process ends; all
// calls on one GPU share it (the last call's partials stay in it).
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  // Host code must not pass `scratch` itself to a kernel (on the host it is
  // only a stand-in for the symbol); its device address is looked up once
  // per device, with that device current, and kept.
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_cache_append(const CacheDims& c, int seq, int start, const void* k,
                               const void* v, bool src_bf16, int n_rows, hipStream_t st) {
  const size_t total = (size_t)n_rows * c.Hkv * (c.D / 8);
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (src_bf16)
    CART_LAUNCH("cache_append", (cache_append_kernel<bf16>), blocks ? blocks : 1, 256, 0, st, c,
                seq, start, reinterpret_cast<const bf16*>(k), reinterpret_cast<const bf16*>(v),
                n_rows);
  else
    CART_LAUNCH("cache_append", (cache_append_kernel<float>), blocks ? blocks : 1, 256, 0, st, c,
                seq, start, reinterpret_cast<const float*>(k), reinterpret_cast<const float*>(v),
                n_rows);
  return hipGetLastError();
}

hipError_t launch_cache_set_len(const CacheDims& c, int seq, int len, hipStream_t st) {
  cache_set_len_kernel<<<1, 64, 0, st>>>(c.seq_lens, seq, len);
  return hipGetLastError();
}

// Pages per split: about as many (sequence, kv head, split) waves as the
// GPU holds at once when every sequence is full (256 CUs x 8 waves; fewer
// splits leave CUs short of streams, more run in a second round: 6 or 8
// splits per sequence instead of 4 measured 11% and 3% slower on the
// 64-sequence serving cache), between 8 and kMaxPps pages.
constexpr long long kResidentWgs = 256 * 8;
// Most splits per sequence merged on chip (eight waves' LDS tiles fill a CU).
constexpr int kOnChipSplits = 8;

DecodePlan plan_decode(const CacheDims& c, int Hq, int kq) {
  DecodePlan pl{};
  const long long work = (long long)c.n_seqs * c.Hkv * c.max_pages;
  long long pps = (work + kResidentWgs - 1) / kResidentWgs;
  if (pps < 8) pps = 8;
  if (pps > kMaxPps) pps = kMaxPps;
  pps = (pps + 3) / 4 * 4;
  pl.pages_per_split = (int)pps;
  pl.max_splits = (int)((c.max_pages + pps - 1) / pps);
  pl.chunks = (Hq / c.Hkv * kq + 31) / 32;
  const long long wgs = (long long)c.n_seqs * c.Hkv * pl.chunks;
  if (pl.max_splits <= kOnChipSplits) {
    // splits merged on chip: one wave per split, the next power of two
    pl.waves = 1;
    while (pl.waves < pl.max_splits) pl.waves *= 2;
    pl.grid = wgs;
    pl.part_bytes = 0;
  } else {
    pl.waves = 0;
    pl.grid = wgs * pl.max_splits;
    pl.part_bytes = (size_t)c.n_seqs * kq * Hq * pl.max_splits * (kPartHead + c.D) * sizeof(float);
  }
  return pl;
}

hipError_t launch_decode(const CacheDims& c, int Hq, int kq, float scale, const void* q,
                         const void* k_new, const void* v_new, void* out, void* ws,
                         hipStream_t st) {
  if (k_new) {
    CART_LAUNCH("decode_append", (decode_append_kernel), c.n_seqs, 256, 0, st, c,
                reinterpret_cast<const bf16*>(k_new), reinterpret_cast<const bf16*>(v_new), kq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const DecodePlan pl = plan_decode(c, Hq, kq);
  DecArgs a{};
  a.c = c;
  a.q = reinterpret_cast<const bf16*>(q);
  a.out = reinterpret_cast<bf16*>(out);
  a.part = reinterpret_cast<float*>(ws);
  a.Hq = Hq;
  a.g = Hq / c.Hkv;
  a.pps = pl.pages_per_split;
  a.max_splits = pl.max_splits;
  a.kq = kq;
  a.n_chunks = pl.chunks;
  a.scale_log2 = scale * kLog2e;
  return c.D == 128 ? launch_dec_d<128>(a, pl, st) : launch_dec_d<64>(a, pl, st);
}

}  // namespace cartattn
