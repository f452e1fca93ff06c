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
// Decode is HBM-bound (4 flop per byte of K/V), so it uses no MFMA: one
// workgroup per (sequence, kv head, split of the pages); a sequence's pages
// are cut into ns = ceil(pages / pages-per-split) nearly equal splits, so
// the workgroups of a step run about equally long. The q-heads of the
// GQA group share every K/V byte read. Each thread owns one 8-element chunk
// of one row per pass and keeps a private online-softmax state per q-head;
// the states are merged with cross-lane shuffles and through LDS at the end,
// and a second kernel merges the splits of a sequence by log-sum-exp.
#include <math.h>

#include <mutex>

#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace cartattn {

namespace {

constexpr int kPage = 16;
constexpr int kDecThreads = 256;
constexpr int kUnroll = 4;   // passes per group of loads
constexpr int kMaxPps = 256; // pages per split at most (a launch plan bound)
constexpr int kPartHead = 4; // floats before a split partial's accumulator (m, l, 2 unused)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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

// R query rows per workgroup: rows c R .. c R + R - 1 (chunk c) of the
// (token, q-head) rows r = t g + j that read kv head kv; token t of a verify
// step sees the stored rows below len - kq + t + 1 (MASKED; a plain decode
// step sees every stored row).
template <int D, int G, bool MASKED>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecArgs a) {
  constexpr int CPR = D / 8;                 // chunks per row
  constexpr int RPP = kDecThreads / CPR;     // rows per pass
  constexpr int GPW = 64 / CPR;              // row groups per wave
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int chunk = tid % CPR;
  const int rsub = tid / CPR;

  const int nb = a.max_splits;
  const int lg = xcd_remap(blockIdx.x, gridDim.x);
  const int split = lg % nb;
  const int chunk_id = (lg / nb) % a.n_chunks;
  const int kv = (lg / (nb * a.n_chunks)) % a.c.Hkv;
  const int s = lg / (nb * a.n_chunks * a.c.Hkv);
  const int len = a.c.seq_lens[s];
  const int n_rows = a.kq * a.g;   // query rows of this (sequence, kv head)
  // the sequence's pages in ns nearly equal splits (ns as the merge counts them)
  const int len_c = min(len, a.c.max_pages * kPage);
  const int pages = (len_c + kPage - 1) / kPage;
  const int ns = min(nb, (pages + a.pps - 1) / a.pps);
  const int pb = split < ns ? (int)((long long)split * pages / ns) : pages;
  const int pe = split < ns ? (int)((long long)(split + 1) * pages / ns) : pages;
  const int row_begin = pb * kPage;
  const int row_end = min(len_c, pe * kPage);

  // q chunks stay bf16: scores are bf16 x bf16 dot products accumulated in
  // f32 (v_dot2), scaled afterwards.
  bf16x8 qb[G];
  int lim[G];   // rows below lim[j] are visible to query row j
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int r = min(chunk_id * G + j, n_rows - 1);
    const int tok = r / a.g;
    qb[j] = *reinterpret_cast<const bf16x8*>(
        a.q + (((size_t)s * a.kq + tok) * a.Hq + kv * a.g + r % a.g) * D + chunk * 8);
    lim[j] = chunk_id * G + j < n_rows ? len - a.kq + tok + 1 : 0;
  }
  const float c = a.scale_log2;
  // Online softmax per q-head with a lazily moved reference max m (log2
  // domain): probabilities are exp2(score - m) <= 2^8, and acc, l are
  // rescaled only when some score exceeds m by more than 8.
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }

  // Physical pages of this split, validated once, into LDS: the K/V loads
  // then depend on no other global load.
  __shared__ int pg[kMaxPps];
  const int n_pg = row_end > row_begin ? (row_end - row_begin + kPage - 1) / kPage : 0;
  {
    const int32_t* bt = a.c.block_table + (size_t)s * a.c.max_pages + row_begin / kPage;
    for (int i = tid; i < n_pg; i += kDecThreads) {
      const int p = bt[i];
      pg[i] = (p >= 0 && p < a.c.n_pages) ? p : -1;
    }
  }
  __syncthreads();

  // Rows are streamed kUnroll * RPP at a time; the raw 16-byte chunks of
  // the next group are loaded before the current group is used, so two
  // groups of loads are in flight per thread.
  const bf16* kp = reinterpret_cast<const bf16*>(a.c.k_pages);
  const bf16* vp = reinterpret_cast<const bf16*>(a.c.v_pages);
  struct Grp { uint4 k[kUnroll], v[kUnroll]; bool ok[kUnroll]; int row[kUnroll]; };
  // Loads are unconditional, so the wait counts stay exact: a row past the
  // split re-reads the split's last row (a cache hit) and a row on an invalid
  // page reads page 0; both are masked.
  auto load_grp = [&](int r0, Grp& x) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int row = r0 + u * RPP + rsub;
      const int rr = min(row, row_end - 1);
      const int page = pg[(rr - row_begin) / kPage];
      x.ok[u] = row < row_end && page >= 0;
      if constexpr (MASKED) x.row[u] = row;
      const size_t off = (((size_t)max(page, 0) * a.c.Hkv + kv) * kPage + rr % kPage) * D + chunk * 8;
      x.k[u] = *reinterpret_cast<const uint4*>(kp + off);
      x.v[u] = *reinterpret_cast<const uint4*>(vp + off);
    }
  };
  auto use_grp = [&](const Grp& x) {
    float p[G][kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bf16x8 kb = __builtin_bit_cast(bf16x8, x.k[u]);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 qa = {qb[j][2 * e], qb[j][2 * e + 1]};
          const bf16x2 ka = {kb[2 * e], kb[2 * e + 1]};
          d = __builtin_amdgcn_fdot2_f32_bf16(qa, ka, d, false);
        }
        d = row_sum<CPR>(d);
        bool ok = x.ok[u];
        if constexpr (MASKED) ok = ok && x.row[u] < lim[j];
        p[j][u] = ok ? d * c : -INFINITY;
      }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float mx = p[j][0];
#pragma unroll
      for (int u = 1; u < kUnroll; ++u) mx = fmaxf(mx, p[j][u]);
      if (mx > m[j] + 8.f) {   // per lane; taken rarely after the first rows
        const float alpha = (m[j] == -INFINITY) ? 0.f : exp2f(m[j] - mx);
        l[j] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] *= alpha;
        m[j] = mx;
      }
      const float mu = (m[j] == -INFINITY) ? 0.f : m[j];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        p[j][u] = __builtin_amdgcn_exp2f(p[j][u] - mu);
        l[j] += p[j][u];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bf16x8 vb = __builtin_bit_cast(bf16x8, x.v[u]);
      float vx[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) vx[e] = (float)vb[e];
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(p[j][u], vx[e], acc[j][e]);
    }
  };
  constexpr int STEP = kUnroll * RPP;
  if (row_begin < row_end) {
    // ping-pong between two register groups: the loads of the next group are
    // in flight while the current one is used
    Grp ga, gb;
    load_grp(row_begin, ga);
    for (int r0 = row_begin;;) {
      load_grp(r0 + STEP, gb);
      use_grp(ga);
      if ((r0 += STEP) >= row_end) break;
      load_grp(r0 + STEP, ga);
      use_grp(gb);
      if ((r0 += STEP) >= row_end) break;
    }
  }

  // Merge the row groups of a wave (lanes with the same chunk).
#pragma unroll
  for (int off = CPR; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float mo = __shfl_xor(m[j], off);
      const float lo = __shfl_xor(l[j], off);
      const float mn = fmaxf(m[j], mo);
      const float mu = (mn == -INFINITY) ? 0.f : mn;
      const float wa = exp2f(m[j] - mu);
      const float wb = exp2f(mo - mu);
      l[j] = l[j] * wa + lo * wb;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] = acc[j][e] * wa + __shfl_xor(acc[j][e], off) * wb;
      m[j] = mn;
    }
  }
  (void)GPW;
  // Merge the 4 waves through LDS.
  __shared__ __align__(16) float sm[4][G];
  __shared__ __align__(16) float sl[4][G];
  __shared__ __align__(16) float sacc[4][G][D];
  if (lane < CPR) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (lane == 0) { sm[wave][j] = m[j]; sl[wave][j] = l[j]; }
#pragma unroll
      for (int e = 0; e < 8; ++e) sacc[wave][j][chunk * 8 + e] = acc[j][e];
    }
  }
  __syncthreads();
  // Every thread finishes (head j, element d) pairs.
  for (int t = tid; t < G * D; t += kDecThreads) {
    const int j = t / D;
    const int dd = t % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, sm[w][j]);
    const float mu = (mx == -INFINITY) ? 0.f : mx;
    float lt = 0.f, at = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = exp2f(sm[w][j] - mu);
      lt += sl[w][j] * wt;
      at += sacc[w][j][dd] * wt;
    }
    const int r = chunk_id * G + j;
    if (r >= n_rows) continue;
    const int tok = r / a.g;
    float* pp = a.part + ((((size_t)s * a.kq + tok) * a.Hq + kv * a.g + r % a.g) * a.max_splits +
                          split) * (kPartHead + D);
    if (dd == 0) { pp[0] = mx; pp[1] = lt; }
    pp[kPartHead + dd] = at;
  }
}

// out[s, h] = sum over the sequence's splits, weighted by exp2(m_split - M).
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecArgs a) {
  const int sh = blockIdx.x;          // (s * kq + t) * Hq + h
  const int s = sh / (a.Hq * a.kq);
  const int lane = threadIdx.x;
  const int len = min(a.c.seq_lens[s], a.c.max_pages * kPage);
  const int pages = (len + kPage - 1) / kPage;
  const int ns = min(a.max_splits, (pages + a.pps - 1) / a.pps);
  constexpr int PS = kPartHead + D;   // floats per partial
  const float* pp = a.part + (size_t)sh * a.max_splits * PS;
  float mx = -INFINITY;
  for (int t = 0; t < ns; ++t) mx = fmaxf(mx, pp[t * PS]);
  const float mu = (mx == -INFINITY) ? 0.f : mx;
  float lt = 0.f;
  float o[D / 64];
#pragma unroll
  for (int e = 0; e < D / 64; ++e) o[e] = 0.f;
  for (int t = 0; t < ns; ++t) {
    const float w = exp2f(pp[t * PS] - mu);
    lt += w * pp[t * PS + 1];
#pragma unroll
    for (int e = 0; e < D / 64; ++e) o[e] += w * pp[t * PS + kPartHead + lane + 64 * e];
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) a.out[(size_t)sh * D + lane + 64 * e] = (bf16)(o[e] * inv);
}

// ---- MFMA decode / verify -------------------------------------------------
// A verify step has kq * g query rows per (sequence, kv head); the VALU
// kernel above takes at most 8 of them per workgroup and so reads every K/V
// byte once per 8 rows. This kernel takes up to 32 rows as the columns of
// 32x32x16 bf16 MFMAs, so a K/V byte is read once for all of them: over
// tiles of two pages (32 keys), S^T = K Q^T, an online softmax per row (the
// forward's, lazily rescaled), then O^T += V^T P^T with V^T taken by LDS
// transpose reads. Each wave streams its own tiles (the waves of a
// workgroup take alternate tiles of the split) through a private
// double-buffered LDS ring filled by direct global->LDS loads, one 16-row
// tile per page, so no barrier orders the page stream; the waves' states are
// merged through LDS at the end and written as one split partial.
constexpr int kMmaWaves = 1;

template <int D, bool MASKED>
__global__ __launch_bounds__(64 * kMmaWaves) void decode_mma_kernel(DecArgs a) {
  using M = Mfma<bf16>;
  using TL = Tile<D>;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int PT = tile_elems<D, kPage>();   // bf16 elements of one page's LDS tile
  constexpr int CH = PT / 8;                    // its 16-byte chunk positions
  constexpr int NB = (CH + 63) / 64;            // 1 KiB copies per page tile
  constexpr int LASTL = CH - 64 * (NB - 1);     // lanes of the last, partial copy
  constexpr int NDMA = 2 * 2 * NB;              // copies per tile (2 pages, K and V)
  static_assert(2 * PT == tile_elems<D, 2 * kPage>(), "two page tiles form one 32-row tile");
  // [wave][stage][K, V][two page tiles]
  __shared__ __align__(16) bf16 ring[kMmaWaves][2][2][2 * PT];
  __shared__ int pg[kMaxPps];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  const int nb = a.max_splits;
  const int lg = xcd_remap(blockIdx.x, gridDim.x);
  const int split = lg % nb;
  const int chunk_id = (lg / nb) % a.n_chunks;
  const int kv = (lg / (nb * a.n_chunks)) % a.c.Hkv;
  const int s = lg / (nb * a.n_chunks * a.c.Hkv);
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

  // the split's physical pages (-1: outside the pool, read as zeros, masked)
  for (int i = tid; i < n_pg; i += 64 * kMmaWaves) {
    const int pgid = a.c.block_table[(size_t)s * a.c.max_pages + pb + i];
    pg[i] = (pgid >= 0 && pgid < a.c.n_pages) ? pgid : -1;
  }
  __syncthreads();

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
  // Tile t of the split: pages 2t and 2t + 1. Rows at or past row_end read as
  // zeros (the buffer range ends there), so no stale or non-finite bytes
  // enter the products.
  const int n_tiles = (n_pg + 1) / 2;
  auto issue = [&](int t, int st) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = 2 * t + h;
      const int page = i < n_pg ? pg[i] : -1;
      const int rows = page >= 0 ? min(kPage, max(0, row_end - (row_begin + i * kPage))) : 0;
      const size_t base = ((size_t)max(page, 0) * a.c.Hkv + kv) * kPage * D;
      const buf_rsrc rk = make_rsrc(kpool + base, (uint32_t)(rows * D * 2));
      const buf_rsrc rv = make_rsrc(vpool + base, (uint32_t)(rows * D * 2));
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        if (k < NB - 1 || lane < LASTL) {
          dma16_at(rk, src_off[k], ring[wave][st][0], (uint32_t)(h * PT * 2 + k * 1024));
          dma16_at(rv, src_off[k], ring[wave][st][1], (uint32_t)(h * PT * 2 + k * 1024));
        }
      }
    }
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m_ref = -INFINITY;   // log2-domain reference max of this lane's row
  float l_run = 0.f;
  const float c = a.scale_log2;

  auto compute = [&](int t, int st) {
    const uint32_t kst = lds_addr(ring[wave][st][0]);
    const uint32_t vst = lds_addr(ring[wave][st][1]);
    // S^T = K Q^T: K row fragments (row l32, 8 elements at 16 ks + 8 hl)
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
    const uint32_t kb = kst + TL::off(l32, 8 * hl);
    bf16x8 kf[NKS];
    static_for<NKS>([&](auto KS) {
      constexpr int ks = decltype(KS)::value;
      kf[ks] = __builtin_bit_cast(bf16x8, lds_read16<32 * ks>(kb));
    });
    lds_wait<0>();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) lds_tie(kf[ks]);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) sc = M::mma(kf[ks], qf[ks], sc);
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
    const int row0 = row_begin + 32 * t;
    const bool ok0 = pg[2 * t] >= 0;
    const bool ok1 = 2 * t + 1 < n_pg && pg[2 * t + 1] >= 0;
    const int lo = ok0 ? 0 : kPage;
    const int hi = ok1 ? min(32, hi_row - row0) : min(kPage, hi_row - row0);
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

  // this wave's tiles: wave, wave + kMmaWaves, ... (two stages, static
  // addresses: the loop is unrolled by two)
  const int t0 = wave;
  if (t0 < n_tiles) issue(t0, 0);
  for (int t = t0; t < n_tiles; t += 2 * kMmaWaves) {
    if (t + kMmaWaves < n_tiles) {
      issue(t + kMmaWaves, 1);
      CART_WAIT_VMCNT(NDMA);
    } else {
      CART_WAIT_VMCNT(0);
    }
    compute(t, 0);
    const int t1 = t + kMmaWaves;
    if (t1 >= n_tiles) break;
    if (t1 + kMmaWaves < n_tiles) {
      issue(t1 + kMmaWaves, 0);
      CART_WAIT_VMCNT(NDMA);
    } else {
      CART_WAIT_VMCNT(0);
    }
    compute(t1, 1);
  }
  CART_WAIT_VMCNT(0);
  l_run = wave_sum_halves(l_run);

  // Merge the waves through LDS (the rings are free once every wave is here):
  // red[w][row][d] holds wave w's unnormalised O, sm/sl its row max and sum.
  __syncthreads();
  float* red = reinterpret_cast<float*>(&ring[0][0][0][0]);
  static_assert(sizeof(ring) >= (size_t)kMmaWaves * 32 * D * 4 + 2 * kMmaWaves * 32 * 4,
                "the merge fits the rings");
  float* sm = red + kMmaWaves * 32 * D;
  float* sl = sm + kMmaWaves * 32;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const f32x4 v = {acc[db][4 * cc], acc[db][4 * cc + 1], acc[db][4 * cc + 2],
                       acc[db][4 * cc + 3]};
      *reinterpret_cast<f32x4*>(red + ((size_t)wave * 32 + l32) * D + 32 * db + 8 * cc + 4 * hl) = v;
    }
  if (hl == 0) {
    sm[wave * 32 + l32] = m_ref;
    sl[wave * 32 + l32] = l_run;
  }
  __syncthreads();
  constexpr int PS = kPartHead + D;
  for (int e = tid; e < 32 * D; e += 64 * kMmaWaves) {
    const int r = e / D;
    const int dd = e % D;
    const int row = chunk_id * 32 + r;
    if (row >= n_rows) break;   // rows grow with e
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kMmaWaves; ++w) mx = fmaxf(mx, sm[w * 32 + r]);
    const float mu = (mx == -INFINITY) ? 0.f : mx;
    float lt = 0.f, at = 0.f;
#pragma unroll
    for (int w = 0; w < kMmaWaves; ++w) {
      const float wt = exp2f(sm[w * 32 + r] - mu);
      lt += sl[w * 32 + r] * wt;
      at += red[((size_t)w * 32 + r) * D + dd] * wt;
    }
    const int tok = row / a.g;
    float* pp = a.part +
                ((((size_t)s * a.kq + tok) * a.Hq + kv * a.g + row % a.g) * a.max_splits + split) * PS;
    if (dd == 0) { pp[0] = mx; pp[1] = lt; }
    pp[kPartHead + dd] = at;
  }
}

template <int D, bool MASKED>
hipError_t launch_dec_mma(DecArgs a, hipStream_t st) {
  a.n_chunks = (a.g * a.kq + 31) / 32;
  const int grid = a.c.n_seqs * a.c.Hkv * a.n_chunks * a.max_splits;
  CART_LAUNCH("decode", (decode_mma_kernel<D, MASKED>), grid, 64 * kMmaWaves, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  CART_LAUNCH("decode_merge", (decode_merge_kernel<D>), a.c.n_seqs * a.kq * a.Hq, 64, 0, st, a);
  return hipGetLastError();
}

template <int D, int G, bool MASKED>
hipError_t launch_dec_t(const DecArgs& a, hipStream_t st) {
  const int grid = a.c.n_seqs * a.c.Hkv * a.n_chunks * a.max_splits;
  CART_LAUNCH("decode", (decode_kernel<D, G, MASKED>), grid, kDecThreads, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  CART_LAUNCH("decode_merge", (decode_merge_kernel<D>), a.c.n_seqs * a.kq * a.Hq, 64, 0, st, a);
  return hipGetLastError();
}

// Rows per workgroup: the kv head's query rows (g per token, kq tokens), at
// most 8 (the per-row online-softmax state lives in registers).
inline int dec_rows(int g, int kq) {
  const int n = g * kq;
  return n >= 8 ? 8 : (n >= 4 ? 4 : (n >= 2 ? 2 : 1));
}

template <int D>
hipError_t launch_dec_d(DecArgs a, hipStream_t st) {
  // more than 4 query rows per kv head: the MFMA kernel, which reads K/V
  // once for up to 32 of them (measured: as fast as the VALU kernel at 4
  // rows, and half again as fast at 8, where the VALU kernel's per-row work
  // holds it back)
  if (a.g * a.kq > 4)
    return a.kq == 1 ? launch_dec_mma<D, false>(a, st) : launch_dec_mma<D, true>(a, st);
  const int R = dec_rows(a.g, a.kq);
  a.n_chunks = (a.g * a.kq + R - 1) / R;
  if (a.kq == 1) {
    switch (R) {
      case 1: return launch_dec_t<D, 1, false>(a, st);
      case 2: return launch_dec_t<D, 2, false>(a, st);
      case 4: return launch_dec_t<D, 4, false>(a, st);
      default: return launch_dec_t<D, 8, false>(a, st);
    }
  }
  switch (R) {
    case 2: return launch_dec_t<D, 2, true>(a, st);
    case 4: return launch_dec_t<D, 4, true>(a, st);
    default: return launch_dec_t<D, 8, true>(a, st);
  }
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

DecodePlan plan_decode(const CacheDims& c, int Hq, int kq) {
  DecodePlan pl{};
  const long long work = (long long)c.n_seqs * c.Hkv * c.max_pages;
  long long pps = (work + 2047) / 2048;
  if (pps < 8) pps = 8;
  if (pps > 256) pps = 256;
  pps = (pps + 3) / 4 * 4;
  pl.pages_per_split = (int)pps;
  pl.max_splits = (int)((c.max_pages + pps - 1) / pps);
  pl.part_bytes = (size_t)c.n_seqs * kq * Hq * pl.max_splits * (kPartHead + c.D) * sizeof(float);
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
  a.scale_log2 = scale * kLog2e;
  return c.D == 128 ? launch_dec_d<128>(a, st) : launch_dec_d<64>(a, st);
}

}  // namespace cartattn
