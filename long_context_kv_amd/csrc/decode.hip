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
  float* part;         // [n_seqs][kq * Hq][max_splits][D + 2]: m, l, acc[D]
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
                          split) * (D + 2);
    if (dd == 0) { pp[0] = mx; pp[1] = lt; }
    pp[2 + dd] = at;
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
  const float* pp = a.part + (size_t)sh * a.max_splits * (D + 2);
  float mx = -INFINITY;
  for (int t = 0; t < ns; ++t) mx = fmaxf(mx, pp[t * (D + 2)]);
  const float mu = (mx == -INFINITY) ? 0.f : mx;
  float lt = 0.f;
  float o[D / 64];
#pragma unroll
  for (int e = 0; e < D / 64; ++e) o[e] = 0.f;
  for (int t = 0; t < ns; ++t) {
    const float w = exp2f(pp[t * (D + 2)] - mu);
    lt += w * pp[t * (D + 2) + 1];
#pragma unroll
    for (int e = 0; e < D / 64; ++e) o[e] += w * pp[t * (D + 2) + 2 + lane + 64 * e];
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) a.out[(size_t)sh * D + lane + 64 * e] = (bf16)(o[e] * inv);
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
  pl.part_bytes = (size_t)c.n_seqs * kq * Hq * pl.max_splits * (c.D + 2) * sizeof(float);
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
