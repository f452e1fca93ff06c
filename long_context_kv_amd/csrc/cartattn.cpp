// libcartattn C ABI: argument checking, workspace sizing, the paged-cache
// handle and kernel launches. Every check runs on the host before any HIP
// call, so each error path can be exercised without a GPU.
#include "cartattn.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <new>
#include <vector>

#include "launch.hpp"

using namespace cartattn;

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

bool sync_each_call() {
  static const bool on = [] {
    const char* e = getenv("CARTATTN_SYNC");
    return e && e[0] && e[0] != '0';
  }();
  return on;
}

int hip_result(hipError_t e, hipStream_t st, const char* what) {
  if (e == hipSuccess && sync_each_call()) {
    e = hipStreamSynchronize(st);
    if (e == hipSuccess) e = hipGetLastError();
  }
  if (e != hipSuccess) return fail(CART_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  g_err[0] = '\0';
  return CART_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_dtype(int d) { return d == CART_F32 || d == CART_BF16; }
bool valid_head_dim(int d) { return d == 64 || d == 128; }
constexpr long long kMaxElems = (1LL << 31) - 1;   // element offsets stay in int range per tensor

int check_shape(const cart_attn_shape* s) {
  if (!s) return fail(CART_ERR_INVALID_ARG, "shape is NULL");
  if (s->batch < 1 || s->q_seq < 1)
    return fail(CART_ERR_INVALID_ARG, "batch (%d) and q_seq (%d) must be >= 1", s->batch, s->q_seq);
  if (s->p < 0) return fail(CART_ERR_INVALID_ARG, "p (%d) must be >= 0", s->p);
  if (s->frozen_rows < 0 || s->frozen_rows > s->p)
    return fail(CART_ERR_INVALID_ARG, "frozen_rows (%d) must lie in [0, p=%d]", s->frozen_rows, s->p);
  if (s->n_q_heads < 1 || s->n_kv_heads < 1)
    return fail(CART_ERR_INVALID_ARG, "head counts must be >= 1");
  if (s->n_q_heads % s->n_kv_heads != 0)
    return fail(CART_ERR_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                s->n_q_heads, s->n_kv_heads);
  if (!valid_head_dim(s->head_dim))
    return fail(CART_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", s->head_dim);
  if (!(s->scale >= 0.f) || isinf(s->scale))
    return fail(CART_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (!valid_dtype(s->tok_dtype) || !valid_dtype(s->row_dtype))
    return fail(CART_ERR_INVALID_ARG, "unknown dtype");
  if (s->tok_dtype == CART_F32 && s->row_dtype != CART_F32)
    return fail(CART_ERR_UNSUPPORTED, "f32 tokens need f32 cartridge rows");
  if (s->window < 0) return fail(CART_ERR_INVALID_ARG, "window (%d) must be >= 0", s->window);
  if (s->seg_lens) {
    if (s->batch > kMaxSegs)
      return fail(CART_ERR_UNSUPPORTED, "%d packed segments (at most %d)", s->batch, kMaxSegs);
    long long total = 0;
    for (int b = 0; b < s->batch; ++b) {
      if (s->seg_lens[b] < 1 || s->seg_lens[b] > s->q_seq)
        return fail(CART_ERR_INVALID_ARG, "segment %d has length %d (1..q_seq=%d)", b,
                    s->seg_lens[b], s->q_seq);
      total += s->seg_lens[b];
    }
    if (total * s->n_q_heads * s->head_dim > kMaxElems)
      return fail(CART_ERR_UNSUPPORTED, "packed tensor too large");
  }
  const long long qe = (long long)s->batch * s->q_seq * s->n_q_heads * s->head_dim;
  const long long ce = (long long)s->p * s->n_kv_heads * s->head_dim;
  if (qe > kMaxElems || ce > kMaxElems)
    return fail(CART_ERR_UNSUPPORTED, "tensor too large for 32-bit element counts");
  const long long grid = (long long)s->batch * s->q_seq * s->n_q_heads;
  if (grid > kMaxElems / 4) return fail(CART_ERR_UNSUPPORTED, "too many query rows");
  return CART_OK;
}

AttnDims dims_of(const cart_attn_shape* s) {
  AttnDims d{};
  d.B = s->batch; d.n = s->q_seq; d.p = s->p; d.f = s->frozen_rows;
  d.Hq = s->n_q_heads; d.Hkv = s->n_kv_heads; d.D = s->head_dim;
  d.scale = s->scale > 0.f ? s->scale : 1.0f / sqrtf((float)s->head_dim);
  d.tok_bf16 = s->tok_dtype == CART_BF16;
  d.row_bf16 = s->row_dtype == CART_BF16;
  // a window reaching every row is no window (one plan, one code path)
  d.window = (s->window > 0 && (long long)s->window < (long long)s->p + s->q_seq) ? s->window : 0;
  d.seg = Segs{};
  if (s->seg_lens) {
    d.seg.packed = s->batch;
    for (int b = 0; b < s->batch; ++b) d.seg.off[b + 1] = d.seg.off[b] + s->seg_lens[b];
  }
  return d;
}

int need_ptr(const void* p, const char* name) {
  if (!p) return fail(CART_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(CART_ERR_ALIGNMENT, "%s is not 16-byte aligned", name);
  return CART_OK;
}

int opt_ptr(const void* p, const char* name) {
  if (p && !aligned16(p)) return fail(CART_ERR_ALIGNMENT, "%s is not 16-byte aligned", name);
  return CART_OK;
}

int check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return CART_OK;
  if (!ws) return fail(CART_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if (have < need)
    return fail(CART_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  if (!aligned16(ws)) return fail(CART_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
  return CART_OK;
}

#define CHECK(expr)               \
  do {                            \
    const int _st = (expr);       \
    if (_st != CART_OK) return _st; \
  } while (0)

}  // namespace

struct cart_cache {
  cart_cache_desc d;
  std::vector<int32_t> lens;   // host mirror of seq_lens
};

namespace {

CacheDims cache_dims(const cart_cache* c) {
  CacheDims cd{};
  cd.n_seqs = c->d.n_seqs; cd.Hkv = c->d.n_kv_heads; cd.D = c->d.head_dim;
  cd.page = c->d.page_size; cd.max_pages = c->d.max_pages_per_seq; cd.n_pages = c->d.n_pages;
  cd.k_pages = c->d.k_pages; cd.v_pages = c->d.v_pages;
  cd.block_table = c->d.block_table; cd.seq_lens = c->d.seq_lens;
  return cd;
}

long long capacity(const cart_cache* c) {
  return (long long)c->d.max_pages_per_seq * c->d.page_size;
}

int check_seq(const cart_cache* c, int32_t seq) {
  if (!c) return fail(CART_ERR_INVALID_ARG, "cache handle is NULL");
  if (seq < 0 || seq >= c->d.n_seqs)
    return fail(CART_ERR_INVALID_ARG, "seq %d outside [0, %d)", seq, c->d.n_seqs);
  return CART_OK;
}

int check_rows(const cart_cache* c, int32_t seq, const void* k, const void* v, cart_dtype src,
               int32_t n_rows, int32_t n_kv_heads, int32_t head_dim) {
  CHECK(check_seq(c, seq));
  if (n_kv_heads != c->d.n_kv_heads || head_dim != c->d.head_dim)
    return fail(CART_ERR_GEOMETRY, "rows have %d kv heads x %d, the cache %d x %d", n_kv_heads,
                head_dim, c->d.n_kv_heads, c->d.head_dim);
  if (!valid_dtype(src)) return fail(CART_ERR_INVALID_ARG, "unknown source dtype");
  if (n_rows < 0) return fail(CART_ERR_INVALID_ARG, "row count %d < 0", n_rows);
  if ((long long)c->lens[seq] + n_rows > capacity(c))
    return fail(CART_ERR_CACHE_FULL, "seq %d: %d + %d rows exceed capacity %lld", seq,
                c->lens[seq], n_rows, capacity(c));
  if (n_rows > 0) {
    CHECK(need_ptr(k, "k"));
    CHECK(need_ptr(v, "v"));
  }
  return CART_OK;
}

}  // namespace

namespace {

// Validate a parts description and fill the kernels' table. need_ptrs: the
// parts' row pointers must be given (16-byte aligned) for parts with rows.
int parts_table(const cart_parts* parts, bool need_ptrs, PartTable* t) {
  if (!parts) return fail(CART_ERR_INVALID_ARG, "parts is NULL");
  if (parts->n_parts < 1 || parts->n_parts > kMaxParts)
    return fail(CART_ERR_INVALID_ARG, "n_parts (%d) must lie in [1, %d]", parts->n_parts,
                kMaxParts);
  if (!parts->rows || !parts->frozen)
    return fail(CART_ERR_INVALID_ARG, "parts->rows and parts->frozen must be given");
  if (need_ptrs && (!parts->k || !parts->v))
    return fail(CART_ERR_INVALID_ARG, "parts->k and parts->v must be given");
  *t = PartTable{};
  t->n = parts->n_parts;
  long long off = 0;
  for (int i = 0; i < t->n; ++i) {
    const int r = parts->rows[i], f = parts->frozen[i];
    if (r < 0) return fail(CART_ERR_INVALID_ARG, "part %d has %d rows", i, r);
    if (f < 0 || f > r)
      return fail(CART_ERR_INVALID_ARG, "part %d: frozen rows %d outside [0, %d]", i, f, r);
    t->rows[i] = r;
    t->frozen[i] = f;
    t->off[i] = (int)off;
    off += r;
    if (off > 0x7fffffffLL) return fail(CART_ERR_UNSUPPORTED, "composed prefix too long");
    if (need_ptrs) {
      if (r > 0) {
        char name[32];
        snprintf(name, sizeof(name), "parts->k[%d]", i);
        CHECK(need_ptr(parts->k[i], name));
        snprintf(name, sizeof(name), "parts->v[%d]", i);
        CHECK(need_ptr(parts->v[i], name));
      }
      t->k[i] = parts->k[i];
      t->v[i] = parts->v[i];
    }
  }
  t->off[t->n] = (int)off;
  return CART_OK;
}

}  // namespace

extern "C" {

const char* cart_status_string(int status) {
  switch (status) {
    case CART_OK: return "ok";
    case CART_ERR_INVALID_ARG: return "invalid argument";
    case CART_ERR_UNSUPPORTED: return "unsupported";
    case CART_ERR_ALIGNMENT: return "misaligned pointer";
    case CART_ERR_WORKSPACE: return "workspace missing or too small";
    case CART_ERR_CACHE_NOT_EMPTY: return "cache sequence not empty";
    case CART_ERR_CACHE_FULL: return "cache sequence full";
    case CART_ERR_GEOMETRY: return "geometry mismatch";
    case CART_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* cart_last_error(void) { return g_err; }

int cart_rope_tokens(void* q, void* k, cart_dtype dt, int32_t batch, int32_t seq,
                     int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t pos_base,
                     const int32_t* pos_offsets, double theta, int32_t inverse, void* stream) {
  if (!valid_dtype(dt)) return fail(CART_ERR_INVALID_ARG, "unknown dtype");
  if (batch < 0 || seq < 0) return fail(CART_ERR_INVALID_ARG, "batch and seq must be >= 0");
  if (n_q_heads < 1) return fail(CART_ERR_INVALID_ARG, "n_q_heads must be >= 1");
  if (k && n_kv_heads < 1) return fail(CART_ERR_INVALID_ARG, "n_kv_heads must be >= 1");
  if (!valid_head_dim(head_dim))
    return fail(CART_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", head_dim);
  if (!(theta > 0.0) || isinf(theta)) return fail(CART_ERR_INVALID_ARG, "theta must be > 0");
  if (pos_base < 0) return fail(CART_ERR_INVALID_ARG, "pos_base must be >= 0");
  const long long rows = (long long)batch * seq;
  if (rows * (n_q_heads + (k ? n_kv_heads : 0)) * head_dim > kMaxElems || rows > 0x7fffffffLL)
    return fail(CART_ERR_UNSUPPORTED, "tensor too large");
  if (rows == 0) { g_err[0] = '\0'; return CART_OK; }
  CHECK(need_ptr(q, "q"));
  CHECK(opt_ptr(k, "k"));
  if (pos_offsets && (reinterpret_cast<uintptr_t>(pos_offsets) & 3u))
    return fail(CART_ERR_ALIGNMENT, "pos_offsets is not 4-byte aligned");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return hip_result(launch_rope(q, k, dt == CART_BF16, batch, seq, n_q_heads, k ? n_kv_heads : 0,
                                head_dim, pos_base, pos_offsets, theta, inverse != 0, nullptr, st),
                    st, "cart_rope_tokens");
}

int cart_rope_tokens_packed(void* q, void* k, cart_dtype dt, int32_t n_segs,
                            const int32_t* seg_lens, int32_t n_q_heads, int32_t n_kv_heads,
                            int32_t head_dim, int32_t pos_base, double theta, int32_t inverse,
                            void* stream) {
  if (n_segs < 1 || n_segs > kMaxSegs)
    return fail(CART_ERR_INVALID_ARG, "n_segs (%d) must lie in [1, %d]", n_segs, kMaxSegs);
  if (!seg_lens) return fail(CART_ERR_INVALID_ARG, "seg_lens is NULL");
  Segs sg{};
  sg.packed = n_segs;
  for (int b = 0; b < n_segs; ++b) {
    if (seg_lens[b] < 1) return fail(CART_ERR_INVALID_ARG, "segment %d has length %d", b, seg_lens[b]);
    if ((long long)sg.off[b] + seg_lens[b] > 0x7fffffffLL)
      return fail(CART_ERR_UNSUPPORTED, "too many packed rows");
    sg.off[b + 1] = sg.off[b] + seg_lens[b];
  }
  const int T = sg.off[n_segs];
  // the remaining checks are cart_rope_tokens' for one sequence of T rows
  if (!valid_dtype(dt)) return fail(CART_ERR_INVALID_ARG, "unknown dtype");
  if (n_q_heads < 1) return fail(CART_ERR_INVALID_ARG, "n_q_heads must be >= 1");
  if (k && n_kv_heads < 1) return fail(CART_ERR_INVALID_ARG, "n_kv_heads must be >= 1");
  if (!valid_head_dim(head_dim))
    return fail(CART_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", head_dim);
  if (!(theta > 0.0) || isinf(theta)) return fail(CART_ERR_INVALID_ARG, "theta must be > 0");
  if (pos_base < 0) return fail(CART_ERR_INVALID_ARG, "pos_base must be >= 0");
  if ((long long)T * (n_q_heads + (k ? n_kv_heads : 0)) * head_dim > kMaxElems)
    return fail(CART_ERR_UNSUPPORTED, "tensor too large");
  CHECK(need_ptr(q, "q"));
  CHECK(opt_ptr(k, "k"));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return hip_result(launch_rope(q, k, dt == CART_BF16, 1, T, n_q_heads, k ? n_kv_heads : 0,
                                head_dim, pos_base, nullptr, theta, inverse != 0, &sg, st),
                    st, "cart_rope_tokens_packed");
}

namespace {

int check_norm_rope(cart_dtype dt, int32_t batch, int32_t seq, int32_t n_q_heads,
                    int32_t n_kv_heads, int32_t head_dim, float eps, int32_t pos_base,
                    const int32_t* pos_offsets, double theta, const void* k, const float* w_k) {
  if (!valid_dtype(dt)) return fail(CART_ERR_INVALID_ARG, "unknown dtype");
  if (batch < 0 || seq < 0) return fail(CART_ERR_INVALID_ARG, "batch and seq must be >= 0");
  if (n_q_heads < 1) return fail(CART_ERR_INVALID_ARG, "n_q_heads must be >= 1");
  if (k && n_kv_heads < 1) return fail(CART_ERR_INVALID_ARG, "n_kv_heads must be >= 1");
  if (!valid_head_dim(head_dim))
    return fail(CART_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", head_dim);
  if (!(eps > 0.f) || isinf(eps)) return fail(CART_ERR_INVALID_ARG, "eps must be > 0");
  if (!(theta > 0.0) || isinf(theta)) return fail(CART_ERR_INVALID_ARG, "theta must be > 0");
  if (pos_base < 0) return fail(CART_ERR_INVALID_ARG, "pos_base must be >= 0");
  const long long rows = (long long)batch * seq;
  if (rows * (n_q_heads + (k ? n_kv_heads : 0)) * head_dim > kMaxElems || rows > 0x7fffffffLL)
    return fail(CART_ERR_UNSUPPORTED, "tensor too large");
  if (k && !w_k) return fail(CART_ERR_INVALID_ARG, "w_k is NULL but k is given");
  if (pos_offsets && (reinterpret_cast<uintptr_t>(pos_offsets) & 3u))
    return fail(CART_ERR_ALIGNMENT, "pos_offsets is not 4-byte aligned");
  return CART_OK;
}

}  // namespace

int cart_qk_norm_rope(const void* q_in, const void* k_in, void* q_out, void* k_out,
                      const float* w_q, const float* w_k, cart_dtype dt, int32_t batch,
                      int32_t seq, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                      float eps, int32_t pos_base, const int32_t* pos_offsets, double theta,
                      void* stream) {
  CHECK(check_norm_rope(dt, batch, seq, n_q_heads, n_kv_heads, head_dim, eps, pos_base,
                        pos_offsets, theta, k_in, w_k));
  if ((long long)batch * seq == 0) { g_err[0] = '\0'; return CART_OK; }
  CHECK(need_ptr(q_in, "q_in"));
  CHECK(need_ptr(q_out, "q_out"));
  CHECK(need_ptr(w_q, "w_q"));
  if (k_in) {
    CHECK(need_ptr(k_in, "k_in"));
    CHECK(need_ptr(k_out, "k_out"));
    CHECK(need_ptr(w_k, "w_k"));
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return hip_result(launch_qk_norm_rope(q_in, k_in, nullptr, nullptr, q_out, k_in ? k_out : nullptr,
                                        w_q, w_k, dt == CART_BF16, batch, seq, n_q_heads,
                                        k_in ? n_kv_heads : 0, head_dim, eps, pos_base,
                                        pos_offsets, theta, false, st),
                    st, "cart_qk_norm_rope");
}

int cart_qk_norm_rope_bwd(const void* q_in, const void* k_in, const void* dq_out,
                          const void* dk_out, void* dq_in, void* dk_in, const float* w_q,
                          const float* w_k, cart_dtype dt, int32_t batch, int32_t seq,
                          int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float eps,
                          int32_t pos_base, const int32_t* pos_offsets, double theta,
                          void* stream) {
  CHECK(check_norm_rope(dt, batch, seq, n_q_heads, n_kv_heads, head_dim, eps, pos_base,
                        pos_offsets, theta, k_in, w_k));
  if ((long long)batch * seq == 0) { g_err[0] = '\0'; return CART_OK; }
  CHECK(need_ptr(q_in, "q_in"));
  CHECK(need_ptr(dq_out, "dq_out"));
  CHECK(need_ptr(dq_in, "dq_in"));
  CHECK(need_ptr(w_q, "w_q"));
  if (k_in) {
    CHECK(need_ptr(k_in, "k_in"));
    CHECK(need_ptr(dk_out, "dk_out"));
    CHECK(need_ptr(dk_in, "dk_in"));
    CHECK(need_ptr(w_k, "w_k"));
  }
  if (dq_in == q_in || (k_in && dk_in == k_in))
    return fail(CART_ERR_INVALID_ARG, "the input gradient may not overwrite the inputs");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return hip_result(launch_qk_norm_rope(q_in, k_in, dq_out, k_in ? dk_out : nullptr, dq_in,
                                        k_in ? dk_in : nullptr, w_q, w_k, dt == CART_BF16, batch,
                                        seq, n_q_heads, k_in ? n_kv_heads : 0, head_dim, eps,
                                        pos_base, pos_offsets, theta, true, st),
                    st, "cart_qk_norm_rope_bwd");
}

int cart_adam_rows(float* rows, const float* grad, float* m, float* v, void* rows_bf16,
                   int64_t n_rows, int32_t row_elems, int32_t frozen_rows, int32_t step,
                   double lr, double beta1, double beta2, double eps, void* stream) {
  if (n_rows < 0 || row_elems < 1)
    return fail(CART_ERR_INVALID_ARG, "n_rows must be >= 0 and row_elems >= 1");
  if (row_elems % 4 != 0)
    return fail(CART_ERR_UNSUPPORTED, "row_elems (%d) must be a multiple of 4", row_elems);
  if (frozen_rows < 0 || frozen_rows > n_rows)
    return fail(CART_ERR_INVALID_ARG, "frozen_rows (%d) must lie in [0, n_rows]", frozen_rows);
  if (step < 1) return fail(CART_ERR_INVALID_ARG, "step (%d) must be >= 1", step);
  if (!(lr >= 0.0) || isinf(lr)) return fail(CART_ERR_INVALID_ARG, "lr must be finite and >= 0");
  if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0))
    return fail(CART_ERR_INVALID_ARG, "betas must lie in [0, 1)");
  if (!(eps > 0.0) || isinf(eps)) return fail(CART_ERR_INVALID_ARG, "eps must be > 0");
  const long long n = (long long)n_rows * row_elems;
  if (n > (1LL << 40)) return fail(CART_ERR_UNSUPPORTED, "tensor too large");
  if (n == 0) { g_err[0] = '\0'; return CART_OK; }
  CHECK(need_ptr(rows, "rows"));
  CHECK(need_ptr(grad, "grad"));
  CHECK(need_ptr(m, "m"));
  CHECK(need_ptr(v, "v"));
  CHECK(opt_ptr(rows_bf16, "rows_bf16"));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return hip_result(launch_adam_rows(rows, grad, m, v, rows_bf16, (size_t)n,
                                     (size_t)frozen_rows * row_elems, step, lr, beta1, beta2,
                                     eps, st),
                    st, "cart_adam_rows");
}

int cart_rows_to_bf16(const float* k, const float* v, void* k_bf16, void* v_bf16,
                      int64_t n_rows, int32_t row_elems, void* stream) {
  if (n_rows < 0 || row_elems < 1)
    return fail(CART_ERR_INVALID_ARG, "n_rows must be >= 0 and row_elems >= 1");
  if (row_elems % 4 != 0)
    return fail(CART_ERR_UNSUPPORTED, "row_elems (%d) must be a multiple of 4", row_elems);
  const long long n = (long long)n_rows * row_elems;
  if (n > (1LL << 40)) return fail(CART_ERR_UNSUPPORTED, "tensor too large");
  if (n == 0) { g_err[0] = '\0'; return CART_OK; }
  CHECK(need_ptr(k, "k"));
  CHECK(need_ptr(v, "v"));
  CHECK(need_ptr(k_bf16, "k_bf16"));
  CHECK(need_ptr(v_bf16, "v_bf16"));
  const auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
  };
  const size_t fb = (size_t)n * 4, hb = (size_t)n * 2;
  if (overlap(k_bf16, hb, k, fb) || overlap(k_bf16, hb, v, fb) || overlap(v_bf16, hb, k, fb) ||
      overlap(v_bf16, hb, v, fb) || overlap(k_bf16, hb, v_bf16, hb))
    return fail(CART_ERR_INVALID_ARG, "cart_rows_to_bf16: outputs overlap the inputs or each other");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return hip_result(launch_rows_to_bf16(k, v, reinterpret_cast<__bf16*>(k_bf16),
                                        reinterpret_cast<__bf16*>(v_bf16), (size_t)n, st),
                    st, "cart_rows_to_bf16");
}

size_t cart_attn_workspace_size(const cart_attn_shape* s, int32_t for_backward) {
  if (check_shape(s) != CART_OK) return 0;
  const AttnDims d = dims_of(s);
  return for_backward ? bwd_workspace_bytes(d) : fwd_workspace_bytes(d);
}

int cart_attn_fwd(const cart_attn_shape* s, const void* q, const void* k_tok, const void* v_tok,
                  const void* k_cart, const void* v_cart, void* out, float* lse, void* workspace,
                  size_t workspace_bytes, void* stream) {
  CHECK(check_shape(s));
  CHECK(need_ptr(q, "q"));
  CHECK(need_ptr(k_tok, "k_tok"));
  CHECK(need_ptr(v_tok, "v_tok"));
  if (s->p > 0) {
    CHECK(need_ptr(k_cart, "k_cart"));
    CHECK(need_ptr(v_cart, "v_cart"));
  }
  CHECK(need_ptr(out, "out"));
  CHECK(need_ptr(lse, "lse"));
  const AttnDims d = dims_of(s);
  CHECK(check_workspace(workspace, workspace_bytes, fwd_workspace_bytes(d)));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return hip_result(launch_fwd(d, q, k_tok, v_tok, k_cart, v_cart, out, lse, workspace, st), st,
                    "cart_attn_fwd");
}

int cart_attn_bwd(const cart_attn_shape* s, const void* q, const void* k_tok, const void* v_tok,
                  const void* k_cart, const void* v_cart, const void* out, const float* lse,
                  const void* dout, void* dq, void* dk_tok, void* dv_tok, float* dk_cart,
                  float* dv_cart, int32_t accumulate_cart, void* workspace,
                  size_t workspace_bytes, void* stream) {
  CHECK(check_shape(s));
  CHECK(need_ptr(q, "q"));
  CHECK(need_ptr(k_tok, "k_tok"));
  CHECK(need_ptr(v_tok, "v_tok"));
  CHECK(need_ptr(out, "out"));
  CHECK(need_ptr(lse, "lse"));
  CHECK(need_ptr(dout, "dout"));
  CHECK(need_ptr(dq, "dq"));
  CHECK(need_ptr(dk_tok, "dk_tok"));
  CHECK(need_ptr(dv_tok, "dv_tok"));
  if (s->p > 0) {
    CHECK(need_ptr(k_cart, "k_cart"));
    CHECK(need_ptr(v_cart, "v_cart"));
    CHECK(need_ptr(dk_cart, "dk_cart"));
    CHECK(need_ptr(dv_cart, "dv_cart"));
  }
  const AttnDims d = dims_of(s);
  CHECK(check_workspace(workspace, workspace_bytes, bwd_workspace_bytes(d)));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return hip_result(launch_bwd(d, q, k_tok, v_tok, k_cart, v_cart, out, lse, dout, dq, dk_tok,
                               dv_tok, dk_cart, dv_cart, accumulate_cart != 0, workspace, st),
                    st, "cart_attn_bwd");
}

int cart_attn_schedule_query(const cart_attn_shape* s, cart_attn_schedule* out) {
  CHECK(check_shape(s));
  if (!out) return fail(CART_ERR_INVALID_ARG, "out is NULL");
  const AttnDims d = dims_of(s);
  const FwdPlan fp = plan_fwd(d);
  const BwdPlan bp = plan_bwd(d);
  cart_attn_schedule r{};
  r.fwd_grid = fp.grid;
  r.fwd_key_splits = fp.n_splits;
  r.bwd_cart_tiles = bp.n_ct;
  r.bwd_tok_tiles = bp.n_tt;
  if (d.tok_bf16) {
    r.bwd_units_per_piece = bp.kv_target;
    r.bwd_cart_pieces = bp.kv_splits_c;
    r.bwd_tok_pieces_max = bp.kv_stmax;
    r.bwd_kv_grid = bp.grid_kv;
    r.bwd_dq_grid = bp.grid_q;
    r.bwd_dq_key_splits = bp.q_splits;
    r.bwd_tok_units_per_piece = bp.kv_ttok;
  } else {
    // float32 reference mode: one kernel, cartridge tiles split over units,
    // dQ accumulated in the same kernel
    const long long units = (long long)d.B * (d.Hq / d.Hkv) * bp.nqt;
    r.bwd_units_per_piece = (int)((units + bp.splits_c - 1) / bp.splits_c);
    r.bwd_cart_pieces = bp.splits_c;
    r.bwd_tok_pieces_max = 1;
    r.bwd_kv_grid = bp.grid_c + bp.grid_t;
    r.bwd_dq_grid = 0;
    r.bwd_dq_key_splits = 1;
  }
  *out = r;
  g_err[0] = '\0';
  return CART_OK;
}

int32_t cart_parts_rows(const cart_parts* parts) {
  PartTable t;
  if (parts_table(parts, false, &t) != CART_OK) return -1;
  return t.off[t.n];
}

int cart_compose_rows(const cart_parts* parts, cart_dtype src, int32_t n_kv_heads,
                      int32_t head_dim, void* k_out, void* v_out, cart_dtype dst,
                      void* stream) {
  PartTable t;
  CHECK(parts_table(parts, true, &t));
  if (!valid_dtype(src) || !valid_dtype(dst)) return fail(CART_ERR_INVALID_ARG, "unknown dtype");
  if (src == CART_BF16 && dst == CART_F32)
    return fail(CART_ERR_UNSUPPORTED, "bf16 parts compose into bf16 rows only");
  if (n_kv_heads < 1) return fail(CART_ERR_INVALID_ARG, "n_kv_heads must be >= 1");
  if (!valid_head_dim(head_dim))
    return fail(CART_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", head_dim);
  const long long total = (long long)t.off[t.n] * n_kv_heads * head_dim;
  if (total > kMaxElems) return fail(CART_ERR_UNSUPPORTED, "composed prefix too large");
  if (total == 0) { g_err[0] = '\0'; return CART_OK; }
  CHECK(need_ptr(k_out, "k_out"));
  CHECK(need_ptr(v_out, "v_out"));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return hip_result(launch_compose_rows(t, src == CART_BF16, dst == CART_BF16,
                                        n_kv_heads * head_dim, k_out, v_out, st),
                    st, "cart_compose_rows");
}

int cart_attn_bwd_composed(const cart_attn_shape* s, const cart_parts* parts, const void* q,
                           const void* k_tok, const void* v_tok, const void* k_cart,
                           const void* v_cart, const void* out, const float* lse,
                           const void* dout, void* dq, void* dk_tok, void* dv_tok,
                           float* dk_cart, float* dv_cart, int32_t accumulate_cart,
                           void* workspace, size_t workspace_bytes, void* stream) {
  PartTable t;
  CHECK(parts_table(parts, false, &t));
  if (!s) return fail(CART_ERR_INVALID_ARG, "shape is NULL");
  if (s->p != t.off[t.n])
    return fail(CART_ERR_INVALID_ARG, "shape p (%d) differs from the parts' %d rows", s->p,
                t.off[t.n]);
  // the first part's frozen rows are a prefix the backward zeroes itself; the
  // others' are zeroed after it (both end as exact zeros)
  cart_attn_shape s0 = *s;
  s0.frozen_rows = t.frozen[0];
  CHECK(cart_attn_bwd(&s0, q, k_tok, v_tok, k_cart, v_cart, out, lse, dout, dq, dk_tok, dv_tok,
                      dk_cart, dv_cart, accumulate_cart, workspace, workspace_bytes, stream));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return hip_result(launch_zero_frozen(t, s->n_kv_heads * s->head_dim, dk_cart, dv_cart, st),
                    st, "cart_attn_bwd_composed");
}

int cart_cache_create(const cart_cache_desc* d, cart_cache** out) {
  if (!d || !out) return fail(CART_ERR_INVALID_ARG, "desc and out must be non-NULL");
  *out = nullptr;
  if (d->n_seqs < 1 || d->n_kv_heads < 1 || d->max_pages_per_seq < 1 || d->n_pages < 1)
    return fail(CART_ERR_INVALID_ARG, "cache counts must be >= 1");
  if (!valid_head_dim(d->head_dim))
    return fail(CART_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", d->head_dim);
  if (d->page_size != 16) return fail(CART_ERR_UNSUPPORTED, "page_size must be 16");
  if (d->dtype != CART_BF16) return fail(CART_ERR_UNSUPPORTED, "cache dtype must be bf16");
  if ((long long)d->n_pages * d->n_kv_heads * d->page_size * d->head_dim > (1LL << 40))
    return fail(CART_ERR_UNSUPPORTED, "page pool too large");
  if ((long long)d->max_pages_per_seq * d->page_size > 0x7fffffffLL)
    return fail(CART_ERR_UNSUPPORTED, "sequence capacity too large");
  CHECK(need_ptr(d->k_pages, "k_pages"));
  CHECK(need_ptr(d->v_pages, "v_pages"));
  CHECK(need_ptr(d->block_table, "block_table"));
  CHECK(need_ptr(d->seq_lens, "seq_lens"));
  cart_cache* c = new (std::nothrow) cart_cache;
  if (!c) return fail(CART_ERR_INVALID_ARG, "out of host memory");
  c->d = *d;
  c->lens.assign(d->n_seqs, 0);
  *out = c;
  g_err[0] = '\0';
  return CART_OK;
}

int cart_cache_destroy(cart_cache* c) {
  delete c;
  return CART_OK;
}

int cart_cache_reset(cart_cache* c, int32_t seq, void* stream) {
  CHECK(check_seq(c, seq));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int r = hip_result(launch_cache_set_len(cache_dims(c), seq, 0, st), st, "cart_cache_reset");
  if (r == CART_OK) c->lens[seq] = 0;
  return r;
}

int32_t cart_cache_seq_len(const cart_cache* c, int32_t seq) {
  if (!c || seq < 0 || seq >= c->d.n_seqs) return -1;
  return c->lens[seq];
}

int cart_append_cache(cart_cache* c, int32_t seq, const void* k, const void* v, cart_dtype src,
                      int32_t n_rows, int32_t n_kv_heads, int32_t head_dim, void* stream) {
  CHECK(check_rows(c, seq, k, v, src, n_rows, n_kv_heads, head_dim));
  if (n_rows == 0) { g_err[0] = '\0'; return CART_OK; }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int start = c->lens[seq];
  const int r = hip_result(
      launch_cache_append(cache_dims(c), seq, start, k, v, src == CART_BF16, n_rows, st), st,
      "cart_append_cache");
  if (r == CART_OK) c->lens[seq] = start + n_rows;
  return r;
}

int cart_write_cache(cart_cache* c, int32_t seq, const void* k_cart, const void* v_cart,
                     cart_dtype src, int32_t p, int32_t n_kv_heads, int32_t head_dim,
                     void* stream) {
  CHECK(check_seq(c, seq));
  if (c->lens[seq] != 0)
    return fail(CART_ERR_CACHE_NOT_EMPTY, "seq %d already holds %d rows", seq, c->lens[seq]);
  return cart_append_cache(c, seq, k_cart, v_cart, src, p, n_kv_heads, head_dim, stream);
}

int cart_write_composed_cache(cart_cache* c, int32_t seq, const cart_parts* parts,
                              cart_dtype src, int32_t n_kv_heads, int32_t head_dim,
                              void* stream) {
  PartTable t;
  CHECK(parts_table(parts, true, &t));
  CHECK(check_seq(c, seq));
  if (c->lens[seq] != 0)
    return fail(CART_ERR_CACHE_NOT_EMPTY, "seq %d already holds %d rows", seq, c->lens[seq]);
  // every check up front, so a refused composition appends nothing:
  // geometry and dtype (as for zero rows), then the capacity for all parts
  CHECK(check_rows(c, seq, nullptr, nullptr, src, 0, n_kv_heads, head_dim));
  if ((long long)t.off[t.n] > capacity(c))
    return fail(CART_ERR_CACHE_FULL, "seq %d: %d composed rows exceed capacity %lld", seq,
                t.off[t.n], capacity(c));
  for (int i = 0; i < t.n; ++i)
    CHECK(cart_append_cache(c, seq, t.k[i], t.v[i], src, t.rows[i], n_kv_heads, head_dim,
                            stream));
  return CART_OK;
}

size_t cart_decode_workspace_size(const cart_cache* c, int32_t n_q_heads) {
  if (!c || n_q_heads < 1 || n_q_heads % c->d.n_kv_heads != 0) return 0;
  return plan_decode(cache_dims(c), n_q_heads, 1).part_bytes;
}

namespace {

// Checks shared by the decode entry points (kq query tokens per sequence,
// whose rows k_new/v_new are appended first when given); on success *part
// is the bytes of split partials the launch needs.
int check_decode(cart_cache* c, const void* q, const void* k_new, const void* v_new,
                 int32_t kq, int32_t n_q_heads, float scale, void* out, size_t* part) {
  if (!c) return fail(CART_ERR_INVALID_ARG, "cache handle is NULL");
  if (kq < 1 || kq > 64) return fail(CART_ERR_INVALID_ARG, "tokens per sequence (%d) outside [1, 64]", kq);
  if (n_q_heads < 1 || n_q_heads % c->d.n_kv_heads != 0)
    return fail(CART_ERR_GEOMETRY, "n_q_heads %d is not a multiple of the cache's %d kv heads",
                n_q_heads, c->d.n_kv_heads);
  const int g = n_q_heads / c->d.n_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(CART_ERR_UNSUPPORTED, "GQA group size %d not built (1, 2, 4, 8)", g);
  if (!(scale >= 0.f) || isinf(scale)) return fail(CART_ERR_INVALID_ARG, "scale must be >= 0");
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(CART_ERR_INVALID_ARG, "k_new and v_new must both be given or both be NULL");
  CHECK(need_ptr(q, "q"));
  CHECK(need_ptr(out, "out"));
  CHECK(opt_ptr(k_new, "k_new"));
  CHECK(opt_ptr(v_new, "v_new"));
  const int add = k_new ? kq : 0;
  for (int s = 0; s < c->d.n_seqs; ++s) {
    const long long len = (long long)c->lens[s] + add;
    if (len < 1) return fail(CART_ERR_INVALID_ARG, "seq %d holds no rows to attend over", s);
    if (len > capacity(c))
      return fail(CART_ERR_CACHE_FULL, "seq %d: appending exceeds capacity %lld", s, capacity(c));
  }
  *part = plan_decode(cache_dims(c), n_q_heads, kq).part_bytes;
  return CART_OK;
}

int run_decode(cart_cache* c, const void* q, const void* k_new, const void* v_new, int32_t kq,
               int32_t n_q_heads, float scale, void* out, void* ws, void* stream,
               const char* what) {
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)c->d.head_dim);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int r = hip_result(launch_decode(cache_dims(c), n_q_heads, kq, sc, q, k_new, v_new, out,
                                         ws, st),
                           st, what);
  if (r == CART_OK && k_new)
    for (int s = 0; s < c->d.n_seqs; ++s) c->lens[s] += kq;
  return r;
}

}  // namespace

int cart_decode(cart_cache* c, const void* q, const void* k_new, const void* v_new,
                int32_t n_q_heads, float scale, void* out, void* workspace,
                size_t workspace_bytes, void* stream) {
  size_t part = 0;
  CHECK(check_decode(c, q, k_new, v_new, 1, n_q_heads, scale, out, &part));
  CHECK(check_workspace(workspace, workspace_bytes, part));
  return run_decode(c, q, k_new, v_new, 1, n_q_heads, scale, out, workspace, stream,
                    "cart_decode");
}

int cart_decode_verify(cart_cache* c, const void* q, const void* k_new, const void* v_new,
                       int32_t n_tokens, int32_t n_q_heads, float scale, void* out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_new || !v_new)
    return fail(CART_ERR_INVALID_ARG, "a verify step appends its rows: k_new and v_new needed");
  size_t part = 0;
  CHECK(check_decode(c, q, k_new, v_new, n_tokens, n_q_heads, scale, out, &part));
  CHECK(check_workspace(workspace, workspace_bytes, part));
  return run_decode(c, q, k_new, v_new, n_tokens, n_q_heads, scale, out, workspace, stream,
                    "cart_decode_verify");
}

int cart_decode_schedule_query(const cart_cache* c, int32_t n_tokens, int32_t n_q_heads,
                               cart_decode_schedule* out) {
  if (!c) return fail(CART_ERR_INVALID_ARG, "cache handle is NULL");
  if (!out) return fail(CART_ERR_INVALID_ARG, "out is NULL");
  if (n_tokens < 1 || n_tokens > 64)
    return fail(CART_ERR_INVALID_ARG, "tokens per sequence (%d) outside [1, 64]", n_tokens);
  if (n_q_heads < 1 || n_q_heads % c->d.n_kv_heads != 0)
    return fail(CART_ERR_INVALID_ARG, "n_q_heads %d is not a multiple of the cache's %d kv heads",
                n_q_heads, c->d.n_kv_heads);
  const DecodePlan pl = plan_decode(cache_dims(c), n_q_heads, n_tokens);
  cart_decode_schedule r{};
  r.pages_per_split = pl.pages_per_split;
  r.max_splits = pl.max_splits;
  r.waves_per_group = pl.waves;
  r.grid = (int32_t)pl.grid;
  r.workspace_bytes = (int64_t)pl.part_bytes;
  *out = r;
  return CART_OK;
}

size_t cart_decode_verify_workspace_size(const cart_cache* c, int32_t n_tokens,
                                         int32_t n_q_heads) {
  if (!c || n_tokens < 1 || n_tokens > 64 || n_q_heads < 1 || n_q_heads % c->d.n_kv_heads != 0)
    return 0;
  return plan_decode(cache_dims(c), n_q_heads, n_tokens).part_bytes;
}

int cart_cache_truncate(cart_cache* c, int32_t seq, int32_t new_len, void* stream) {
  CHECK(check_seq(c, seq));
  if (new_len < 0 || new_len > c->lens[seq])
    return fail(CART_ERR_INVALID_ARG, "seq %d: new length %d outside [0, %d]", seq, new_len,
                c->lens[seq]);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int r = hip_result(launch_cache_set_len(cache_dims(c), seq, new_len, st), st,
                           "cart_cache_truncate");
  if (r == CART_OK) c->lens[seq] = new_len;
  return r;
}

int cart_decode_noalloc(cart_cache* c, const void* q, const void* k_new, const void* v_new,
                        int32_t n_q_heads, float scale, void* out, void* stream) {
  size_t part = 0;
  CHECK(check_decode(c, q, k_new, v_new, 1, n_q_heads, scale, out, &part));
  if (part > kDecodeScratchBytes)
    return fail(CART_ERR_WORKSPACE,
                "cart_decode_noalloc: %zu bytes of split partials exceed the library's "
                "%zu-byte scratch (use cart_decode with a workspace)",
                part, kDecodeScratchBytes);
  void* ws = nullptr;
  if (part > 0) {
    const hipError_t e = decode_scratch(&ws);
    if (e != hipSuccess)
      return fail(CART_ERR_HIP, "cart_decode_noalloc: scratch address: %s", hipGetErrorString(e));
  }
  return run_decode(c, q, k_new, v_new, 1, n_q_heads, scale, out, ws, stream,
                    "cart_decode_noalloc");
}

size_t cart_decode_noalloc_max_bytes(void) { return kDecodeScratchBytes; }

}  // extern "C"
