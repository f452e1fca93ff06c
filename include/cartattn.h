/*
 * libcartattn: the cartridge-attention hot path for AMD MI355X (gfx950).
 *
 * A cartridge is a trained KV prefix: per layer, p key/value rows of shape
 * [p, n_kv_heads, head_dim] living in the space of KV-cache rows. Keys are
 * already rotated (RoPE at positions 0..p-1) and are never rotated again;
 * real tokens sit at RoPE positions p, p+1, ...; row 0 is a frozen "sink".
 * Attention runs over concat(sink, trainable rows, real tokens) with the
 * causal mask aligned to the end (source_offset = kv_seq - q_seq = p): all p
 * prefix rows are visible to every token's query, and among the real tokens
 * a query reaches only itself and the tokens before it. Gradients flow
 * through the concat into the trainable rows; serving writes the prefix into
 * an empty KV cache and decodes behind it.
 *   Source: "Cartridges: trained KV-prefix corpus compression" (Fucina
 *   guide), section "Semantics (pinned to the reference implementation)".
 *
 * Conventions for every call below
 *   - Pointers are caller-owned DEVICE pointers unless marked (host).
 *   - Layouts are dense row-major: Q, O, dO, dQ [batch, q_seq, n_q_heads,
 *     head_dim]; token K/V and their gradients [batch, q_seq, n_kv_heads,
 *     head_dim]; cartridge K/V and their gradients [p, n_kv_heads, head_dim];
 *     LSE [batch, n_q_heads, q_seq] float32 (natural log).
 *   - q-head h reads kv-head h / (n_q_heads / n_kv_heads).
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL is the default stream), never synchronizes, never allocates
 *     device memory and keeps no pointer after it returns.
 *   - All argument checks run on the host before any HIP call, so every
 *     error is reported without touching the GPU. A failed check launches
 *     nothing. A launch failure returns CART_ERR_HIP; the HIP message is in
 *     cart_last_error(). Faults inside kernels surface at the caller's next
 *     synchronization (set CARTATTN_SYNC=1 to synchronize after each call).
 *   - Device pointers must be 16-byte aligned (CART_ERR_ALIGNMENT).
 *   - Calls are thread-safe except on the same cart_cache, which the caller
 *     must serialize.
 */
#ifndef CARTATTN_H
#define CARTATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CART_OK = 0,
  CART_ERR_INVALID_ARG = 1,     /* null pointer, bad size or count */
  CART_ERR_UNSUPPORTED = 2,     /* valid but not built: head_dim, dtype mix */
  CART_ERR_ALIGNMENT = 3,       /* a device pointer is not 16-byte aligned */
  CART_ERR_WORKSPACE = 4,       /* workspace missing or too small */
  CART_ERR_CACHE_NOT_EMPTY = 5, /* cart_write_cache into a non-empty seq */
  CART_ERR_CACHE_FULL = 6,      /* rows would exceed the sequence's pages */
  CART_ERR_GEOMETRY = 7,        /* cache and cartridge disagree on heads/dim */
  CART_ERR_HIP = 8              /* a HIP launch or runtime call failed */
} cart_status;

typedef enum { CART_F32 = 0, CART_BF16 = 1 } cart_dtype;

/* Shape of one attention layer of a cartridge training step. */
typedef struct {
  int32_t batch;        /* B >= 1 */
  int32_t q_seq;        /* n >= 1 real tokens per sequence */
  int32_t p;            /* cartridge rows, p >= 0 (p = 0: plain causal) */
  int32_t frozen_rows;  /* 0 <= frozen_rows <= p; the pages' default is 1 */
  int32_t n_q_heads;    /* Hq, a multiple of n_kv_heads */
  int32_t n_kv_heads;   /* Hkv >= 1 */
  int32_t head_dim;     /* d in {64, 128} */
  float scale;          /* softmax scale; 0 selects 1/sqrt(head_dim) */
  cart_dtype tok_dtype; /* Q, token K/V, O, dO, dQ, token dK/dV */
  cart_dtype row_dtype; /* cartridge K/V storage (f32 master rows or bf16) */
  int32_t window;       /* 0: none; W > 0: sliding window, see below */
  const int32_t* seg_lens; /* (host) NULL, or [batch] packed segment lengths, see below */
} cart_attn_shape;
/* Sliding window (local attention layers, e.g. gemma4's; Cartridges guide,
   section "gemma4 (measured)": such layers see the cartridge exactly as a
   real prefix, within the window, and the window may cut through it):
   the query of token i, at position p + i, sees only the rows at positions
   above p + i - W (cartridge row j is at position j, token row t at p + t),
   itself included. W >= p + q_seq is the same as no window. */
/* Packed segments (Cartridges guide, "Deliberate divergences from the
   reference": a group of conversations runs as contiguous segments of one
   forward, RoPE restarting and attention running per segment behind the one
   shared prefix, whose gradient sums over the segments): with seg_lens set,
   the token tensors hold batch = 1..64 segments back to back -- Q, O, dO, dQ
   [T, n_q_heads, head_dim], token K/V and their gradients [T, n_kv_heads,
   head_dim], T = the sum of seg_lens -- segment b at rows off_b ..
   off_b + seg_lens[b] - 1 (off_b = the lengths before it). Each segment
   attends like one sequence of the batch (its token i at position p + i;
   rotate with cart_rope_tokens_packed). 1 <= seg_lens[b] <= q_seq, and LSE
   keeps the padded layout [batch, n_q_heads, q_seq] (entries past a
   segment's end are not written or read). The array is read during the call
   only. */
/* Supported dtype pairs: (tok F32, rows F32) is the float32 reference mode
   (all arithmetic in f32); (tok BF16, rows F32 or BF16) is the bf16 mode:
   MFMA operands are bf16 (f32 rows are rounded to nearest-even on load),
   accumulation and softmax are f32. Anything else: CART_ERR_UNSUPPORTED. */

/*
 * cart_rope_tokens -- rotate the real-token queries and keys in place.
 *   Source: Cartridges guide, "Semantics": real tokens sit at RoPE positions
 *   p, p+1, ...; cartridge keys are never rotated again (so they are never
 *   passed here). RIG cartridge-injection hand-off, section 5: a shifted
 *   base position silently corrupts attention.
 *
 * q [batch, seq, n_q_heads, head_dim] and k [batch, seq, n_kv_heads,
 * head_dim] (k may be NULL) of dtype `dt`. Token (b, i) is at position
 *   pos = pos_base + (pos_offsets ? pos_offsets[b] : 0) + i,
 * pos_offsets being a DEVICE int32 array [batch] or NULL. Element k and
 * k + d/2 form a pair rotated by angle pos * theta^(-2k/d) (angle computed in
 * double precision, rotation in f32, result rounded to `dt`):
 *   x'[k] = x[k] cos - x[k+d/2] sin,   x'[k+d/2] = x[k+d/2] cos + x[k] sin.
 * inverse != 0 rotates by -angle: the transpose of the forward rotation,
 * which carries dQ and dK_tok back through RoPE in the backward pass.
 * For a training step pos_base = p; for a decode step pos_base = 0 and
 * pos_offsets = the cache's seq_lens (the new token sits at seq_len).
 */
int cart_rope_tokens(void* q, void* k, cart_dtype dt, int32_t batch, int32_t seq,
                     int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                     int32_t pos_base, const int32_t* pos_offsets, double theta,
                     int32_t inverse, void* stream);

/* cart_rope_tokens over packed segments: q [T, n_q_heads, head_dim] and k
   [T, n_kv_heads, head_dim] (nullable) hold n_segs (1..64) segments back to
   back, of lengths seg_lens (host, each >= 1, T = their sum); token t of a
   segment sits at position pos_base + t (positions restart per segment). */
int cart_rope_tokens_packed(void* q, void* k, cart_dtype dt, int32_t n_segs,
                            const int32_t* seg_lens, int32_t n_q_heads, int32_t n_kv_heads,
                            int32_t head_dim, int32_t pos_base, double theta, int32_t inverse,
                            void* stream);

/*
 * cart_qk_norm_rope -- the per-head RMS normalization of the real-token
 * queries and keys followed by RoPE, in one pass (the step before attention).
 *   Source: Cartridges guide, "Semantics": cartridge keys are rows of the KV
 *   cache, i.e. taken after the q/k normalization and after RoPE, so the
 *   real tokens' queries and keys enter the attention normalized and rotated
 *   at positions p, p+1, .... The normalization is the Qwen3 q/k RMSNorm.
 *
 * q_in [batch, seq, n_q_heads, head_dim], k_in [batch, seq, n_kv_heads,
 * head_dim] (k_in may be NULL, then k_out and w_k are ignored) of dtype `dt`;
 * w_q, w_k: float32 [head_dim] weights. For each head row x:
 *   y = x * w / sqrt(mean(x^2) + eps),
 * then y is rotated exactly as cart_rope_tokens rotates (position
 * pos_base + pos_offsets[b] + i, theta, angle in double precision). The
 * arithmetic is f32 and the result is rounded once to `dt` into q_out/k_out,
 * which may be q_in/k_in (in place) when the backward is not needed.
 * batch * seq = 0 is a no-op. eps > 0.
 */
int cart_qk_norm_rope(const void* q_in, const void* k_in, void* q_out, void* k_out,
                      const float* w_q, const float* w_k, cart_dtype dt, int32_t batch,
                      int32_t seq, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                      float eps, int32_t pos_base, const int32_t* pos_offsets, double theta,
                      void* stream);

/*
 * cart_qk_norm_rope_bwd -- the gradient of cart_qk_norm_rope with respect to
 * its inputs (the weights are frozen: no weight gradient).
 *   Source: as cart_qk_norm_rope; the gradients of the real tokens' queries
 *   and keys flow back through it towards earlier layers (and their
 *   cartridges, through the residual stream).
 *
 * q_in/k_in: the forward's inputs; dq_out/dk_out: gradients of its outputs
 * (the attention backward's dq, dk_tok). With r = 1/sqrt(mean(x^2) + eps)
 * and dy = the output gradient rotated by -angle:
 *   dx = r w dy - (r^3 / head_dim) x sum_j(w_j dy_j x_j)
 * into dq_in/dk_in (dtype `dt`), which may alias dq_out/dk_out but not the
 * inputs (CART_ERR_INVALID_ARG). Other arguments as for the forward.
 */
int cart_qk_norm_rope_bwd(const void* q_in, const void* k_in, const void* dq_out,
                          const void* dk_out, void* dq_in, void* dk_in, const float* w_q,
                          const float* w_k, cart_dtype dt, int32_t batch, int32_t seq,
                          int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float eps,
                          int32_t pos_base, const int32_t* pos_offsets, double theta,
                          void* stream);

/*
 * cart_adam_rows -- one Adam step on a cartridge tensor (the step after the
 * backward), optionally writing its bf16 copy for the next step's attention.
 *   Source: Cartridges guide, "Semantics" (objective paragraph): Adam, no
 *   weight decay, no schedule, lr 2e-2; row 0 is frozen (frozen_prefix);
 *   "Learning rate vs batch size (measured)": lr 2e-3 at small batches.
 *
 * rows, grad, m, v: float32 [n_rows, row_elems] (for a cartridge tensor
 * [p, n_kv_heads, head_dim]: n_rows = p, row_elems = n_kv_heads * head_dim);
 * m and v are the caller-owned moments (zero before step 1). For every
 * element of rows >= frozen_rows, at step `step` >= 1:
 *   m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
 *   x -= (lr / (1 - b1^step)) m / (sqrt(v) / sqrt(1 - b2^step) + eps).
 * Frozen rows keep x, m and v. rows_bf16 (nullable, bf16 [n_rows,
 * row_elems]) receives every row of the updated x rounded to nearest even:
 * passing it as bf16 cartridge rows to cart_attn_fwd / cart_attn_bwd is
 * the same as passing the f32 rows. row_elems % 4 == 0; 16-byte aligned.
 * The hyperparameters are given in double precision; the bias corrections
 * and the factors (1 - beta) are formed in double and rounded once to f32,
 * the update itself is f32.
 */
int cart_adam_rows(float* rows, const float* grad, float* m, float* v, void* rows_bf16,
                   int64_t n_rows, int32_t row_elems, int32_t frozen_rows, int32_t step,
                   double lr, double beta1, double beta2, double eps, void* stream);

/*
 * cart_rows_to_bf16 -- the bf16 operands of f32 cartridge rows, made once.
 *   Source: Cartridges guide, "Semantics" (parameterization): the trainable
 *   rows are float32; the attention's products read them as bf16 operands.
 *
 * k_bf16[i] = bf16(k[i]) and v_bf16[i] = bf16(v[i]) (nearest even) for the
 * n_rows x row_elems elements of k and v (float32; for a cartridge tensor
 * n_rows = p, row_elems = n_kv_heads * head_dim). This is the rounding that
 * cart_attn_fwd and cart_attn_bwd apply to f32 rows as they load them, so
 * passing the outputs as bf16 cartridge rows gives the same results as
 * passing k and v; a step that runs the forward and the backward on the same
 * rows converts them once instead of in each call. The outputs must not
 * overlap the inputs. row_elems % 4 == 0; every pointer 16-byte aligned and
 * non-NULL unless n_rows = 0.
 */
int cart_rows_to_bf16(const float* k, const float* v, void* k_bf16, void* v_bf16,
                      int64_t n_rows, int32_t row_elems, void* stream);

/*
 * Workspace bytes that cart_attn_fwd (for_backward = 0) or cart_attn_bwd
 * (for_backward = 1) needs for shape `s` (host pointer). Returns 0 for an
 * invalid shape. The workspace is caller-owned device memory, 256-byte
 * aligned, with no required contents; its contents are undefined afterwards.
 */
size_t cart_attn_workspace_size(const cart_attn_shape* s, int32_t for_backward);

/*
 * cart_attn_fwd -- end-aligned causal GQA over concat(cartridge, tokens).
 *   Source: Cartridges guide, "Semantics" (attention paragraph) and
 *   "Evidence" (kv_seq > q_seq with GQA).
 *
 * For query i of (b, h) and concatenated row j in [0, p + q_seq):
 *   key_j = k_cart[j, h/g] if j < p else k_tok[b, j - p, h/g] (same for V);
 *   row j is visible iff j <= i + p (and, with a window W, j > i + p - W);
 *   out[b,i,h] = sum_j softmax_j(scale * q[b,i,h] . key_j) v_j;
 *   lse[b,h,i] = log sum_j exp(scale * q[b,i,h] . key_j)   (visible j).
 * The concat is virtual: the two row sources are read in place.
 * q, k_tok, v_tok, out: tok_dtype; k_cart, v_cart: row_dtype (may be NULL
 * when p = 0); lse: float32, required (the backward reads it).
 */
int cart_attn_fwd(const cart_attn_shape* s, const void* q, const void* k_tok,
                  const void* v_tok, const void* k_cart, const void* v_cart,
                  void* out, float* lse, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * cart_attn_bwd -- gradients of the forward above, through the concat.
 *   Source: Cartridges guide, "Semantics": the f32-KV backward routes
 *   gradients through the concat into the trainable rows; row 0 is frozen.
 *
 * Inputs as for cart_attn_fwd plus `out` and `lse` from it and `dout`.
 * With D_i = dout_i . out_i, P_ij = exp(scale q_i.key_j - lse_i) on visible
 * pairs and dS_ij = P_ij (dout_i . v_j - D_i):
 *   dq_i   = scale sum_j dS_ij key_j                  -> dq (tok_dtype)
 *   dkey_j = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dout_i.
 * Token rows j >= p go to dk_tok/dv_tok (tok_dtype), summed over the q-heads
 * of the GQA group for their own sequence. Cartridge rows j < p are summed
 * over the whole batch and the group into dk_cart/dv_cart (float32
 * [p, n_kv_heads, head_dim]); rows below frozen_rows are written as exact
 * zeros. accumulate_cart != 0 adds the new cartridge gradients to the
 * buffers' contents (frozen rows still end as zeros) instead of overwriting.
 * No RoPE adjoint is applied: call cart_rope_tokens(inverse=1) on dq and
 * dk_tok afterwards. All accumulation is float32.
 */
int cart_attn_bwd(const cart_attn_shape* s, const void* q, const void* k_tok,
                  const void* v_tok, const void* k_cart, const void* v_cart,
                  const void* out, const float* lse, const void* dout, void* dq,
                  void* dk_tok, void* dv_tok, float* dk_cart, float* dv_cart,
                  int32_t accumulate_cart, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * cart_attn_schedule_query -- how cart_attn_fwd / cart_attn_bwd will split
 * the work of shape `s` (host pointer) over the GPU. Host-only (no HIP call,
 * no device memory); the same plan the launches use, so a caller or a test
 * can see which code paths a shape takes (for example whether key tiles are
 * cut into pieces that the dK/dV kernel reduces itself). Not one of the
 * method's operations: a diagnostic of this library's schedule.
 * Returns CART_ERR_INVALID_ARG (or _UNSUPPORTED) for a bad shape or NULL out.
 */
typedef struct {
  int32_t fwd_grid;               /* forward workgroups */
  int32_t fwd_key_splits;         /* > 1: key range split, partials merged by LSE */
  int32_t bwd_cart_tiles;         /* 128-row cartridge key tiles per kv head */
  int32_t bwd_tok_tiles;          /* 128-row token key tiles per (batch, kv head) */
  int32_t bwd_units_per_piece;    /* target (batch, q-head, 32-query) units per piece */
  int32_t bwd_cart_pieces;        /* pieces per cartridge tile (> 1: cut, reduced in-kernel) */
  int32_t bwd_tok_pieces_max;     /* most pieces of one token tile (> 1: cut) */
  int32_t bwd_kv_grid;            /* dK/dV workgroups */
  int32_t bwd_dq_grid;            /* dQ workgroups */
  int32_t bwd_dq_key_splits;      /* > 1: dQ key range split, pieces summed after */
  int32_t bwd_tok_units_per_piece; /* token tiles: pieces of at most this many units
                                      (bf16 tokens; 0 in the float32 mode) */
} cart_attn_schedule;
int cart_attn_schedule_query(const cart_attn_shape* s, cart_attn_schedule* out);

/* ------------------------------------------------------------------------
 * Composed cartridges.
 *   Source: Cartridges guide, section "Composition": independently trained
 *   cartridges compose by concatenation (part 0's rows, then part 1's, ...);
 *   real tokens sit at RoPE positions starting at the composed length; every
 *   part keeps the rotations it was trained at; the composed prefix is one
 *   concatenation per layer, so the attention backward routes gradients into
 *   every part's trainable rows while each part's sink stays frozen; serving
 *   writes the parts in order into an empty cache with the append primitive.
 *
 * A composed layer runs the single-cartridge calls on the composed rows:
 *   cart_compose_rows  -> k_cart, v_cart [P, Hkv, d] (P = cart_parts_rows)
 *   cart_rope_tokens(pos_base = P), cart_attn_fwd(p = P)
 *   cart_attn_bwd_composed -> dk_cart, dv_cart [P, Hkv, d] float32, part i's
 *     gradient being rows off_i .. off_i + rows[i] - 1 (off_i = the rows of
 *     the parts before it), each part's first frozen[i] rows exact zeros.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t n_parts;          /* 1 .. 64 */
  const int32_t* rows;      /* (host) [n_parts]: rows of each part, >= 0 */
  const int32_t* frozen;    /* (host) [n_parts]: frozen rows of each part, 0..rows[i] */
  const void* const* k;     /* (host) [n_parts] device pointers: part i's K [rows[i], Hkv, d] */
  const void* const* v;     /* (host) [n_parts] device pointers: part i's V */
} cart_parts;

/* Composed length P = sum of rows[], or -1 for an invalid description. */
int32_t cart_parts_rows(const cart_parts* parts);

/* Concatenate the parts' K and V rows (dtype src) into k_out/v_out
   [P, n_kv_heads, head_dim] of dtype dst, rounding f32 to bf16 to nearest
   even (bf16 -> f32 is CART_ERR_UNSUPPORTED). With dst = bf16 the result is
   what cart_attn_fwd/bwd would round f32 rows to, so passing it as bf16 rows
   gives the same results as passing f32 rows. Parts with 0 rows may have
   NULL pointers. */
int cart_compose_rows(const cart_parts* parts, cart_dtype src, int32_t n_kv_heads,
                      int32_t head_dim, void* k_out, void* v_out, cart_dtype dst,
                      void* stream);

/* cart_attn_bwd over a composed prefix: s->p must equal the composed length
   and s->frozen_rows is ignored (each part freezes its own first frozen[i]
   rows; only rows[] and frozen[] of `parts` are read). k_cart/v_cart are the
   composed rows; dk_cart/dv_cart receive the composed gradient. Everything
   else is as for cart_attn_bwd (same workspace size). */
int cart_attn_bwd_composed(const cart_attn_shape* s, const cart_parts* parts, const void* q,
                           const void* k_tok, const void* v_tok, const void* k_cart,
                           const void* v_cart, const void* out, const float* lse,
                           const void* dout, void* dq, void* dk_tok, void* dv_tok,
                           float* dk_cart, float* dv_cart, int32_t accumulate_cart,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Serving: a paged KV cache that hosts a prefix no tokens produced.
 *   Source: Cartridges guide, "Semantics" (serving): an empty cache receives
 *   all p prefix rows in its own dtype, its length becomes p, and ordinary
 *   decoding resumes at position p. "Evidence"
 *   (serving parity). Composition section: appendToCache is the primitive.
 *   RIG hand-off, section 5: cartridges are locked to the model geometry
 *   and the KV dtype must match the serving cache.
 * ------------------------------------------------------------------------ */
typedef struct cart_cache cart_cache; /* opaque; holds only host state */

typedef struct {
  int32_t n_seqs;            /* sequences (slots) in the cache */
  int32_t n_kv_heads;
  int32_t head_dim;          /* 64 or 128 */
  int32_t page_size;         /* rows per page; must be 16 */
  int32_t max_pages_per_seq; /* columns of block_table */
  int32_t n_pages;           /* pages in each pool */
  cart_dtype dtype;          /* must be CART_BF16 */
  void* k_pages;             /* [n_pages, n_kv_heads, page_size, head_dim] */
  void* v_pages;             /* same */
  const int32_t* block_table;/* [n_seqs, max_pages_per_seq], page ids */
  int32_t* seq_lens;         /* [n_seqs]; must hold zeros at creation */
} cart_cache_desc;
/* Page ids in block_table must lie in [0, n_pages); kernels skip rows whose
   page id does not (they neither read nor write out of bounds). Each
   sequence holds at most max_pages_per_seq * page_size rows. The library
   keeps a host mirror of every seq_len, so no call reads device memory back;
   every call that changes a length also writes the device seq_lens. */

int cart_cache_create(const cart_cache_desc* d /*host*/, cart_cache** out /*host*/);
int cart_cache_destroy(cart_cache* c);
/* seq_len := 0 for one sequence (device copy updated on `stream`). */
int cart_cache_reset(cart_cache* c, int32_t seq, void* stream);
/* Host mirror of one sequence's length, or -1 for a bad handle/seq. */
int32_t cart_cache_seq_len(const cart_cache* c, int32_t seq);

/* Append n_rows rows k/v [n_rows, n_kv_heads, head_dim] of dtype `src` at the
   end of sequence `seq`, converting to the cache dtype (bf16, round to
   nearest even), and advance the sequence by n_rows. The rows' geometry must
   equal the cache's (else CART_ERR_GEOMETRY); the sequence must have room
   (else CART_ERR_CACHE_FULL). n_rows = 0 is a no-op. */
int cart_append_cache(cart_cache* c, int32_t seq, const void* k, const void* v,
                      cart_dtype src, int32_t n_rows, int32_t n_kv_heads,
                      int32_t head_dim, void* stream);

/* Write a cartridge prefix k_cart/v_cart [p, n_kv_heads, head_dim] (one
   layer) into an EMPTY sequence (else CART_ERR_CACHE_NOT_EMPTY), converting
   to bf16, and advance the sequence to p. A cartridge whose head count or
   head_dim differs from the cache's is refused with CART_ERR_GEOMETRY. */
int cart_write_cache(cart_cache* c, int32_t seq, const void* k_cart,
                     const void* v_cart, cart_dtype src, int32_t p,
                     int32_t n_kv_heads, int32_t head_dim, void* stream);

/* Write a composed prefix into an EMPTY sequence (else CART_ERR_CACHE_NOT_EMPTY):
   the parts in order, each appended with cart_append_cache (dtype src,
   converted to bf16), so the sequence ends at the composed length. Geometry
   and the capacity for all parts are checked before anything is appended. */
int cart_write_composed_cache(cart_cache* c, int32_t seq, const cart_parts* parts,
                              cart_dtype src, int32_t n_kv_heads, int32_t head_dim,
                              void* stream);

/*
 * cart_decode -- one decode step (q_seq = 1) for every sequence.
 *   Source: Cartridges guide, "Semantics" (serving) and "Evidence" (serving
 *   parity: decode behind the written prefix matches the trainer's eval).
 *
 * q [n_seqs, n_q_heads, head_dim] bf16, already rotated at position seq_len.
 * If k_new and v_new [n_seqs, n_kv_heads, head_dim] bf16 are both non-NULL
 * they are appended at row seq_len first and every length advances by one
 * (the token sees itself); both NULL attends over the stored rows only.
 * Then out[s,h] = sum_j softmax_j(scale q[s,h] . K[s,j,h/g]) V[s,j,h/g] over
 * all rows of sequence s (no mask). out: [n_seqs, n_q_heads, head_dim] bf16.
 * scale 0 selects 1/sqrt(head_dim). Every sequence must hold >= 1 row.
 * The GQA group n_q_heads / n_kv_heads must be 1, 2, 4 or 8
 * (else CART_ERR_UNSUPPORTED; not a multiple of the cache's kv heads:
 * CART_ERR_GEOMETRY). The workspace size depends only on the cache geometry
 * and n_q_heads; it is 0 (workspace may be NULL) when the splits of every
 * sequence are merged on chip, which cart_decode_schedule_query reports.
 */
int cart_decode(cart_cache* c, const void* q, const void* k_new, const void* v_new,
                int32_t n_q_heads, float scale, void* out, void* workspace,
                size_t workspace_bytes, void* stream);
size_t cart_decode_workspace_size(const cart_cache* c, int32_t n_q_heads);

/*
 * cart_decode_verify -- one verify step of n_tokens draft tokens per
 * sequence (speculative decoding) behind the cache.
 *   Source: Cartridges guide, "Batched self-study (measured)": every stream
 *   verifies a span of draft tokens in one pass, attention per stream
 *   against its own cache, greedy acceptance per row, rejected rows removed
 *   by truncating rewinds (cart_cache_truncate).
 *
 * q [n_seqs, n_tokens, n_q_heads, head_dim] bf16, token t rotated at
 * position seq_len + t; k_new, v_new [n_seqs, n_tokens, n_kv_heads,
 * head_dim] bf16 (required) are appended first, so every sequence grows by
 * n_tokens; token t then attends over rows 0 .. old_len + t (itself and the
 * drafts before it, not those after). out [n_seqs, n_tokens, n_q_heads,
 * head_dim] bf16. n_tokens in [1, 64]; n_tokens = 1 is cart_decode with an
 * appended row. Other rules as for cart_decode; its workspace is
 * cart_decode_verify_workspace_size(c, n_tokens, n_q_heads) bytes.
 */
int cart_decode_verify(cart_cache* c, const void* q, const void* k_new, const void* v_new,
                       int32_t n_tokens, int32_t n_q_heads, float scale, void* out,
                       void* workspace, size_t workspace_bytes, void* stream);
size_t cart_decode_verify_workspace_size(const cart_cache* c, int32_t n_tokens,
                                         int32_t n_q_heads);

/*
 * cart_decode_schedule_query -- how cart_decode (n_tokens = 1),
 * cart_decode_verify and cart_decode_noalloc will split the pages of cache
 * `c` for n_q_heads query heads over the GPU. Host-only (no HIP call, no
 * device memory); the same plan the launches use, so a caller or a test can
 * see which path a geometry takes. Not one of the method's operations: a
 * diagnostic of this library's schedule. CART_ERR_INVALID_ARG for a NULL
 * handle or out, n_tokens outside [1, 64], or n_q_heads not a positive
 * multiple of the cache's kv heads.
 */
typedef struct {
  int32_t pages_per_split;   /* 16-row pages a split streams at most */
  int32_t max_splits;        /* splits of a sequence at full capacity */
  int32_t waves_per_group;   /* > 0: a sequence's splits are the waves of one workgroup,
                                merged on chip; 0: one workgroup per split, partials
                                merged by a second kernel through the workspace */
  int32_t grid;              /* decode workgroups */
  int64_t workspace_bytes;   /* the workspace the call needs (0: none) */
} cart_decode_schedule;
int cart_decode_schedule_query(const cart_cache* c, int32_t n_tokens, int32_t n_q_heads,
                               cart_decode_schedule* out);

/* Shorten one sequence to new_len rows (0 <= new_len <= its length), e.g. to
   drop the rejected drafts of a verify step; cart_cache_reset is new_len 0. */
int cart_cache_truncate(cart_cache* c, int32_t seq, int32_t new_len, void* stream);

/*
 * cart_decode_noalloc -- cart_decode without a workspace argument and without
 * any device allocation, for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, checks, kernels and results as cart_decode; the split
 * partials (when they are not merged on chip) go to a scratch array that
 * the library holds in device memory (one per GPU, kept until the process
 * ends), of at most
 * cart_decode_noalloc_max_bytes() bytes: a cache/head geometry whose
 * cart_decode_workspace_size() exceeds it is refused with CART_ERR_WORKSPACE.
 * Every call on one GPU shares that GPU's scratch, so calls that overlap on
 * one GPU (concurrent streams or threads) race and must be serialized by the
 * caller. The first call on a device looks up the scratch's address there
 * (a HIP runtime query; CART_ERR_HIP if it fails).
 */
int cart_decode_noalloc(cart_cache* c, const void* q, const void* k_new, const void* v_new,
                        int32_t n_q_heads, float scale, void* out, void* stream);
size_t cart_decode_noalloc_max_bytes(void);

/* ------------------------------------------------------------------------
 * Launch timing (profiling aid). When enabled, every kernel launch of this
 * library is bracketed by two HIP events on its own stream. Kernel names:
 * "rope", "rows_to_bf16" (the forward's bf16 shadow of f32 cartridge rows;
 * the backward's is made by "bwd_preprocess"), "attn_fwd", "attn_fwd_combine", "bwd_preprocess",
 * "attn_bwd" (dK/dV, including the reduction of key tiles cut into pieces,
 * for bf16 tokens), "attn_bwd_dq" (dQ of bf16 tokens), "bwd_dq_combine",
 * "bwd_dq_finalize" (dQ of f32 tokens), "bwd_cart_reduce" (f32 tokens),
 * "cache_append", "decode_append", "decode", "decode_merge" (past 8 splits per
 * sequence), "qk_norm_rope",
 * "qk_norm_rope_bwd", "adam_rows", "compose_rows", "zero_frozen" (the
 * per-part frozen rows of cart_attn_bwd_composed). cart_timing_enable clears earlier records (after
 * waiting for them). cart_timing_query waits for the recorded events of one
 * kernel name and returns their summed duration (ms) and count.
 * ------------------------------------------------------------------------ */
int cart_timing_enable(int32_t on);
/* Restrict recording to launches of one kernel name (NULL or "" = all), so
 * that timing one kernel adds two event records per launch of that kernel
 * only. Kept across cart_timing_enable calls. */
int cart_timing_only(const char* kernel);
int cart_timing_query(const char* kernel, double* total_ms, int32_t* launches);

const char* cart_status_string(int status);
const char* cart_last_error(void); /* detail of the last failure, this thread */

#ifdef __cplusplus
}
#endif
#endif /* CARTATTN_H */
