// Internal interface between the C-ABI host layer (cartattn.cpp) and the
// kernel translation units. Everything here runs on the host; argument
// checking has already been done by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cartattn {

// Where each sequence's token rows are. A uniform batch: sequence b at rows
// b n .. b n + n - 1. Packed segments (at most kMaxSegs): segment b at rows
// off[b] .. off[b+1] - 1 of one packed tensor, of length off[b+1] - off[b]
// (<= n, the longest). Passed by value to the kernels.
constexpr int kMaxSegs = 64;
struct Segs {
  int packed;             // 0: a uniform batch; else the number of segments
  int off[kMaxSegs + 1];
  __host__ __device__ int base(int b, int n) const { return packed ? off[b] : b * n; }
  __host__ __device__ int len(int b, int n) const { return packed ? off[b + 1] - off[b] : n; }
  __host__ __device__ int rows(int B, int n) const { return packed ? off[B] : B * n; }
};

struct AttnDims {
  int B, n, p, f;       // batch, q_seq, cartridge rows, frozen rows
  int Hq, Hkv, D;       // heads and head_dim
  float scale;          // resolved softmax scale (never 0)
  bool tok_bf16;        // token tensors are bf16 (else f32)
  bool row_bf16;        // cartridge rows are bf16 (else f32)
  int window;           // > 0: sliding window of positions (0: none)
  Segs seg;             // token rows of each sequence (uniform or packed)
};

// Forward launch plan; the workspace size and the launch both derive from it.
struct FwdPlan {
  int hpw, wph, n_hg, n_qb, n_splits, grid;
  size_t shadow_bytes, o_part_bytes, lse_part_bytes;
};
FwdPlan plan_fwd(const AttnDims& a);
size_t fwd_workspace_bytes(const AttnDims& a);
hipError_t launch_fwd(const AttnDims& a, const void* q, const void* k_tok, const void* v_tok,
                      const void* k_cart, const void* v_cart, void* out, float* lse,
                      void* ws, hipStream_t st);

struct BwdPlan {
  int n_ct, n_tt, nqt, splits_c, grid_c, grid_t;   // float32 path
  // bf16 dK/dV kernel: every key tile's unit list is cut into pieces of about
  // kv_target units (cartridge tiles into kv_splits_c pieces, token tile t
  // into ceil(units_t / kv_target)); kv_ptok pieces per (kv head, batch) of
  // token tiles, at most kv_stmax per token tile.
  int kv_target, kv_splits_c, kv_ptok, kv_stmax, grid_kv;
  int kv_ttok;          // token tiles: pieces of at most this many units (<= kv_target)
  int kv_cart_pieces;   // dK/dV pieces of one kv head's cartridge tiles
  int kv_tok_pieces;    // dK/dV pieces of one kv head's token tiles (all sequences)
  int hpw, wph, n_hg, n_qb, q_splits, grid_q;     // query-major dQ kernel
  int q_pair;           // 1: the dQ grid is resident at once (query blocks dealt in pairs)
  size_t shadow_bytes, dq_bytes, delta_bytes, part_bytes, tok_part_bytes, dq_part_bytes, cnt_bytes;
};
BwdPlan plan_bwd(const AttnDims& a);
size_t bwd_workspace_bytes(const AttnDims& a);
hipError_t launch_bwd(const AttnDims& a, const void* q, const void* k_tok, const void* v_tok,
                      const void* k_cart, const void* v_cart, const void* out,
                      const float* lse, const void* dout, void* dq, void* dk_tok,
                      void* dv_tok, float* dk_cart, float* dv_cart, bool accumulate,
                      void* ws, hipStream_t st);

// f32 cartridge rows -> bf16 shadow (n elements per tensor, n % 4 == 0).
hipError_t launch_rows_to_bf16(const float* k, const float* v, __bf16* kb, __bf16* vb, size_t n,
                               hipStream_t st);

// seg (nullable): packed segments, token t of segment b at position
// pos_base + (t - off[b]); B, S are then 1 and the packed row count.
hipError_t launch_rope(void* q, void* k, bool bf16, int B, int S, int Hq, int Hkv, int D,
                       int pos_base, const int32_t* pos_offsets, double theta, bool inverse,
                       const Segs* seg, hipStream_t st);

// q/k RMSNorm + RoPE (bwd = false: q_out/k_out = rotate(norm(q_in/k_in));
// bwd = true: q_out/k_out = input gradients from the output gradients gq/gk).
hipError_t launch_qk_norm_rope(const void* q_in, const void* k_in, const void* gq,
                               const void* gk, void* q_out, void* k_out, const float* w_q,
                               const float* w_k, bool bf16_, int B, int S, int Hq, int Hkv,
                               int D, float eps, int pos_base, const int32_t* pos_offsets,
                               double theta, bool bwd, hipStream_t st);

// Adam on n f32 elements (n % 4 == 0), the first `frozen` left unchanged;
// xb (nullable) receives the bf16 rounding of every updated element.
hipError_t launch_adam_rows(float* x, const float* g, float* m, float* v, void* xb, size_t n,
                            size_t frozen, int step, double lr, double b1, double b2,
                            double eps, hipStream_t st);

// A composed prefix: the parts' row counts, frozen rows, row offsets in the
// composition and device pointers (passed by value to the kernels).
constexpr int kMaxParts = 64;
struct PartTable {
  int n;
  int rows[kMaxParts];
  int frozen[kMaxParts];
  int off[kMaxParts + 1];
  const void* k[kMaxParts];
  const void* v[kMaxParts];
};
// Concatenate the parts' K and V rows (row_elems = Hkv * D elements each,
// f32 or bf16) into k_out/v_out (bf16, or f32 from f32).
hipError_t launch_compose_rows(const PartTable& t, bool src_bf16, bool dst_bf16, int row_elems,
                               void* k_out, void* v_out, hipStream_t st);
// Zero every part's frozen rows of the composed f32 gradients.
hipError_t launch_zero_frozen(const PartTable& t, int row_elems, float* dk, float* dv,
                              hipStream_t st);

struct CacheDims {
  int n_seqs, Hkv, D, page, max_pages, n_pages;
  void* k_pages;
  void* v_pages;
  const int32_t* block_table;
  int32_t* seq_lens;
};
// Append rows [n_rows, Hkv, D] (f32 or bf16) at row `start` of `seq` and set
// the device seq_len of `seq` to start + n_rows.
hipError_t launch_cache_append(const CacheDims& c, int seq, int start, const void* k,
                               const void* v, bool src_bf16, int n_rows, hipStream_t st);
hipError_t launch_cache_set_len(const CacheDims& c, int seq, int len, hipStream_t st);

struct DecodePlan {
  int pages_per_split, max_splits;
  int chunks;          // workgroups per (sequence, kv head): query rows / 32
  int waves;           // > 0: waves per workgroup, splits merged on chip; 0: merge kernel
  long long grid;      // decode workgroups
  size_t part_bytes;   // workspace for split partials (0 when merged on chip)
};
// kq query tokens per sequence: 1 for a decode step, more for a verify step
// (whose k_new/v_new rows, kq per sequence, are appended first).
DecodePlan plan_decode(const CacheDims& c, int Hq, int kq);
hipError_t launch_decode(const CacheDims& c, int Hq, int kq, float scale, const void* q,
                         const void* k_new, const void* v_new, void* out, void* ws,
                         hipStream_t st);

// Library-held decode scratch (allocation-free entry point): its size, and
// its device address on the current device (looked up on first use there).
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace cartattn
