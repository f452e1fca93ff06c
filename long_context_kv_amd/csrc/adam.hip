// The step after the attention kernels: Adam on the trainable cartridge
// rows, with the bf16 copy that the next step's attention reads written in
// the same pass.
//
// Source: "Cartridges: trained KV-prefix corpus compression", section
// "Semantics (pinned to the reference implementation)": the rows below
// frozen_prefix are constants, the rest are the only trainable parameters,
// optimized by Adam without weight decay or schedule (lr 2e-2); section
// "Learning rate vs batch size (measured)": lr 2e-3 at small batches.
//
// Per element of a trainable row, at step t >= 1 (the usual Adam with bias
// correction):
//   m = b1 m + (1 - b1) g,   v = b2 v + (1 - b2) g^2,
//   x = x - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps).
// Frozen rows keep x, m and v. The optional bf16 output receives every row
// of the updated x rounded to nearest even (frozen rows included), so a
// training loop can hand it to cart_attn_fwd / cart_attn_bwd as bf16 rows
// and skip their own cast of the f32 rows.
//
// HBM-bound elementwise pass: per element 16 bytes read (x, g, m, v) and
// 12 written (x, m, v), plus 2 for the bf16 copy; 16-byte accesses.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace cartattn {

namespace {

struct AdamArgs {
  f32x4* x;
  const f32x4* g;
  f32x4* m;
  f32x4* v;
  bf16x4* xb;          // may be null
  size_t n4;           // 4-element groups in the tensor
  size_t frozen4;      // 4-element groups of the frozen rows (a prefix)
  // (1 - b1), (1 - b2) formed in double on the host and rounded once, so
  // that e.g. b2 = 0.999 weights g^2 by the f32 nearest to 0.001
  float lr_c, b1, b2, omb1, omb2, eps, inv_sqrt_bc2;
};

__global__ __launch_bounds__(256) void adam_rows_kernel(AdamArgs a) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.n4; i += stride) {
    f32x4 x = a.x[i];
    if (i >= a.frozen4) {
      const f32x4 g = a.g[i];
      f32x4 m = a.m[i];
      f32x4 v = a.v[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m[e] = fmaf(a.b1, m[e], a.omb1 * g[e]);
        v[e] = fmaf(a.b2, v[e], a.omb2 * g[e] * g[e]);
        const float den = sqrtf(v[e]) * a.inv_sqrt_bc2 + a.eps;
        x[e] = x[e] - a.lr_c * (m[e] / den);
      }
      a.m[i] = m;
      a.v[i] = v;
      a.x[i] = x;
    }
    if (a.xb) {
      bf16x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (bf16)x[e];
      a.xb[i] = o;
    }
  }
}

}  // namespace

hipError_t launch_adam_rows(float* x, const float* g, float* m, float* v, void* xb, size_t n,
                            size_t frozen, int step, double lr, double b1, double b2, double eps,
                            hipStream_t st) {
  AdamArgs a{};
  a.x = reinterpret_cast<f32x4*>(x);
  a.g = reinterpret_cast<const f32x4*>(g);
  a.m = reinterpret_cast<f32x4*>(m);
  a.v = reinterpret_cast<f32x4*>(v);
  a.xb = reinterpret_cast<bf16x4*>(xb);
  a.n4 = n / 4;
  a.frozen4 = frozen / 4;
  // bias corrections in double on the host
  const double bc1 = 1.0 - pow(b1, (double)step);
  const double bc2 = 1.0 - pow(b2, (double)step);
  a.lr_c = (float)(lr / bc1);
  a.inv_sqrt_bc2 = (float)(1.0 / sqrt(bc2));
  a.b1 = (float)b1; a.b2 = (float)b2; a.eps = (float)eps;
  a.omb1 = (float)(1.0 - b1);
  a.omb2 = (float)(1.0 - b2);
  if (a.n4 == 0) return hipSuccess;
  size_t blocks = (a.n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  CART_LAUNCH("adam_rows", (adam_rows_kernel), (unsigned)blocks, 256, 0, st, a);
  return hipGetLastError();
}

}  // namespace cartattn
