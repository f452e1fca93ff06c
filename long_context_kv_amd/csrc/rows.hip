// Cartridge rows as MFMA operands: the f32 master rows (the trainable
// parameters) are rounded to bf16 (nearest even) into a workspace shadow that
// the bf16 attention kernels read. The concat itself stays virtual.
//
// Source: "Cartridges: trained KV-prefix corpus compression", section
// "Semantics (pinned to the reference implementation)": cartridge rows live in
// the space of KV-cache rows and are the only trainable parameters.
//
// HBM-bound elementwise pass: float4 in, 4 x bf16 out per thread.
#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace cartattn {

namespace {

__global__ __launch_bounds__(256) void rows_to_bf16_kernel(const float4* __restrict__ k,
                                                           const float4* __restrict__ v,
                                                           bf16x4* __restrict__ kb,
                                                           bf16x4* __restrict__ vb, size_t n4) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 a = k[i];
    const float4 b = v[i];
    bf16x4 x, y;
    x[0] = (bf16)a.x; x[1] = (bf16)a.y; x[2] = (bf16)a.z; x[3] = (bf16)a.w;
    y[0] = (bf16)b.x; y[1] = (bf16)b.y; y[2] = (bf16)b.z; y[3] = (bf16)b.w;
    kb[i] = x;
    vb[i] = y;
  }
}

}  // namespace

hipError_t launch_rows_to_bf16(const float* k, const float* v, bf16* kb, bf16* vb, size_t n,
                               hipStream_t st) {
  const size_t n4 = n / 4;   // n = rows x row elements, a multiple of 4
  if (n4 == 0) return hipSuccess;
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  CART_LAUNCH("rows_to_bf16", (rows_to_bf16_kernel), (unsigned)blocks, 256, 0, st,
              reinterpret_cast<const float4*>(k), reinterpret_cast<const float4*>(v),
              reinterpret_cast<bf16x4*>(kb), reinterpret_cast<bf16x4*>(vb), n4);
  return hipGetLastError();
}

}  // namespace cartattn
