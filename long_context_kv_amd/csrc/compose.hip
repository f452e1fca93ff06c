// Composed cartridges: the concatenation of several parts' rows into the
// one prefix buffer the attention kernels read, and the zeroing of every
// part's frozen rows in the composed gradient.
//
// Source: "Cartridges: trained KV-prefix corpus compression", section
// "Composition": parts compose by concatenation (part 0's rows first), the
// composed prefix is one concatenation per layer, so the attention backward
// routes gradients into every part, and every part's sink stays frozen.
//
// The concatenation is where f32 master rows become the bf16 MFMA operands:
// it reads each part once and writes the composed bf16 (or f32) rows, the
// same bytes the single-cartridge path spends on its bf16 copy, so a
// composed layer costs no extra pass. HBM-bound: 16- or 32-byte accesses,
// one grid row of workgroups per part.
#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace cartattn {

namespace {

template <typename TS, typename TD>
__global__ __launch_bounds__(256) void compose_rows_kernel(PartTable t, size_t row8, TD* k_out,
                                                           TD* v_out) {
  const int part = blockIdx.y;
  const size_t n8 = (size_t)t.rows[part] * row8;   // 8-element chunks of this part
  const size_t base = (size_t)t.off[part] * row8;
  const TS* k = reinterpret_cast<const TS*>(t.k[part]);
  const TS* v = reinterpret_cast<const TS*>(t.v[part]);
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    float x[8];
    load8<TS>(k + 8 * i, x);
    store8<TD>(k_out + 8 * (base + i), x);
    load8<TS>(v + 8 * i, x);
    store8<TD>(v_out + 8 * (base + i), x);
  }
}

__global__ __launch_bounds__(256) void zero_frozen_kernel(PartTable t, size_t row4, f32x4* dk,
                                                          f32x4* dv) {
  const int part = blockIdx.y;
  const size_t n4 = (size_t)t.frozen[part] * row4;
  const size_t base = (size_t)t.off[part] * row4;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * blockDim.x) {
    dk[base + i] = z;
    dv[base + i] = z;
  }
}

unsigned grid_x(size_t work) {
  size_t b = (work + 255) / 256;
  if (b > 1024) b = 1024;
  return (unsigned)(b ? b : 1);
}

}  // namespace

hipError_t launch_compose_rows(const PartTable& t, bool src_bf16, bool dst_bf16, int row_elems,
                               void* k_out, void* v_out, hipStream_t st) {
  int max_rows = 0;
  for (int i = 0; i < t.n; ++i) max_rows = t.rows[i] > max_rows ? t.rows[i] : max_rows;
  if (max_rows == 0) return hipSuccess;
  const size_t row8 = (size_t)row_elems / 8;
  const dim3 grid(grid_x((size_t)max_rows * row8), t.n);
  if (src_bf16 && dst_bf16)
    CART_LAUNCH("compose_rows", (compose_rows_kernel<bf16, bf16>), grid, 256, 0, st, t, row8,
                reinterpret_cast<bf16*>(k_out), reinterpret_cast<bf16*>(v_out));
  else if (!src_bf16 && dst_bf16)
    CART_LAUNCH("compose_rows", (compose_rows_kernel<float, bf16>), grid, 256, 0, st, t, row8,
                reinterpret_cast<bf16*>(k_out), reinterpret_cast<bf16*>(v_out));
  else if (!src_bf16 && !dst_bf16)
    CART_LAUNCH("compose_rows", (compose_rows_kernel<float, float>), grid, 256, 0, st, t, row8,
                reinterpret_cast<float*>(k_out), reinterpret_cast<float*>(v_out));
  else
    return hipErrorInvalidValue;   // bf16 -> f32 is refused on the host
  return hipGetLastError();
}

hipError_t launch_zero_frozen(const PartTable& t, int row_elems, float* dk, float* dv,
                              hipStream_t st) {
  int max_f = 0;
  for (int i = 0; i < t.n; ++i) max_f = t.frozen[i] > max_f ? t.frozen[i] : max_f;
  if (max_f == 0) return hipSuccess;
  const size_t row4 = (size_t)row_elems / 4;
  const dim3 grid(grid_x((size_t)max_f * row4), t.n);
  CART_LAUNCH("zero_frozen", (zero_frozen_kernel), grid, 256, 0, st, t, row4,
              reinterpret_cast<f32x4*>(dk), reinterpret_cast<f32x4*>(dv));
  return hipGetLastError();
}

}  // namespace cartattn
