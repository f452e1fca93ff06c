// RoPE on the real-token queries and keys, in place.
//
// Source: "Cartridges: trained KV-prefix corpus compression", section
// "Semantics (pinned to the reference implementation)": cartridge keys are
// rotated at positions 0..p-1 once and never again; real tokens sit at
// positions p, p+1, .... "RIG minimal cognition engine implementation
// hand-off", section 5: a shifted base position silently corrupts attention.
//
// Pairs (k, k + d/2) rotate by pos * theta^(-2k/d). The angle and its cosine
// and sine are computed in double precision (positions reach 2e4, where a
// float angle would be off by ~1e-3 rad); the rotation itself is f32 and the
// result is rounded to the tensor's dtype. The kernel is HBM-bound: one
// workgroup per token, lanes over k so each row half is read coalesced, and
// each lane computes its cos/sin once and reuses it for every head.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace cartattn {

namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_kernel(T* __restrict__ q, T* __restrict__ k,
                                                   int S, int Hq, int Hkv, int pos_base,
                                                   const int32_t* __restrict__ pos_offsets,
                                                   double log_theta, float sign) {
  constexpr int HALF = D / 2;
  constexpr int HPP = 256 / HALF;   // heads handled per pass
  const int tok = blockIdx.x;       // b * S + i
  const int b = tok / S;
  const int i = tok % S;
  const int kk = threadIdx.x % HALF;
  const int hsub = threadIdx.x / HALF;
  const long long pos = (long long)pos_base + (pos_offsets ? pos_offsets[b] : 0) + i;
  const double inv_freq = exp(-2.0 * (double)kk / (double)D * log_theta);
  double sd, cd;
  sincos((double)pos * inv_freq, &sd, &cd);
  const float c = (float)cd;
  const float s = (float)sd * sign;
  T* qr = q + (size_t)tok * Hq * D;
  for (int h = hsub; h < Hq; h += HPP) {
    T* x = qr + (size_t)h * D;
    const float lo = to_f32(x[kk]);
    const float hi = to_f32(x[kk + HALF]);
    x[kk] = from_f32<T>(lo * c - hi * s);
    x[kk + HALF] = from_f32<T>(hi * c + lo * s);
  }
  if (k) {
    T* kr = k + (size_t)tok * Hkv * D;
    for (int h = hsub; h < Hkv; h += HPP) {
      T* x = kr + (size_t)h * D;
      const float lo = to_f32(x[kk]);
      const float hi = to_f32(x[kk + HALF]);
      x[kk] = from_f32<T>(lo * c - hi * s);
      x[kk + HALF] = from_f32<T>(hi * c + lo * s);
    }
  }
}

template <typename T, int D>
hipError_t launch_t(void* q, void* k, int B, int S, int Hq, int Hkv, int pos_base,
                    const int32_t* pos_offsets, double theta, bool inverse, hipStream_t st) {
  CART_TIMED("rope", st,
             rope_kernel<T, D><<<B * S, 256, 0, st>>>(
                 reinterpret_cast<T*>(q), reinterpret_cast<T*>(k), S, Hq, Hkv, pos_base,
                 pos_offsets, log(theta), inverse ? -1.f : 1.f));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(void* q, void* k, bool bf16_, int B, int S, int Hq, int Hkv, int D,
                       int pos_base, const int32_t* pos_offsets, double theta, bool inverse,
                       hipStream_t st) {
  if (bf16_)
    return D == 128 ? launch_t<bf16, 128>(q, k, B, S, Hq, Hkv, pos_base, pos_offsets, theta, inverse, st)
                    : launch_t<bf16, 64>(q, k, B, S, Hq, Hkv, pos_base, pos_offsets, theta, inverse, st);
  return D == 128 ? launch_t<float, 128>(q, k, B, S, Hq, Hkv, pos_base, pos_offsets, theta, inverse, st)
                  : launch_t<float, 64>(q, k, B, S, Hq, Hkv, pos_base, pos_offsets, theta, inverse, st);
}

}  // namespace cartattn
