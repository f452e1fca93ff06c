// RoPE on the real-token queries and keys, in place.
//
// Source: "Cartridges: trained KV-prefix corpus compression", section
// "Semantics (pinned to the reference implementation)": cartridge keys are
// rotated at positions 0..p-1 once and never again; real tokens sit at
// positions p, p+1, .... "RIG minimal cognition engine implementation
// hand-off", section 5: a shifted base position silently corrupts attention.
//
// Pairs (k, k + d/2) rotate by pos * theta^(-2k/d). The frequencies are
// computed on the host in double precision; on the device the angle is formed
// and reduced modulo 2 pi in double precision (positions reach 2e4, where a
// float angle would be off by ~1e-3 rad), and the cosine and sine of the
// reduced angle (|r| <= pi) are f32. The rotation itself is f32 and the result
// is rounded to the tensor's dtype. The kernel is HBM-bound: one workgroup per
// token; every lane loads 4 consecutive pairs of one head row per pass (8- or
// 16-byte loads of each row half), the first pass before the token's first d/2
// lanes put its cos/sin table in LDS.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace cartattn {

namespace {

struct RopeFreq {
  double inv_freq[64];   // theta^(-2k/d), k < d/2
};

template <typename T> struct Vec4;
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<float> { typedef f32x4 type; };

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_kernel(T* __restrict__ q, T* __restrict__ k,
                                                   int S, int Hq, int Hkv, int pos_base,
                                                   const int32_t* __restrict__ pos_offsets,
                                                   RopeFreq fr, float sign, Segs seg) {
  constexpr int HALF = D / 2;
  constexpr int TPR = HALF / 4;      // threads per head row (4 pairs each)
  constexpr int RPP = 256 / TPR;     // head rows per pass
  typedef typename Vec4<T>::type V4;
  __shared__ float cs[HALF], sn[HALF];
  const int tok = blockIdx.x;        // b * S + i, or the packed row
  int b = tok / S;
  int i = tok % S;
  if (seg.packed) {
    // the segment holding the row (off[] ascending): positions restart at
    // pos_base in every segment
    int lo = 0, hi = seg.packed;     // packed = the number of segments
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (seg.off[mid] <= tok) lo = mid; else hi = mid;
    }
    b = lo;
    i = tok - seg.off[lo];
  }
  const int k4 = 4 * (threadIdx.x % TPR);
  const int hsub = threadIdx.x / TPR;
  T* qr = q + (size_t)tok * Hq * D;
  T* kr = k ? k + (size_t)tok * Hkv * D : nullptr;
  // the first pass's rows are loaded before the table is built, so their
  // latency overlaps the angle reduction
  const bool q0 = hsub < Hq;
  const bool k0 = kr && hsub < Hkv;
  V4 qlo{}, qhi{}, klo{}, khi{};
  if (q0) {
    qlo = *reinterpret_cast<const V4*>(qr + (size_t)hsub * D + k4);
    qhi = *reinterpret_cast<const V4*>(qr + (size_t)hsub * D + HALF + k4);
  }
  if (k0) {
    klo = *reinterpret_cast<const V4*>(kr + (size_t)hsub * D + k4);
    khi = *reinterpret_cast<const V4*>(kr + (size_t)hsub * D + HALF + k4);
  }
  if (threadIdx.x < HALF) {
    const long long pos =
        (long long)pos_base + (pos_offsets && !seg.packed ? pos_offsets[b] : 0) + i;
    const double ang = (double)pos * fr.inv_freq[threadIdx.x];
    constexpr double kTwoPi = 6.283185307179586476925286766559;
    const double r = ang - kTwoPi * rint(ang * (1.0 / kTwoPi));
    float sf, cf;
    sincosf((float)r, &sf, &cf);
    cs[threadIdx.x] = cf;
    sn[threadIdx.x] = sf * sign;
  }
  __syncthreads();
  float c[4], s_[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) { c[e] = cs[k4 + e]; s_[e] = sn[k4 + e]; }
  auto rot_store = [&](T* x, const V4& lo, const V4& hi) {
    V4 ol, oh;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float l = to_f32(lo[e]), h = to_f32(hi[e]);
      ol[e] = from_f32<T>(l * c[e] - h * s_[e]);
      oh[e] = from_f32<T>(h * c[e] + l * s_[e]);
    }
    *reinterpret_cast<V4*>(x + k4) = ol;
    *reinterpret_cast<V4*>(x + HALF + k4) = oh;
  };
  auto rot = [&](T* x) {
    rot_store(x, *reinterpret_cast<const V4*>(x + k4), *reinterpret_cast<const V4*>(x + HALF + k4));
  };
  if (q0) rot_store(qr + (size_t)hsub * D, qlo, qhi);
  if (k0) rot_store(kr + (size_t)hsub * D, klo, khi);
  for (int h = hsub + RPP; h < Hq; h += RPP) rot(qr + (size_t)h * D);
  if (kr)
    for (int h = hsub + RPP; h < Hkv; h += RPP) rot(kr + (size_t)h * D);
}

template <typename T, int D>
hipError_t launch_t(void* q, void* k, int B, int S, int Hq, int Hkv, int pos_base,
                    const int32_t* pos_offsets, double theta, bool inverse, const Segs& seg,
                    hipStream_t st) {
  RopeFreq fr{};
  for (int kk = 0; kk < D / 2; ++kk) fr.inv_freq[kk] = exp(-2.0 * (double)kk / (double)D * log(theta));
  CART_LAUNCH("rope", (rope_kernel<T, D>), B * S, 256, 0, st, reinterpret_cast<T*>(q),
              reinterpret_cast<T*>(k), S, Hq, Hkv, pos_base, pos_offsets, fr, inverse ? -1.f : 1.f,
              seg);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(void* q, void* k, bool bf16_, int B, int S, int Hq, int Hkv, int D,
                       int pos_base, const int32_t* pos_offsets, double theta, bool inverse,
                       const Segs* seg, hipStream_t st) {
  Segs sg{};
  if (seg) sg = *seg;
  if (bf16_)
    return D == 128 ? launch_t<bf16, 128>(q, k, B, S, Hq, Hkv, pos_base, pos_offsets, theta, inverse, sg, st)
                    : launch_t<bf16, 64>(q, k, B, S, Hq, Hkv, pos_base, pos_offsets, theta, inverse, sg, st);
  return D == 128 ? launch_t<float, 128>(q, k, B, S, Hq, Hkv, pos_base, pos_offsets, theta, inverse, sg, st)
                  : launch_t<float, 64>(q, k, B, S, Hq, Hkv, pos_base, pos_offsets, theta, inverse, sg, st);
}

}  // namespace cartattn
