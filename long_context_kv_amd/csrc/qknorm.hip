// The step before the attention kernels: per-head RMS normalization of the
// real-token queries and keys followed by RoPE, fused in one pass, and its
// backward (the RoPE adjoint followed by the normalization's input gradient).
//
// Source: "Cartridges: trained KV-prefix corpus compression", section
// "Semantics (pinned to the reference implementation)": cartridge keys live
// in the KV-cache space, i.e. after the q/k normalization and after RoPE, so
// the real tokens' queries and keys must arrive at the attention in that same
// space: normalized, then rotated at positions p, p+1, ....
//
// The normalization is the Qwen3 q/k RMSNorm over one head row of d
// elements with a learned weight w[d]:
//   y = x * w / sqrt(mean(x^2) + eps)
// then (k, k + d/2) pairs rotate by pos * theta^(-2k/d) as cart_rope_tokens
// does. Backward, for the gradient g of the rotated output:
//   dy = R(-angle) g,  r = 1 / sqrt(mean(x^2) + eps),
//   dx = r w dy - (r^3 / d) x sum_j(w_j dy_j x_j).
// The weights are frozen (the cartridge rows are the only trainable
// parameters), so no weight gradient is formed.
//
// HBM-bound: one workgroup per token; a head row is spread over d/8 lanes
// (4 pairs each), its sums taken by DPP adds inside those lanes; the cos/sin
// table of the token is built once in LDS and reused over its heads. The
// arithmetic is f32 and every output is rounded once to the tensor's dtype.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace cartattn {

namespace {

struct NormRopeArgs {
  const void* q_in;
  const void* k_in;
  const void* gq;       // backward: gradient of the rotated output
  const void* gk;
  void* q_out;          // forward output, or the backward's input gradient
  void* k_out;
  const float* w_q;
  const float* w_k;
  const int32_t* pos_offsets;
  int S, Hq, Hkv, pos_base;
  float eps;
  double inv_freq[64];  // theta^(-2k/d), k < d/2
};

template <typename T> struct V4T;
template <> struct V4T<bf16> { typedef bf16x4 type; };
template <> struct V4T<float> { typedef f32x4 type; };

template <typename T, int D, bool BWD>
__global__ __launch_bounds__(256) void norm_rope_kernel(NormRopeArgs a) {
  constexpr int HALF = D / 2;
  constexpr int TPR = HALF / 4;      // lanes per head row (4 pairs each)
  constexpr int RPP = 256 / TPR;     // head rows per pass
  typedef typename V4T<T>::type V4;
  __shared__ float cs[HALF], sn[HALF];
  const int tok = blockIdx.x;        // b * S + i
  const int b = tok / a.S;
  const int i = tok % a.S;
  const int k4 = 4 * (threadIdx.x % TPR);
  const int hsub = threadIdx.x / TPR;
  if (threadIdx.x < HALF) {
    const long long pos = (long long)a.pos_base + (a.pos_offsets ? a.pos_offsets[b] : 0) + i;
    const double ang = (double)pos * a.inv_freq[threadIdx.x];
    constexpr double kTwoPi = 6.283185307179586476925286766559;
    const double r = ang - kTwoPi * rint(ang * (1.0 / kTwoPi));
    float sf, cf;
    sincosf((float)r, &sf, &cf);
    cs[threadIdx.x] = cf;
    sn[threadIdx.x] = sf;
  }
  __syncthreads();
  float c[4], s[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) { c[e] = cs[k4 + e]; s[e] = sn[k4 + e]; }
  const float inv_d = 1.0f / (float)D;

  auto row = [&](const T* x, const T* g, T* out, const float* w) {
    const V4 xl = *reinterpret_cast<const V4*>(x + k4);
    const V4 xh = *reinterpret_cast<const V4*>(x + HALF + k4);
    const f32x4 wl = *reinterpret_cast<const f32x4*>(w + k4);
    const f32x4 wh = *reinterpret_cast<const f32x4*>(w + HALF + k4);
    float lo[4], hi[4], ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = to_f32(xl[e]);
      hi[e] = to_f32(xh[e]);
      ss = fmaf(lo[e], lo[e], ss);
      ss = fmaf(hi[e], hi[e], ss);
    }
    V4 ol, oh;
    if constexpr (!BWD) {
      ss = row_sum<TPR>(ss);
      const float r = 1.0f / sqrtf(fmaf(ss, inv_d, a.eps));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float yl = lo[e] * r * wl[e];
        const float yh = hi[e] * r * wh[e];
        ol[e] = from_f32<T>(yl * c[e] - yh * s[e]);
        oh[e] = from_f32<T>(yh * c[e] + yl * s[e]);
      }
    } else {
      const V4 gl = *reinterpret_cast<const V4*>(g + k4);
      const V4 gh = *reinterpret_cast<const V4*>(g + HALF + k4);
      float dyl[4], dyh[4], t = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a0 = to_f32(gl[e]), a1 = to_f32(gh[e]);
        dyl[e] = a0 * c[e] + a1 * s[e];       // rotation by -angle
        dyh[e] = a1 * c[e] - a0 * s[e];
        t = fmaf(wl[e] * dyl[e], lo[e], t);
        t = fmaf(wh[e] * dyh[e], hi[e], t);
      }
      ss = row_sum<TPR>(ss);
      t = row_sum<TPR>(t);
      const float r = 1.0f / sqrtf(fmaf(ss, inv_d, a.eps));
      const float k3 = r * r * r * inv_d * t;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ol[e] = from_f32<T>(r * wl[e] * dyl[e] - k3 * lo[e]);
        oh[e] = from_f32<T>(r * wh[e] * dyh[e] - k3 * hi[e]);
      }
    }
    *reinterpret_cast<V4*>(out + k4) = ol;
    *reinterpret_cast<V4*>(out + HALF + k4) = oh;
  };

  const size_t qrow = (size_t)tok * a.Hq * D;
  for (int h = hsub; h < a.Hq; h += RPP) {
    const size_t o = qrow + (size_t)h * D;
    row(reinterpret_cast<const T*>(a.q_in) + o, BWD ? reinterpret_cast<const T*>(a.gq) + o : nullptr,
        reinterpret_cast<T*>(a.q_out) + o, a.w_q);
  }
  if (a.k_in) {
    const size_t krow = (size_t)tok * a.Hkv * D;
    for (int h = hsub; h < a.Hkv; h += RPP) {
      const size_t o = krow + (size_t)h * D;
      row(reinterpret_cast<const T*>(a.k_in) + o,
          BWD ? reinterpret_cast<const T*>(a.gk) + o : nullptr,
          reinterpret_cast<T*>(a.k_out) + o, a.w_k);
    }
  }
}

template <typename T, int D>
hipError_t launch_nr(const NormRopeArgs& a, int tokens, bool bwd, hipStream_t st) {
  if (bwd)
    CART_LAUNCH("qk_norm_rope_bwd", (norm_rope_kernel<T, D, true>), tokens, 256, 0, st, a);
  else
    CART_LAUNCH("qk_norm_rope", (norm_rope_kernel<T, D, false>), tokens, 256, 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qk_norm_rope(const void* q_in, const void* k_in, const void* gq,
                               const void* gk, void* q_out, void* k_out, const float* w_q,
                               const float* w_k, bool bf16_, int B, int S, int Hq, int Hkv,
                               int D, float eps, int pos_base, const int32_t* pos_offsets,
                               double theta, bool bwd, hipStream_t st) {
  NormRopeArgs a{};
  a.q_in = q_in; a.k_in = k_in; a.gq = gq; a.gk = gk; a.q_out = q_out; a.k_out = k_out;
  a.w_q = w_q; a.w_k = w_k; a.pos_offsets = pos_offsets;
  a.S = S; a.Hq = Hq; a.Hkv = Hkv; a.pos_base = pos_base; a.eps = eps;
  for (int kk = 0; kk < D / 2; ++kk)
    a.inv_freq[kk] = exp(-2.0 * (double)kk / (double)D * log(theta));
  const int tokens = B * S;
  if (bf16_)
    return D == 128 ? launch_nr<bf16, 128>(a, tokens, bwd, st) : launch_nr<bf16, 64>(a, tokens, bwd, st);
  return D == 128 ? launch_nr<float, 128>(a, tokens, bwd, st) : launch_nr<float, 64>(a, tokens, bwd, st);
}

}  // namespace cartattn
