// Embedding gather and RMSNorm.
//
// RMSNorm: xn = x / sqrt(mean(x^2) + eps) * g over the hidden axis, with the
// fp32 residual row x as input and the GEMM input type as output.  One wave
// per row; sums in fp32.  When the preceding residual GEMM was split over K,
// its nsplit fp32 partials are first added to x in split order (a fixed
// order, so the result does not depend on scheduling) and x is written back.
#pragma once
#include "common.hpp"

namespace phi {

struct NormArgs {
  const int32_t* ids;  // embed variant only
  const void* embed;   // [V][H] of the weight's float type
  float* x;            // [T][H] residual, fp32
  const void* gain;    // [H]
  void* xn;            // [T][H] output (AT)
  const float* part;   // [nsplit][T][H] partial sums to add to x first (nsplit > 0)
  int nsplit;
  int T, H, V;
  float eps;
};

// x[t] = embed[ids[t]] (widened to fp32), then xn[t] = rmsnorm(x[t]) * gain.
// An id outside [0, V) yields a NaN row in x and xn.
template <class ET, class AT>
__global__ __launch_bounds__(256) void phi_norm_embed_kernel(NormArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.T) return;
  const int id = a.ids[row];
  float* xr = a.x + (size_t)row * a.H;
  AT* xo = reinterpret_cast<AT*>(a.xn) + (size_t)row * a.H;
  const ET* g = reinterpret_cast<const ET*>(a.gain);
  if (id < 0 || id >= a.V) {
    const float nan = __builtin_nanf("");
    for (int c = lane * 4; c < a.H; c += 256) {
      vec4<float>::store(xr + c, f32x4{nan, nan, nan, nan});
      vec4<AT>::store(xo + c, f32x4{nan, nan, nan, nan});
    }
    return;
  }
  const ET* e = reinterpret_cast<const ET*>(a.embed) + (size_t)id * a.H;
  float ss = 0.f;
  for (int c = lane * 4; c < a.H; c += 256) {
    f32x4 v = vec4<ET>::load(e + c);
    vec4<float>::store(xr + c, v);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)a.H + a.eps);
  for (int c = lane * 4; c < a.H; c += 256) {
    f32x4 v = vec4<ET>::load(e + c);
    f32x4 gv = vec4<ET>::load(g + c);
    vec4<AT>::store(xo + c, v * r * gv);
  }
}

// x[t] += sum_s part[s][t] (when nsplit > 0); xn[t] = rmsnorm(x[t]) * gain.
template <class ET, class AT>
__global__ __launch_bounds__(256) void phi_norm_rms_kernel(NormArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.T) return;
  float* xr = a.x + (size_t)row * a.H;
  AT* xo = reinterpret_cast<AT*>(a.xn) + (size_t)row * a.H;
  const ET* g = reinterpret_cast<const ET*>(a.gain);
  const size_t plane = (size_t)a.T * a.H;
  float ss = 0.f;
  for (int c = lane * 4; c < a.H; c += 256) {
    f32x4 v = vec4<float>::load(xr + c);
    if (a.nsplit > 0) {
      for (int sp = 0; sp < a.nsplit; ++sp) v += vec4<float>::load(a.part + sp * plane + (size_t)row * a.H + c);
      vec4<float>::store(xr + c, v);
    }
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)a.H + a.eps);
  for (int c = lane * 4; c < a.H; c += 256) {
    f32x4 v = vec4<float>::load(xr + c);
    f32x4 gv = vec4<ET>::load(g + c);
    vec4<AT>::store(xo + c, v * r * gv);
  }
}

}  // namespace phi
