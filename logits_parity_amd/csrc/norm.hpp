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

constexpr int kNormThreads = 256;
constexpr int kNormMaxChunks = 8;  // hidden <= 8 * 4 * 256 = 8192

// Sum over the workgroup (4 waves) via LDS.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// One workgroup per row, up to kNormMaxChunks float4 chunks per thread held in
// registers between the sum of squares and the scaling.
// EMBED: x[t] = embed[ids[t]] (an id outside [0, V) gives a NaN row).
// else:  x[t] += sum_s part[s][t] for nsplit > 0 (then written back).
// Both: xn[t] = x[t] / sqrt(mean(x[t]^2) + eps) * gain.
template <class ET, class AT, bool EMBED>
__global__ __launch_bounds__(kNormThreads) void phi_norm_kernel(NormArgs a) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  float* xr = a.x + (size_t)row * a.H;
  AT* xo = reinterpret_cast<AT*>(a.xn) + (size_t)row * a.H;
  const ET* g = reinterpret_cast<const ET*>(a.gain);
  f32x4 v[kNormMaxChunks];
  float ss = 0.f;
  if constexpr (EMBED) {
    const int id = a.ids[row];
    const bool bad = id < 0 || id >= a.V;
    const ET* e = reinterpret_cast<const ET*>(a.embed) + (size_t)(bad ? 0 : id) * a.H;
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int i = 0; i < kNormMaxChunks; ++i) {
      const int c = (tid + i * kNormThreads) * 4;
      if (c >= a.H) break;
      v[i] = bad ? f32x4{nan, nan, nan, nan} : vec4<ET>::load(e + c);
      vec4<float>::store(xr + c, v[i]);
      ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
    }
  } else {
    const size_t plane = (size_t)a.T * a.H;
#pragma unroll
    for (int i = 0; i < kNormMaxChunks; ++i) {
      const int c = (tid + i * kNormThreads) * 4;
      if (c >= a.H) break;
      v[i] = vec4<float>::load(xr + c);
      if (a.nsplit > 0) {
        for (int sp = 0; sp < a.nsplit; ++sp)
          v[i] += vec4<float>::load(a.part + sp * plane + (size_t)row * a.H + c);
        vec4<float>::store(xr + c, v[i]);
      }
      ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
    }
  }
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)a.H + a.eps);
#pragma unroll
  for (int i = 0; i < kNormMaxChunks; ++i) {
    const int c = (tid + i * kNormThreads) * 4;
    if (c >= a.H) break;
    vec4<AT>::store(xo + c, v[i] * r * vec4<ET>::load(g + c));
  }
}

}  // namespace phi
