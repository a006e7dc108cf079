// Embedding gather and RMSNorm.
//
// RMSNorm: xn = x / sqrt(mean(x^2) + eps) * g over the hidden axis, with the
// fp32 residual row x as input and the GEMM input type as output.  One
// workgroup per row; sums in fp32.  When the preceding residual GEMM was split over K,
// its nsplit binary16 partials are first added to x in split order (a fixed
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
  const f16* part;     // [nsplit][T][H] binary16 partial sums to add to x first (nsplit > 0)
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

// One workgroup per row; thread t holds the CH float4 chunks at columns
// 4 (t + 256 i), i < CH = ceil(H / 1024), in registers between the sum of
// squares and the scaling.  Only the last chunk can pass the row's end (then
// the thread loads column 0 and discards it), so every load of a thread is
// issued before the first use: the chunks of up to four splits are in flight
// together instead of one load per round trip.
// EMBED: x[t] = embed[ids[t]] (an id outside [0, V) gives a NaN row).
// else:  x[t] += sum_s part[s][t] in split order for nsplit > 0 (then written back).
// Both: xn[t] = x[t] / sqrt(mean(x[t]^2) + eps) * gain.
// NSP = 5: exactly five split-K partial planes, all 15 of a thread's partial
// loads issued before the first add (one memory round trip; the residual
// GEMMs' split count at 512 tokens: norm 0.552 -> 0.525 ms per forward at
// 1x512, logits bitwise unchanged); NSP = -1: any count (a.nsplit), at
// most four splits' loads in flight; NSP = 0: no partials.  Separate
// instances, so the partial registers of one do not cost the others
// occupancy.
template <class ET, class AT, bool EMBED, int CH, int NSP = -1>
__global__ __launch_bounds__(kNormThreads) void phi_norm_kernel(NormArgs a) {
  static_assert(CH >= 1 && CH <= kNormMaxChunks, "chunks per thread");
  __shared__ float red[4];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  float* xr = a.x + (size_t)row * a.H;
  AT* xo = reinterpret_cast<AT*>(a.xn) + (size_t)row * a.H;
  const ET* g = reinterpret_cast<const ET*>(a.gain);
  int col[CH];    // column of chunk i, clamped to 0 past the row's end
  bool ok[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = (tid + i * kNormThreads) * 4;
    ok[i] = c < a.H;
    col[i] = ok[i] ? c : 0;
  }
  f32x4 v[CH];
  if constexpr (EMBED) {
    const int id = a.ids[row];
    const bool bad = id < 0 || id >= a.V;
    const ET* e = reinterpret_cast<const ET*>(a.embed) + (size_t)(bad ? 0 : id) * a.H;
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      v[i] = vec4<ET>::load(e + col[i]);
      if (bad) v[i] = f32x4{nan, nan, nan, nan};
    }
#pragma unroll
    for (int i = 0; i < CH; ++i)
      if (ok[i]) vec4<float>::store(xr + col[i], v[i]);
  } else {
#pragma unroll
    for (int i = 0; i < CH; ++i) v[i] = vec4<float>::load(xr + col[i]);
    if (NSP != 0 && a.nsplit > 0) {
      const f16* pr = a.part + (size_t)row * a.H;
      const size_t plane = (size_t)a.T * a.H;
      if constexpr (NSP > 0) {
        f32x4 pv[NSP > 0 ? NSP : 1][CH];
#pragma unroll
        for (int sp = 0; sp < NSP; ++sp)
#pragma unroll
          for (int i = 0; i < CH; ++i) pv[sp][i] = vec4<f16>::load(pr + sp * plane + col[i]);
#pragma unroll
        for (int sp = 0; sp < NSP; ++sp)
#pragma unroll
          for (int i = 0; i < CH; ++i) v[i] += pv[sp][i];
      } else {
#pragma unroll 4
        for (int sp = 0; sp < a.nsplit; ++sp)
#pragma unroll
          for (int i = 0; i < CH; ++i) v[i] += vec4<f16>::load(pr + sp * plane + col[i]);
      }
#pragma unroll
      for (int i = 0; i < CH; ++i)
        if (ok[i]) vec4<float>::store(xr + col[i], v[i]);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CH; ++i)
    if (ok[i]) ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)a.H + a.eps);
#pragma unroll
  for (int i = 0; i < CH; ++i)
    if (ok[i]) vec4<AT>::store(xo + col[i], v[i] * r * vec4<ET>::load(g + col[i]));
}

}  // namespace phi
