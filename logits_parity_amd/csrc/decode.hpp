// K16/V8 paged decode attention: binary16 keys, OCP E4M3FN values with one
// fp32 scale per KV head, 16-token pages, head_dim 128.
//
// Split kernel: a workgroup owns one (sequence, KV head, context split) and
// serves all G query heads of the GQA group from one read of each K/V page.
// Its 4 waves take pages round-robin.  Inside a wave, lane l owns token slot
// l / 4 of the page and dims 32 (l % 4) .. +31: it reads 64 contiguous bytes
// of K and 32 of V per page, forms partial q.k with v_dot2_f32_f16, and two
// xor-shuffles complete each dot product.  Every lane keeps its own online
// softmax state (max, sum, 32-wide output per head) over the tokens it has
// seen, so no cross-lane traffic is needed per page; states are merged by
// log-sum-exp once at the end (shuffles across the 16 token lanes, then LDS
// across the 4 waves).  E4M3 bytes are decoded with the hardware
// v_cvt_pk_f32_fp8; the per-head scale multiplies the final output once.
// The split writes (o unnormalised, max, sum) to the workspace.
//
// Merge kernel: o = sum_s o_s e^(m_s - m) / sum_s l_s e^(m_s - m) * scale.
#pragma once
#include "common.hpp"

namespace phi {

struct DecodeArgs {
  const f16* q;
  const f16* k_pool;
  const uint8_t* v_pool;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  float* part_o;   // [B][Hq][n_split][128]
  float* part_ml;  // [B][Hq][n_split][2]
  f16* out;        // [B][Hq][128]
  int B, Hq, Hkv, n_pages, max_pages, n_split, pages_per_split;
  float scale_log2;  // sm_scale * log2(e)
};

template <int G>
__global__ __launch_bounds__(256) void phi_decode_split_kernel(DecodeArgs a) {
  constexpr int D = 128, PG = 16;
  __shared__ float s_o[4][G][D];
  __shared__ float s_ml[4][G][2];
  __shared__ int s_err[4];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t = lane >> 2, dq = lane & 3;
  const int L = a.ctx_lens[b];
  bool err = L < 1 || L > a.max_pages * PG;
  const int np = err ? 0 : (L + PG - 1) / PG;
  const int p_begin = split * a.pages_per_split;
  const int p_end = min(np, p_begin + a.pages_per_split);

  f16x2 qv[G][16];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const f16* qp = a.q + ((size_t)b * a.Hq + g * G + h) * D + dq * 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x8 v = *reinterpret_cast<const f16x8*>(qp + i * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[h][i * 4 + e] = f16x2{v[2 * e], v[2 * e + 1]};
    }
  }
  float m[G], l[G], o[G][32];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -__builtin_inff();
    l[h] = 0.f;
#pragma unroll
    for (int d = 0; d < 32; ++d) o[h][d] = 0.f;
  }

  const int32_t* bt = a.block_table + (size_t)b * a.max_pages;
  for (int p = p_begin + w; p < p_end; p += 4) {
    const int phys = bt[p];
    if (phys < 0 || phys >= a.n_pages) { err = true; break; }
    const size_t off = ((size_t)(phys * a.Hkv + g) * PG + t) * D + dq * 32;
    const f16x8* kp = reinterpret_cast<const f16x8*>(a.k_pool + off);
    const i32x4* vp = reinterpret_cast<const i32x4*>(a.v_pool + off);
    f16x8 kv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kv[i] = kp[i];
    const i32x4 vb0 = vp[0], vb1 = vp[1];
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc = __builtin_amdgcn_fdot2(qv[h][i * 4 + e], f16x2{kv[i][2 * e], kv[i][2 * e + 1]}, acc, false);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      s[h] = acc * a.scale_log2;
    }
    if (p * PG + t < L) {
      float vf[32];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int wv = i < 4 ? vb0[i] : vb1[i - 4];
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(wv, false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(wv, true);
        vf[4 * i + 0] = lo[0];
        vf[4 * i + 1] = lo[1];
        vf[4 * i + 2] = hi[0];
        vf[4 * i + 3] = hi[1];
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], s[h]);
        const float al = exp2f(m[h] - mn), pp = exp2f(s[h] - mn);
        l[h] = l[h] * al + pp;
#pragma unroll
        for (int d = 0; d < 32; ++d) o[h][d] = fmaf(pp, vf[d], o[h][d] * al);
        m[h] = mn;
      }
    }
  }

  // merge the 16 token lanes of this wave (lane bits 2..5)
#pragma unroll
  for (int mask = 4; mask < 64; mask <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], mask), lo = __shfl_xor(l[h], mask);
      const float mn = fmaxf(m[h], mo);
      const float a1 = m[h] == -__builtin_inff() ? 0.f : exp2f(m[h] - mn);
      const float a2 = mo == -__builtin_inff() ? 0.f : exp2f(mo - mn);
      l[h] = l[h] * a1 + lo * a2;
#pragma unroll
      for (int d = 0; d < 32; ++d) o[h][d] = o[h][d] * a1 + __shfl_xor(o[h][d], mask) * a2;
      m[h] = mn;
    }
  }
  const int any_err = __any(err);
  if (lane < 4) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int d = 0; d < 32; ++d) s_o[w][h][dq * 32 + d] = o[h][d];
      if (lane == 0) { s_ml[w][h][0] = m[h]; s_ml[w][h][1] = l[h]; }
    }
  }
  if (lane == 0) s_err[w] = any_err;
  __syncthreads();
  const bool bad = s_err[0] | s_err[1] | s_err[2] | s_err[3];
  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D, d = idx - h * D;
    float mn = -__builtin_inff();
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) mn = fmaxf(mn, s_ml[ww][h][0]);
    float ls = 0.f, os = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float mw = s_ml[ww][h][0];
      const float f = mw == -__builtin_inff() ? 0.f : exp2f(mw - mn);
      ls += s_ml[ww][h][1] * f;
      os += s_o[ww][h][d] * f;
    }
    const size_t pi = ((size_t)(b * a.Hq + g * G + h) * a.n_split + split);
    a.part_o[pi * D + d] = os;
    if (d == 0) {
      a.part_ml[pi * 2 + 0] = mn;
      a.part_ml[pi * 2 + 1] = bad ? __builtin_nanf("") : ls;
    }
  }
}

__global__ __launch_bounds__(128) void phi_decode_merge_kernel(DecodeArgs a) {
  constexpr int D = 128;
  const int bh = blockIdx.x;  // b * Hq + h
  const int d = threadIdx.x;
  const int g = (bh % a.Hq) / (a.Hq / a.Hkv);
  const float* ml = a.part_ml + (size_t)bh * a.n_split * 2;
  const float* po = a.part_o + (size_t)bh * a.n_split * D;
  float mn = -__builtin_inff();
  for (int s = 0; s < a.n_split; ++s) mn = fmaxf(mn, ml[2 * s]);
  float ls = 0.f, os = 0.f;
  for (int s = 0; s < a.n_split; ++s) {
    const float ms = ml[2 * s];
    const float f = ms == -__builtin_inff() ? 0.f : exp2f(ms - mn);
    ls += ml[2 * s + 1] * f;  // NaN marks a sequence with bad inputs
    os += po[(size_t)s * D + d] * f;
  }
  const float r = (ls > 0.f) ? os / ls * a.v_scale[g] : __builtin_nanf("");
  a.out[(size_t)bh * D + d] = (f16)r;
}

}  // namespace phi
