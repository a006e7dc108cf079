// Causal softmax attention for the prefill, head_dim 96 (binary16 and float32)
// or 64 and 128 (binary16).
//
// binary16 path (split keys, MFMA): a workgroup owns 32 queries of one
// (sequence, head) and its 4 waves take the 64-key blocks that reach those
// queries round-robin, each keeping its own online-softmax state; the states
// are merged by log-sum-exp through LDS at the end.  Small workgroups and
// per-wave key ranges give thousands of short, independent chains, so with
// two workgroups per CU the memory latency of one wave's block hides behind
// the MFMA work of the others.
//
// Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_f16, so
// each lane holds one query's column: the running max, sum and output rescale
// are per-lane scalars, and only the max needs one exchange (lanes l, l + 32).
// The output is accumulated transposed too, O^T += V^T P^T, with P^T taken
// straight from the score registers.  A key block is 64 keys at head_dim 64
// and 96, and 32 at head_dim 128 (register budget).  Key rows enter the score MFMA with bits
// 2 and 3 of their index swapped; then the 8 score registers of each half of
// a lane hold 8 consecutive keys, and the matching V^T operand of the output
// MFMA is one 16-byte load.  Operands come from bounds-checked buffer loads
// over the (sequence, KV head) slice: key rows past the sequence read as zero,
// value columns past it are zeroed before use.  Softmax runs in base 2
// on fp32 scores; P enters the MFMA as binary16.  Query blocks are issued
// last-first so the longest rows start first.
//
// float32 path: one thread per query, online softmax over keys t <= s.
#pragma once
#include "common.hpp"

namespace phi {

struct AttnArgs {
  const void* q;   // [B][nh][S][D]
  const void* k;   // [B][nkv][S][D]
  const void* vt;  // [B][nkv][D][s_pad]
  void* out;       // [B][S][nh * D]
  int S, s_pad, nh, nkv;
  float scale_log2;  // log2(e) / sqrt(D)
};

// Buffer resource over [base, base + bytes): loads outside read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t attn_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

template <int D, int NKV>
__global__ __launch_bounds__(NKV * 64, 2) void phi_attn_prefill_f16_kernel(AttnArgs a) {
  static_assert(D == 64 || D == 96 || D == 128, "head_dim");
  constexpr int HB = D == 128 ? 1 : 2;      // 32-key halves per key block (register budget)
  constexpr int KB = 32 * HB, OLD = D + 4, KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) float sO[NKV][32 * OLD];  // per wave: O[query][d], unnormalised
  __shared__ float sM[NKV][32], sL[NKV][32];

  const int qb = gridDim.x - 1 - blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (a.nh / a.nkv);
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 5, col = lane & 31;
  const int S = a.S;
  const int q0 = qb * 32;
  const int qi = q0 + col;
  const int nkb = min(q0 + 31, S - 1) / KB + 1;             // key blocks reaching this query block
  const int nj = w < nkb ? (nkb - w + NKV - 1) / NKV : 0;   // ... taken by this wave

  const f16* Q = reinterpret_cast<const f16*>(a.q) + ((size_t)(b * a.nh + h) * S) * D;
  const __amdgpu_buffer_rsrc_t krs =
      attn_rsrc(reinterpret_cast<const f16*>(a.k) + ((size_t)(b * a.nkv + g) * S) * D, S * D * 2);
  const __amdgpu_buffer_rsrc_t vrs =
      attn_rsrc(reinterpret_cast<const f16*>(a.vt) + ((size_t)(b * a.nkv + g) * D) * a.s_pad, D * a.s_pad * 2);
  const int kr = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);  // bits 2 and 3 swapped
  const int koff = (kr * D + grp * 8) * 2;
  const int voff = (col * a.s_pad + 8 * grp) * 2;

  f16x8 qf[KS];
  {
    const f16* qrow = Q + (size_t)min(qi, S - 1) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const f16x8*>(qrow + (ks * 2 + grp) * 8);
  }
  // operands of one key block, as HB 32-key halves
  f16x8 kf[HB][KS];
  f16x8 vf[HB][DB][2];
  auto load = [&](int key0) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int k32 = key0 + 32 * hb;
      // the block start goes into the per-lane offset, which the range check covers
      const int kv = koff + k32 * D * 2, vv = voff + k32 * 2;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[hb][ks] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, kv + ks * 32, 0, 0));
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int hv = 0; hv < 2; ++hv)
          vf[hb][db][hv] = __builtin_bit_cast(
              f16x8, __builtin_amdgcn_raw_buffer_load_b128(vrs, vv + (db * 32 * a.s_pad + 16 * hv) * 2, 0, 0));
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};
  float m_run = -__builtin_inff(), l_run = 0.f;

  for (int j = 0; j < nj; ++j) {
    const int key0 = (w + NKV * j) * KB;
    load(key0);
    __builtin_amdgcn_sched_barrier(0);  // all loads of the block in flight before the first MFMA
    f32x16 sc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      sc[hb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[hb][ks], qf[ks], sc[hb], 0, 0, 0);
    }
    // score register v of half hb holds key key0 + 32 hb + 16 (v / 8) + 8 grp + v % 8
    const bool diag = key0 + KB - 1 > q0;
    float mx = -__builtin_inff();
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = key0 + 32 * hb + 16 * (v >> 3) + 8 * grp + (v & 7);
        float t = sc[hb][v] * a.scale_log2;
        t = (diag && (key > qi || key >= S)) ? -__builtin_inff() : t;
        sc[hb][v] = t;
        mx = fmaxf(mx, t);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);  // finite: key0 <= q0 <= qi is never masked
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = exp2f(sc[hb][v] - m_new);
        sc[hb][v] = e;
        psum += e;
      }
    m_run = m_new;
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int i = 0; i < DB; ++i) o[i] *= alpha;
    if (key0 + KB > S) {  // value columns >= S are padding: zero them
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int hv = 0; hv < 2; ++hv)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (key0 + 32 * hb + 16 * hv + 8 * grp + e >= S) vf[hb][db][hv][e] = (f16)0.f;
    }
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int hv = 0; hv < 2; ++hv) {
        f16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = (f16)sc[hb][8 * hv + e];
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[hb][db][hv], pf, o[db], 0, 0, 0);
      }
  }

  // this wave's partial state -> LDS (query = col; d rows of O^T)
  const float l_w = l_run + __shfl_xor(l_run, 32);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) sO[w][col * OLD + db * 32 + 8 * (v >> 2) + 4 * grp + (v & 3)] = o[db][v];
  if (grp == 0) {
    sM[w][col] = m_run;
    sL[w][col] = l_w;
  }
  __syncthreads();
  // merge: one (query, 8-dim chunk) per thread and pass, one 16-byte store
  f16* out = reinterpret_cast<f16*>(a.out);
  const int ld = a.nh * D;
  constexpr int CH = D / 8;
  for (int it = threadIdx.x; it < 32 * CH; it += NKV * 64) {
    const int qq = it / CH, c = it - qq * CH;
    if (q0 + qq >= S) continue;
    float mx = -__builtin_inff();
#pragma unroll
    for (int ww = 0; ww < NKV; ++ww) mx = fmaxf(mx, sM[ww][qq]);
    float den = 0.f;
    f32x4 n0 = f32x4{}, n1 = f32x4{};
#pragma unroll
    for (int ww = 0; ww < NKV; ++ww) {
      const float mw = sM[ww][qq];
      const float f = mw == -__builtin_inff() ? 0.f : exp2f(mw - mx);  // waves with no keys weigh 0
      den += sL[ww][qq] * f;
      const f32x4* src = reinterpret_cast<const f32x4*>(&sO[ww][qq * OLD + c * 8]);
      n0 += src[0] * f;
      n1 += src[1] * f;
    }
    const float inv = 1.0f / den;
    f16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = (f16)(n0[e] * inv);
      r[4 + e] = (f16)(n1[e] * inv);
    }
    *reinterpret_cast<f16x8*>(out + ((size_t)b * S + q0 + qq) * ld + h * D + c * 8) = r;
  }
}

__global__ __launch_bounds__(64) void phi_attn_prefill_f32_kernel(AttnArgs a) {
  constexpr int D = 96;
  const int qi = blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  if (qi >= a.S) return;
  const int g = h / (a.nh / a.nkv);
  const float* Q = reinterpret_cast<const float*>(a.q) + ((size_t)(b * a.nh + h) * a.S + qi) * D;
  const float* Kp = reinterpret_cast<const float*>(a.k) + ((size_t)(b * a.nkv + g) * a.S) * D;
  const float* Vt = reinterpret_cast<const float*>(a.vt) + ((size_t)(b * a.nkv + g) * D) * a.s_pad;
  float qv[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { qv[d] = Q[d]; acc[d] = 0.f; }
  float m = -__builtin_inff(), l = 0.f;
  for (int t = 0; t <= qi; ++t) {
    const float* kr = Kp + (size_t)t * D;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(qv[d], kr[d], s);
    s *= a.scale_log2;
    const float mn = fmaxf(m, s);
    const float al = exp2f(m - mn), p = exp2f(s - mn);
    l = l * al + p;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = acc[d] * al + p * Vt[(size_t)d * a.s_pad + t];
    m = mn;
  }
  float* out = reinterpret_cast<float*>(a.out) + ((size_t)b * a.S + qi) * (a.nh * D) + h * D;
  const float inv = 1.0f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) out[d] = acc[d] * inv;
}

}  // namespace phi
