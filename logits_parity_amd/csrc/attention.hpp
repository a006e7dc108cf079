// Causal softmax attention for the prefill, head_dim 96.
//
// binary16 path (flash style, MFMA): a workgroup owns NW x 32 queries of one
// (sequence, head); each wave owns 32 of them.  Keys are streamed through LDS
// in blocks of 64.  Scores are formed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_f16, so each lane holds one query's column: the running
// max, the running sum and the rescale of the output accumulator are per-lane
// scalars, and only the max needs one cross-lane exchange (lanes l and l+32).
// The output is accumulated transposed too, O^T += V^T P^T, with P^T taken
// straight from the score registers (the 8 keys a lane supplies to the MFMA
// are the ones its score registers hold, and the V^T operand is read from LDS
// with the same key order).  Softmax runs in base 2 on fp32 scores; P enters
// the MFMA as binary16.  Blocks entirely above the diagonal are skipped; the
// diagonal block is masked.  Query blocks are issued last-first so the
// longest rows start first.
//
// binary16 path for short sequences (split keys): a workgroup owns only 32
// queries and its 4 waves split the key range (blocks of 32 keys taken
// round-robin), so a 512-token sequence still yields hundreds of workgroups.
// Each wave loads its K and V^T operands straight from global memory into
// MFMA operand registers, one block ahead, with no LDS and no barrier in the
// key loop; the four partial softmax states (max, sum, output) are merged by
// log-sum-exp through LDS at the end.
//
// float32 path: one thread per query, online softmax over keys t <= s.
#pragma once
#include "common.hpp"

namespace phi {

struct AttnArgs {
  const void* q;   // [B][nh][S][96]
  const void* k;   // [B][nkv][S][96]
  const void* vt;  // [B][nkv][96][s_pad]
  void* out;       // [B][S][nh * 96]
  int S, s_pad, nh, nkv;
  float scale_log2;  // log2(e) / sqrt(96)
};

template <int NW>
__global__ __launch_bounds__(NW * 64) void phi_attn_prefill_f16_kernel(AttnArgs a) {
  constexpr int D = 96, KB = 64, KLD = 104, VLD = 72, NT = NW * 64;
  __shared__ __attribute__((aligned(16))) f16 sK[KB * KLD];
  __shared__ __attribute__((aligned(16))) f16 sV[D * VLD];
  __shared__ __attribute__((aligned(16))) f16 sO[NW][32 * KLD];

  const int qb = gridDim.x - 1 - blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (a.nh / a.nkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int S = a.S;
  const int q_lo = qb * 32 * NW;
  const int wq0 = q_lo + 32 * w;
  const int qi = wq0 + (lane & 31);
  const int grp = lane >> 5;
  const int wq_hi = min(wq0 + 31, S - 1);  // < wq0 when the wave has no queries
  const int blk_end = min(S, q_lo + 32 * NW);
  const int nkb = (blk_end + KB - 1) / KB;

  const f16* Q = reinterpret_cast<const f16*>(a.q) + ((size_t)(b * a.nh + h) * S) * D;
  const f16* Kp = reinterpret_cast<const f16*>(a.k) + ((size_t)(b * a.nkv + g) * S) * D;
  const f16* Vt = reinterpret_cast<const f16*>(a.vt) + ((size_t)(b * a.nkv + g) * D) * a.s_pad;

  f16x8 qf[6];
  {
    const f16* qrow = Q + (size_t)min(qi, S - 1) * D;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) qf[ks] = *reinterpret_cast<const f16x8*>(qrow + (ks * 2 + grp) * 8);
  }

  f32x16 o[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) o[i] = f32x16{};
  float m_run = -__builtin_inff(), l_run = 0.f;

  for (int kb = 0; kb < nkb; ++kb) {
    const int key0 = kb * KB;
    for (int c = tid; c < KB * 12; c += NT) {
      const int r = c / 12, ch = c - r * 12;
      const int kr = min(key0 + r, S - 1);
      *reinterpret_cast<f16x8*>(sK + r * KLD + ch * 8) =
          *reinterpret_cast<const f16x8*>(Kp + (size_t)kr * D + ch * 8);
    }
    for (int c = tid; c < D * 8; c += NT) {
      const int r = c >> 3, ch = c & 7;
      const int kk = key0 + ch * 8;
      f16x8 v = *reinterpret_cast<const f16x8*>(Vt + (size_t)r * a.s_pad + kk);
      if (kk + 8 > S) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (kk + e >= S) v[e] = (f16)0.f;
      }
      *reinterpret_cast<f16x8*>(sV + r * VLD + ch * 8) = v;
    }
    __syncthreads();

    if (key0 <= wq_hi) {
      f32x16 s[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        s[sb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 6; ++ks) {
          const f16x8 kf = *reinterpret_cast<const f16x8*>(sK + (sb * 32 + (lane & 31)) * KLD + (ks * 2 + grp) * 8);
          s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], s[sb], 0, 0, 0);
        }
      }
      const bool diag = key0 + KB - 1 > wq0;
      float mx = -__builtin_inff();
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float t = s[sb][v] * a.scale_log2;
          if (diag) {
            const int key = key0 + sb * 32 + 8 * (v >> 2) + 4 * grp + (v & 3);
            if (key > qi || key >= S) t = -__builtin_inff();
          }
          s[sb][v] = t;
          mx = fmaxf(mx, t);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = exp2f(s[sb][v] - m_new);
          s[sb][v] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int i = 0; i < 3; ++i) o[i] *= alpha;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int hv = 0; hv < 2; ++hv) {
          f16x8 pf;
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[e] = (f16)s[sb][8 * hv + e];
          const int koff = sb * 32 + 16 * hv + 4 * grp;
#pragma unroll
          for (int db = 0; db < 3; ++db) {
            const f16* vr = sV + (db * 32 + (lane & 31)) * VLD + koff;
            const f16x4 v0 = *reinterpret_cast<const f16x4*>(vr);
            const f16x4 v1 = *reinterpret_cast<const f16x4*>(vr + 8);
            const f16x8 vf = f16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf, o[db], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  f16* so = sO[w];
#pragma unroll
  for (int db = 0; db < 3; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int d = db * 32 + 8 * (v >> 2) + 4 * grp + (v & 3);
      so[(lane & 31) * KLD + d] = (f16)(o[db][v] * inv);
    }
  __syncthreads();
  f16* out = reinterpret_cast<f16*>(a.out);
  const int ld = a.nh * D;
  for (int c = lane; c < 32 * 12; c += 64) {
    const int r = c / 12, ch = c - r * 12;
    const int qq = wq0 + r;
    if (qq < S)
      *reinterpret_cast<f16x8*>(out + ((size_t)b * S + qq) * ld + h * D + ch * 8) =
          *reinterpret_cast<const f16x8*>(so + r * KLD + ch * 8);
  }
}


template <int NKV>
__global__ __launch_bounds__(NKV * 64) void phi_attn_prefill_split_kernel(AttnArgs a) {
  constexpr int D = 96, KB = 32, OLD = 97;
  __shared__ float sO[NKV][32 * OLD];  // per wave: O[query][d], unnormalised
  __shared__ float sM[NKV][32], sL[NKV][32];

  const int qb = gridDim.x - 1 - blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (a.nh / a.nkv);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int grp = lane >> 5, col = lane & 31;
  const int S = a.S;
  const int q0 = qb * 32;
  const int qi = q0 + col;
  const int q_last = min(q0 + 31, S - 1);
  const int nkb = q_last / KB + 1;  // key blocks that reach this query block

  const f16* Q = reinterpret_cast<const f16*>(a.q) + ((size_t)(b * a.nh + h) * S) * D;
  const f16* Kp = reinterpret_cast<const f16*>(a.k) + ((size_t)(b * a.nkv + g) * S) * D;
  const f16* Vt = reinterpret_cast<const f16*>(a.vt) + ((size_t)(b * a.nkv + g) * D) * a.s_pad;

  f16x8 qf[6];
  {
    const f16* qrow = Q + (size_t)min(qi, S - 1) * D;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) qf[ks] = *reinterpret_cast<const f16x8*>(qrow + (ks * 2 + grp) * 8);
  }

  // operand registers of one key block: K rows as the A operand of S^T = K Q^T,
  // V^T rows (keys in this lane's score order) as the A operand of O^T = V^T P^T
  f16x8 kf[2][6];
  f16x8 vf[2][3][2];
  auto load_block = [&](int kb, f16x8* kk, f16x8 (*vv)[2]) {
    const int key0 = kb * KB;
    const f16* krow = Kp + (size_t)min(key0 + col, S - 1) * D;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) kk[ks] = *reinterpret_cast<const f16x8*>(krow + (ks * 2 + grp) * 8);
#pragma unroll
    for (int db = 0; db < 3; ++db) {
      const f16* vr = Vt + (size_t)(db * 32 + col) * a.s_pad + key0;
#pragma unroll
      for (int hv = 0; hv < 2; ++hv) {
        const int k0 = 16 * hv + 4 * grp;
        f16x4 v0 = *reinterpret_cast<const f16x4*>(vr + k0);
        f16x4 v1 = *reinterpret_cast<const f16x4*>(vr + k0 + 8);
        if (key0 + KB > S) {  // keys >= S hold padding: zero them
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (key0 + k0 + e >= S) v0[e] = (f16)0.f;
            if (key0 + k0 + 8 + e >= S) v1[e] = (f16)0.f;
          }
        }
        vv[db][hv] = f16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      }
    }
  };

  f32x16 o[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) o[i] = f32x16{};
  float m_run = -__builtin_inff(), l_run = 0.f;

  // one key block: scores, online softmax, P V; buffers fixed at compile time
  auto step = [&](int kb, const f16x8* kk, const f16x8 (*vv)[2]) {
    const int key0 = kb * KB;
    f32x16 sc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kk[ks], qf[ks], sc, 0, 0, 0);
    const bool diag = key0 + KB - 1 > q0;
    float mx = -__builtin_inff();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float t = sc[v] * a.scale_log2;
      if (diag) {
        const int key = key0 + 8 * (v >> 2) + 4 * grp + (v & 3);
        if (key > qi || key >= S) t = -__builtin_inff();
      }
      sc[v] = t;
      mx = fmaxf(mx, t);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = exp2f(sc[v] - m_new);
      sc[v] = p;
      psum += p;
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int i = 0; i < 3; ++i) o[i] *= alpha;
#pragma unroll
    for (int hv = 0; hv < 2; ++hv) {
      f16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = (f16)sc[8 * hv + e];
#pragma unroll
      for (int db = 0; db < 3; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vv[db][hv], pf, o[db], 0, 0, 0);
    }
  };

  // blocks w, w + NKV, ... alternate between the two register buffers
  int kb = w;
  if (kb < nkb) load_block(kb, kf[0], vf[0]);
  while (kb < nkb) {
    if (kb + NKV < nkb) load_block(kb + NKV, kf[1], vf[1]);
    step(kb, kf[0], vf[0]);
    kb += NKV;
    if (kb >= nkb) break;
    if (kb + NKV < nkb) load_block(kb + NKV, kf[0], vf[0]);
    step(kb, kf[1], vf[1]);
    kb += NKV;
  }

  // this wave's partial state -> LDS (query = col; d rows of O^T)
  const float l_w = l_run + __shfl_xor(l_run, 32);
#pragma unroll
  for (int db = 0; db < 3; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) sO[w][col * OLD + db * 32 + 8 * (v >> 2) + 4 * grp + (v & 3)] = o[db][v];
  if (grp == 0) {
    sM[w][col] = m_run;
    sL[w][col] = l_w;
  }
  __syncthreads();
  f16* out = reinterpret_cast<f16*>(a.out);
  const int ld = a.nh * D;
  for (int idx = threadIdx.x; idx < 32 * D; idx += NKV * 64) {
    const int qq = idx / D, d = idx - qq * D;
    if (q0 + qq >= S) continue;
    float mx = -__builtin_inff();
#pragma unroll
    for (int ww = 0; ww < NKV; ++ww) mx = fmaxf(mx, sM[ww][qq]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < NKV; ++ww) {
      const float mw = sM[ww][qq];
      const float f = mw == -__builtin_inff() ? 0.f : exp2f(mw - mx);
      num += sO[ww][qq * OLD + d] * f;
      den += sL[ww][qq] * f;
    }
    out[((size_t)b * S + q0 + qq) * ld + h * D + d] = (f16)(num / den);
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
