// Causal softmax attention for the prefill, head_dim 96 (binary16 and float32)
// or 64 and 128 (binary16).
//
// binary16 paths (MFMA).  Two kernels share the score/softmax/output
// formulation below: the split-key kernel for launches with few workgroups,
// and the shared-key-block kernel (further down) for long sequences and
// large batches, where it reads each key block from HBM once per 128 queries.
//
// Split keys: a workgroup owns 32 queries of one
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
// on fp32 scores; P enters the MFMA as binary16.  The grid is (heads x
// batch, query blocks) with query blocks reversed, so the longest workgroups
// of every head are dispatched first (a greedy longest-first schedule over
// the whole grid), and consecutive workgroups, which go to different XCDs,
// are different heads of the same query block.
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

// One key block of the online softmax, in place.  sc holds raw scores
// q . k of NH 32-key halves (register v of half hb: key 32 hb + 16 (v / 8) +
// 8 grp + v % 8 of the block); on return it holds P = 2^(c s - m) with the
// running max m (in log2 units, c = log2(e) / sqrt(D)) and the running sum
// l updated.  Keys above kmax (relative to the lane's 8 grp offset) are
// masked when diag is set.  The output accumulators are rescaled only when
// some lane's max grew (a wave-uniform branch; the factor is exactly 1
// otherwise).  v_exp_f32 is used directly: arguments below -126 give 0 or a
// subnormal instead of the exact tiny value, which binary16 P cannot hold.
template <int NH, int DB>
__device__ __forceinline__ void softmax_block(f32x16 (&sc)[NH], f32x16 (&o)[DB], float& m_run, float& l_run, float c,
                                              bool diag, int kmax) {
  if (diag) {
#pragma unroll
    for (int hb = 0; hb < NH; ++hb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        sc[hb][v] = 32 * hb + 16 * (v >> 3) + (v & 7) > kmax ? -__builtin_inff() : sc[hb][v];
  }
  float mx = -__builtin_inff();
#pragma unroll
  for (int hb = 0; hb < NH; ++hb)
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[hb][v]);
  mx = max_xor32(mx);
  const float m_new = fmaxf(m_run, mx * c);  // finite: every lane has an unmasked key in its first block
  float psum = 0.f;
#pragma unroll
  for (int hb = 0; hb < NH; ++hb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float e = __builtin_amdgcn_exp2f(fmaf(sc[hb][v], c, -m_new));
      sc[hb][v] = e;
      psum += e;
    }
  if (__ballot(m_new > m_run)) {
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first block (m_run = -inf)
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < DB; ++i) o[i] *= alpha;
  }
  m_run = m_new;
  l_run += psum;
}

template <int D, int NKV>
__global__ __launch_bounds__(NKV * 64, 2) void phi_attn_prefill_f16_kernel(AttnArgs a) {
  static_assert(D == 64 || D == 96 || D == 128, "head_dim");
  constexpr int HB = D == 128 ? 1 : 2;      // 32-key halves per key block (register budget)
  constexpr int KB = 32 * HB, OLD = D + 4, KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) float sO[NKV][32 * OLD];  // per wave: O[query][d], unnormalised
  __shared__ float sM[NKV][32], sL[NKV][32];

  // grid (heads x batch, query blocks): every (sequence, head) of the
  // longest query block is dispatched before any shorter one
  const int qb = gridDim.y - 1 - blockIdx.y;
  const int h = blockIdx.x % a.nh, b = blockIdx.x / a.nh;
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
    // keys past min(qi, S - 1) are masked, in blocks that reach the diagonal
    softmax_block<HB, DB>(sc, o, m_run, l_run, a.scale_log2, key0 + KB - 1 > q0, min(qi, S - 1) - key0 - 8 * grp);
    if (key0 + KB > S) {  // value columns >= S are padding: zero them
      const int vlim = S - key0 - 8 * grp;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int hv = 0; hv < 2; ++hv)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              vf[hb][db][hv][e] = 32 * hb + 16 * hv + e < vlim ? vf[hb][db][hv][e] : (f16)0.f;
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
  const float l_w = add_xor32(l_run);
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

// binary16 path for long sequences (shared key blocks): a workgroup owns 128
// queries of one (sequence, head), 32 per wave, and walks the 64-key blocks
// up to its last query once.  Each block's keys [64][D] and V^T columns
// [D][64] go global -> LDS by DMA into a ring of 3 stages (2 at head_dim
// 128, where 3 would leave one workgroup per CU), the others ahead of the one
// being read, and all four waves read them from LDS (one global read
// per block per workgroup instead of one per wave).  With 8 waves a
// workgroup owns 256 queries.  Each wave keeps its own online softmax over
// every block up to its diagonal, so no merge is needed.  The softmax here
// differs from the split-key kernel's in three ways that take VALU work off
// the block loop: the queries are pre-scaled by log2(e) / sqrt(D); the score
// MFMA starts from the lane's reference max (no per-score fma), and the
// reference moves only when a block exceeds it by more than 8 (so P <= 2^8);
// the row sums come from one more MFMA per 16 keys with an all-ones operand
// instead of 32 adds.
// LDS rows: a key row is D / 8 + 1 16-byte slots (the extra slot is padding
// that makes the 32 rows of a fragment read conflict free); a V^T row is 8
// slots with chunk' = chunk ^ ((d >> 1) & 7).  The MFMA formulation and the
// key-row permutation are those of the split-key kernel.
template <int D, int NWV = 4>
__global__ __launch_bounds__(64 * NWV, 8 / NWV) void phi_attn_prefill_lds_kernel(AttnArgs a) {
  static_assert(D == 64 || D == 96 || D == 128, "head_dim");
  static_assert(NWV == 4 || NWV == 8, "waves per workgroup");
  constexpr int KB = 64, KS = D / 16, DB = D / 32;
  constexpr int QPW = 32 * NWV;                          // queries per workgroup
  constexpr int HW = NWV / 2;                            // waves copying keys (the rest copy V^T)
  // stages: 4 waves keep two workgroups per CU in LDS; 8 waves run one
  constexpr int NSTG = (D == 128 && NWV == 4) ? 2 : 3;
  constexpr int PD = NSTG - 1;                           // blocks in flight ahead of the one read
  constexpr int KSLOT = D / 8 + 1;                       // 16-byte slots per LDS key row
  constexpr int NK = KB * KSLOT / 64, NV = D * 8 / 64;   // 1 KB DMA instructions per block
  constexpr int NI = NK + NV, LPW = ((NK > NV ? NK : NV) + HW - 1) / HW;  // loads per wave and block
  constexpr int STG = NI * 1024;                          // bytes per stage
  constexpr int OLD = D + 8;                              // output staging row (f16)
  constexpr bool kEarlyV = D <= 96;                       // value fragments read with the key fragments
  static_assert(NK * 64 == KB * KSLOT, "key slots fill whole instructions");
  static_assert(NWV * 32 * OLD * 2 <= NSTG * STG, "output staging fits");
  static_assert((8 / NWV) * NSTG * STG <= 160 * 1024, "workgroups per CU fit in LDS");
  __shared__ __attribute__((aligned(1024))) char lds[NSTG * STG];

  const int qb = gridDim.y - 1 - blockIdx.y;   // query block, longest first over the whole grid
  const int h = blockIdx.x % a.nh, b = blockIdx.x / a.nh;
  const int g = h / (a.nh / a.nkv);
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 5, col = lane & 31;
  const int S = a.S;
  const int q0 = qb * QPW + 32 * w;            // this wave's first query
  const int qi = q0 + col;
  const int last_q = min(qb * QPW + QPW - 1, S - 1);
  const int nb = last_q / KB + 1;              // key blocks of the workgroup
  const int wave_last = q0 < S ? min(q0 + 31, S - 1) : -1;  // -1: the wave has no queries

  const f16* Q = reinterpret_cast<const f16*>(a.q) + ((size_t)(b * a.nh + h) * S) * D;
  const f16* Kp = reinterpret_cast<const f16*>(a.k) + ((size_t)(b * a.nkv + g) * S) * D;
  const f16* Vt = reinterpret_cast<const f16*>(a.vt) + ((size_t)(b * a.nkv + g) * D) * a.s_pad;

  // DMA work: the first HW waves copy the key rows (instructions 0 .. NK - 1,
  // round robin), the other HW waves the V^T rows (NK .. NI - 1); a wave with
  // fewer instructions than LPW repeats its last one, so every wave has LPW
  // loads in flight per block and one vmcnt count fits all.
  const bool kwave = w < HW;
  const int nown = kwave ? NK : NV, wi = w % HW;
  int lrow[LPW], loff[LPW], ldst[LPW];
#pragma unroll
  for (int t = 0; t < LPW; ++t) {
    const int jj = min(wi + HW * t, nown - 1 - (nown - 1 - wi) % HW);  // index among the wave's kind
    const int sl = jj * 64 + lane;
    if (kwave) {
      const int r = sl / KSLOT, c = min(sl - r * KSLOT, D / 8 - 1);  // the padding slot re-reads the last chunk
      lrow[t] = r;
      loff[t] = c * 8;
      ldst[t] = jj * 1024;
    } else {
      const int d = sl >> 3, c = (sl & 7) ^ ((d >> 1) & 7);
      lrow[t] = 0;
      loff[t] = d * a.s_pad + c * 8;             // + key0: columns < s_pad, inside the buffer
      ldst[t] = (NK + jj) * 1024;
    }
  }
  // The copies are buffer loads into LDS (MUBUF): the compiler counts a
  // global (FLAT) load into LDS as an LDS access in flight as well, and then
  // waits for lgkmcnt(0) before the first use of any later LDS read; with the
  // buffer form each fragment read gets its own lgkmcnt wait.
  const __amdgpu_buffer_rsrc_t krs = attn_rsrc(Kp, S * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = attn_rsrc(Vt, D * a.s_pad * 2);
  auto issue = [&](int blk, int stage) {
    const int key0 = blk * KB;
    char* st = lds + stage * STG;
    if (kwave) {
#pragma unroll
      for (int t = 0; t < LPW; ++t) {
        // key rows past the sequence re-read the last row (their scores are masked)
        const int off = (min(key0 + lrow[t], S - 1) * D + loff[t]) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)(st + ldst[t]), 16, off, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int t = 0; t < LPW; ++t) {
        const int off = (loff[t] + key0) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)(st + ldst[t]), 16, off, 0, 0, 0);
      }
    }
  };

  const int kr = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);  // bits 2 and 3 swapped

  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};
  float m_run = -__builtin_inff();  // the lane's reference b (log2 units of c s); -inf before its first block

  issue(0, 0);
  f16x8 qf[KS];
  {
    const f16* qrow = Q + (size_t)min(qi, S - 1) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const f16x8*>(qrow + (ks * 2 + grp) * 8);
  }
  if (PD > 1 && nb > 1) issue(1, 1);
  // Wait for the query fragments here, where only block 1's loads are newer,
  // so that the compiler does not wait for every load in flight at their
  // first use inside the loop.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
  // queries pre-scaled by c = log2(e) / sqrt(D) (rounded to binary16), so
  // the score MFMA yields c s directly, in log2 units
  {
    const float c = a.scale_log2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = (f16)((float)qf[ks][e] * c);
  }
  // Lazy running max: the score MFMA accumulates onto -b (b: this lane's
  // reference, negm its splat), so it yields c s - b; b moves only when a
  // block's max exceeds it by more than kLazy (P then stays <= 2^kLazy) or
  // on the lane's first block.  The row sums come from the value MFMA with
  // an all-ones operand, i.e. from the same binary16 P as the output.
  constexpr float kLazy = 8.f;
  f32x16 negm = f32x16{};
  f32x16 lacc = f32x16{};
  const f16x8 ones = {(f16)1.f, (f16)1.f, (f16)1.f, (f16)1.f, (f16)1.f, (f16)1.f, (f16)1.f, (f16)1.f};
  for (int j = 0; j < nb; ++j) {
    // block j landed: only the (PD - 1) newer blocks' loads may still be in flight
    if (PD > 1 && j + 1 < nb) PHI_WAIT_VMCNT((PD - 1) * LPW);
    else PHI_WAIT_VMCNT(0);
    lds_barrier();  // every wave's share of block j is in LDS; block j - 1's stage is free
    if (j + PD < nb) issue(j + PD, (j + PD) % NSTG);
    const int key0 = j * KB;
    if (key0 > wave_last) continue;            // above this wave's diagonal (barriers still met)
    const char* ks_base = lds + (j % NSTG) * STG;
    const char* vs_base = ks_base + NK * 1024;
    // LDS fragment reads are issued in groups ahead of the MFMAs that use
    // them, so a group pays the LDS latency once instead of once per MFMA.
    // Up to head_dim 96 the whole block's key fragments go first, then the
    // value fragments, which land under the score MFMAs and the softmax; at
    // 128 (registers) the key fragments go per 32-key half and the value
    // fragments per 16-key group, after the softmax.
    auto read_v = [&](int hb, int hv, f16x8 (&v)[DB]) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = db * 32 + col, chunk = 4 * hb + 2 * hv + grp;
        v[db] = *reinterpret_cast<const f16x8*>(vs_base + d * 128 + 16 * (chunk ^ ((d >> 1) & 7)));
      }
    };
    f16x8 vf[kEarlyV ? 2 : 1][2][DB];
    f32x16 sc[2];
    if constexpr (kEarlyV) {
      f16x8 kf[2][KS];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kf[hb][ks] = *reinterpret_cast<const f16x8*>(ks_base + ((32 * hb + kr) * KSLOT + ks * 2 + grp) * 16);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int hv = 0; hv < 2; ++hv) read_v(hb, hv, vf[hb][hv]);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        sc[hb] = negm;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          sc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[hb][ks], qf[ks], sc[hb], 0, 0, 0);
      }
      // order: the key reads, then each score MFMA followed by one value
      // read (2 KS MFMAs, 4 DB = 2 KS value reads)
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS, 0);
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    } else {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        f16x8 kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kf[ks] = *reinterpret_cast<const f16x8*>(ks_base + ((32 * hb + kr) * KSLOT + ks * 2 + grp) * 16);
        __builtin_amdgcn_sched_barrier(0);
        sc[hb] = negm;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ks], qf[ks], sc[hb], 0, 0, 0);
      }
    }
    if (key0 + KB - 1 > q0) {  // keys past min(qi, S - 1) are masked, in blocks that reach the diagonal
      const int kmax = min(qi, S - 1) - key0 - 8 * grp;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[hb][v] = 32 * hb + 16 * (v >> 3) + (v & 7) > kmax ? -__builtin_inff() : sc[hb][v];
    }
    {
      float mx = -__builtin_inff();
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[hb][v]);
      mx = max_xor32(mx);  // block max of c s - b (b = 0 before the lane's first block)
      const bool first = m_run == -__builtin_inff();
      const bool move = first || mx > kLazy;
      if (__ballot(move)) {
        const float delta = move ? mx : 0.f;  // finite: every lane has an unmasked key in its first block
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int v = 0; v < 16; ++v) sc[hb][v] -= delta;
        const float alpha = first ? 0.f : __builtin_amdgcn_exp2f(-delta);
#pragma unroll
        for (int i = 0; i < DB; ++i) o[i] *= alpha;
        lacc *= alpha;
        m_run = (first ? 0.f : m_run) + delta;
#pragma unroll
        for (int v = 0; v < 16; ++v) negm[v] = -m_run;
      }
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[hb][v] = __builtin_amdgcn_exp2f(sc[hb][v]);
    const bool tail = key0 + KB > S;  // value columns >= S are padding: zero them
    const int vlim = S - key0;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int hv = 0; hv < 2; ++hv) {
        f16x8 (&v)[DB] = vf[kEarlyV ? hb : 0][kEarlyV ? hv : 0];
        if constexpr (!kEarlyV) read_v(hb, hv, v);
        const int chunk = 4 * hb + 2 * hv + grp;
        if (tail) {
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 8; ++e) v[db][e] = 8 * chunk + e < vlim ? v[db][e] : (f16)0.f;
        }
        f16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = (f16)sc[hb][8 * hv + e];
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v[db], pf, o[db], 0, 0, 0);
        lacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ones, pf, lacc, 0, 0, 0);
      }
  }

  // normalise, stage [query][d] through LDS, 16-byte stores
  const float l_tot = lacc[0];  // every row of the ones product is the query's sum over all keys
  const float inv = wave_last >= q0 ? 1.0f / l_tot : 0.f;
  __syncthreads();  // every wave is done with the stages
  f16* so = reinterpret_cast<f16*>(lds) + w * 32 * OLD;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) so[col * OLD + db * 32 + 8 * (v >> 2) + 4 * grp + (v & 3)] = (f16)(o[db][v] * inv);
  __syncthreads();
  f16* out = reinterpret_cast<f16*>(a.out);
  const int ld = a.nh * D;
  constexpr int CH = D / 8;
  for (int c = lane; c < 32 * CH; c += 64) {
    const int r = c / CH, ch = c - r * CH;
    const int qq = q0 + r;
    if (qq < S)
      *reinterpret_cast<f16x8*>(out + ((size_t)b * S + qq) * ld + h * D + ch * 8) =
          *reinterpret_cast<const f16x8*>(so + r * OLD + ch * 8);
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
