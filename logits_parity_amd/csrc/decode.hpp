// K16/V8 paged decode attention: binary16 keys, OCP E4M3FN values with one
// fp32 scale per KV head, 16-token pages, head_dim 128.
//
// Split kernel: a workgroup owns one (sequence, KV head, context split) and
// serves all G query heads of the GQA group from one read of each K/V page.
// Its NWV waves (4, or 8 for one long split per sequence): wave w takes pages
// w, w + NWV, ... of the split and streams them through its
// own LDS ring by direct global -> LDS loads (no VGPR staging), so page
// reads stay in flight while it computes.  Per page a wave
//  1. forms the scores S^T[token][head] = K Q^T with v_mfma_f32_16x16x32_f16:
//     16 tokens x 128 dims, 4 MFMAs; lane l supplies key row l % 16 and dims
//     8 (l / 16) + 32 k from LDS, and the query of head l % 16 (zero for
//     l % 16 >= G) as the other operand;
//  2. updates one running max per head (log2 units) and the probabilities
//     p = 2^(c s - max), rescaling the output only when a max grew;
//  3. accumulates O^T += V^T P^T with v_mfma_f32_16x16x16_f16: the score
//     registers already are the P^T operand (tokens 4 (l / 16) + j of head
//     l % 16), rounded to binary16; the V^T operand is built from 8 bytes of
//     E4M3 per token (dims 8 (l % 16) .. +7 of the lane's 4 tokens), transposed
//     bytewise by v_perm_b32 and widened exactly to binary16.
// At the end the waves are merged by log-sum-exp through LDS, and the split's
// (o unnormalised, max, sum) go to the workspace; with a single split the
// kernel normalises and writes the output itself.  The per-head value scale
// multiplies the final output once.
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
  int max_ctx;       // longest context the split plan covers (<= max_pages * 16)
  float scale_log2;  // sm_scale * log2(e)
};

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Each wave's ring has NST one-page stages, filled NST - 1 pages ahead of
// the page it computes; the four rings are independent (no barrier until the
// final merge).  Stage layout: keys [16 tokens][128 dims] binary16 with the
// 16-byte chunk c of token row r stored at slot c ^ r (conflict-free
// fragment reads), then the value codes [16][128] as in the page.
template <int G, int NST, int NWV = 4>
__global__ __launch_bounds__(64 * NWV, 8 / NWV) void phi_decode_stream_kernel(DecodeArgs a) {
  constexpr int D = 128, PG = 16;
  constexpr int KBY = PG * D * 2, VBY = PG * D, SB = KBY + VBY, WB = NST * SB;
  constexpr int LPP = KBY / 1024 + VBY / 1024;  // loads per page and wave
  static_assert(G >= 1 && G <= 8, "GQA group");
  static_assert(NST >= 2 && NST <= 4 && (NST - 2) * LPP <= 63, "ring depth");
  static_assert(NWV == 4 || NWV == 8, "waves per workgroup");
  static_assert(NWV * G * D * 4 + NWV * G * 2 * 4 <= NWV * WB, "merge staging fits in the rings");
  __shared__ __attribute__((aligned(1024))) char lds[NWV * WB];
  __shared__ int s_err[NWV];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane & 15, kq = lane >> 4;  // score layout: head column, token quad
  const int L = a.ctx_lens[b];
  // a length beyond the plan's max_ctx would lose its trailing pages: NaN instead
  bool err = L < 1 || L > a.max_ctx;
  const int np = err ? 0 : (L + PG - 1) / PG;
  const int p_begin = split * a.pages_per_split;
  const int p_end = min(np, p_begin + a.pages_per_split);
  // pages of this wave: w, w + NWV, ... of the split (<= 64: the host keeps pages_per_split <= 64 NWV)
  int nw = p_end - p_begin - w > 0 ? (p_end - p_begin - w + NWV - 1) / NWV : 0;

  // query operand: head hl (zero beyond the group), dims 32 k + 8 kq .. +7;
  // loaded together with the block-table entries, so both cost one latency
  f16x8 qf[4];
  {
    const f16* qrow = a.q + ((size_t)b * a.Hq + g * G + min(hl, G - 1)) * D + 8 * kq;
#pragma unroll
    for (int k = 0; k < 4; ++k) qf[k] = *reinterpret_cast<const f16x8*>(qrow + 32 * k);
  }
  // physical page of the wave's page i in lane i; the row is read without
  // waiting for the context length (lanes past nw read entries that are
  // never used), so the length, table and query loads share one latency
  const int ti = min(p_begin + w + NWV * lane, a.max_pages - 1);
  int my_phys = a.block_table[(size_t)b * a.max_pages + ti];
  if (lane < nw && (my_phys < 0 || my_phys >= a.n_pages)) err = true;
  if (__any(err)) {  // the split's result becomes NaN; read nothing
    err = true;
    nw = 0;
  }
  if (hl >= G) {
#pragma unroll
    for (int k = 0; k < 4; ++k) qf[k] = f16x8{};
  }

  char* ring = lds + w * WB;
  // Page copies are buffer loads into LDS over a resource per page (the
  // page's (KV head) slab is wave-uniform; a pool may exceed the 32-bit
  // offset range of one resource).  The buffer form, unlike a global load
  // into LDS, leaves the compiler's per-read lgkmcnt waits on the fragment
  // reads intact.
  auto issue = [&](int i) {
    const int phys = __builtin_amdgcn_readlane(my_phys, i);
    char* st = ring + (i % NST) * SB;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<f16*>(a.k_pool + ((size_t)phys * a.Hkv + g) * PG * D), 0, KBY, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.v_pool + ((size_t)phys * a.Hkv + g) * PG * D), 0, VBY, 0x00020000);
    const int r0 = lane >> 4, c = lane & 15;
#pragma unroll
    for (int j = 0; j < KBY / 1024; ++j) {  // token rows 4 j .. 4 j + 3; LDS slot c of row r takes chunk c ^ r
      const int r = 4 * j + r0;
      const int off = r * 256 + ((c ^ r) << 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)(st + j * 1024), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < VBY / 1024; ++j) {
      const int off = j * 1024 + lane * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)(st + KBY + j * 1024), 16, off, 0, 0, 0);
    }
  };

  for (int i = 0; i < NST - 1 && i < nw; ++i) issue(i);
#pragma unroll
  for (int k = 0; k < 4; ++k) asm volatile("" ::"v"(qf[k]));  // the query lands before the loop

  // O^T += V^T P^T by v_mfma_f32_16x16x16_f16, one MFMA per 8 dims of the
  // head: block db holds dims 8 r + db at MFMA row r, column = head, so lane l
  // accumulates head hl at dims 8 (4 kq + j) + db, j = 0..3 (its own head's
  // rows: the rescale needs no exchange)
  f32x4 acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = f32x4{};
  float m_run = -__builtin_inff();  // running max of head hl (log2 units)
  float l_run = 0.f;                // partial sum over this lane's tokens
  const float c2 = a.scale_log2;

  for (int i = 0; i < nw; ++i) {
    // page i landed; only the newer pages' loads (NST - 2 of them at most) may be in flight
    const int newer = min(NST - 2, nw - 1 - i);
    if (newer <= 0) PHI_WAIT_VMCNT(0);
    else if (newer == 1) PHI_WAIT_VMCNT(LPP);
    else PHI_WAIT_VMCNT(2 * LPP);
    asm volatile("" ::: "memory");  // the page's LDS reads stay after the wait
    if (i + NST - 1 < nw) issue(i + NST - 1);  // into the stage of page i - 1, whose reads are done
    const char* st = ring + (i % NST) * SB;
    const int pg = p_begin + w + NWV * i;

    // 1. scores of the page's 16 tokens for heads hl: lane l holds tokens 4 kq + j
    f32x4 sc = f32x4{};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f16x8 kf = *reinterpret_cast<const f16x8*>(st + hl * 256 + (((kq + 4 * k) ^ hl) << 4));
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[k], sc, 0, 0, 0);
    }
    // value codes of the lane's 4 tokens, dims 8 hl .. 8 hl + 7 (issued early)
    uint2 vw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vw[j] = *reinterpret_cast<const uint2*>(st + KBY + (4 * kq + j) * D + 8 * hl);
    const bool tail = (pg + 1) * PG > L;
    if (tail) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool live = pg * PG + 4 * kq + j < L;
        sc[j] = live ? sc[j] : -__builtin_inff();
        // slots past the context may hold any bytes (even NaN codes): code 0 there
        vw[j].x = live ? vw[j].x : 0u;
        vw[j].y = live ? vw[j].y : 0u;
      }
    }
    // 2. running max per head (lanes hl, hl + 16, hl + 32, hl + 48 share a head)
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = max_xor32(max_xor16(mx));
    const float m_new = fmaxf(m_run, mx * c2);  // finite: the page's first token is valid
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j] = __builtin_amdgcn_exp2f(fmaf(sc[j], c2, -m_new));
      ps += sc[j];
    }
    if (__ballot(m_new > m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first page
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] *= alpha;
    }
    m_run = m_new;
    l_run += ps;

    // 3. P^T operand (binary16, nearest) and the V^T operands: the 4 tokens'
    // words are transposed bytewise so that word db holds dim 8 hl + db of
    // the 4 tokens; E4M3 widens exactly to binary16
    const f16x4 pf = {(f16)sc[0], (f16)sc[1], (f16)sc[2], (f16)sc[3]};
    uint32_t cw[8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint32_t a0 = hh ? vw[0].y : vw[0].x, a1 = hh ? vw[1].y : vw[1].x;
      const uint32_t a2 = hh ? vw[2].y : vw[2].x, a3 = hh ? vw[3].y : vw[3].x;
      const uint32_t t01l = __builtin_amdgcn_perm(a1, a0, 0x05010400u), t01h = __builtin_amdgcn_perm(a1, a0, 0x07030602u);
      const uint32_t t23l = __builtin_amdgcn_perm(a3, a2, 0x05010400u), t23h = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
      cw[4 * hh + 0] = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u);
      cw[4 * hh + 1] = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
      cw[4 * hh + 2] = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
      cw[4 * hh + 3] = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(cw[db], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(cw[db], true);
      // exact: every E4M3 value is a binary16 value, so round-toward-zero packing loses nothing
      const f16x2 l2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(lo[0], lo[1]));
      const f16x2 h2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(hi[0], hi[1]));
      const f16x4 vf = {l2[0], l2[1], h2[0], h2[1]};
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(vf, pf, acc[db], 0, 0, 0);
    }
  }

  const float l_tot = add_xor32(add_xor16(l_run));
  __syncthreads();  // every wave is done with its ring: reuse it for the merge
  float* s_o = reinterpret_cast<float*>(lds);            // [NWV][G][D]
  float* s_ml = s_o + NWV * G * D;                         // [NWV][G][2]
  if (hl < G) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) s_o[(w * G + hl) * D + 8 * (4 * kq + j) + db] = acc[db][j];
  }
  if (lane < G) {
    s_ml[(w * G + lane) * 2 + 0] = m_run;
    s_ml[(w * G + lane) * 2 + 1] = l_tot;
  }
  if (lane == 0) s_err[w] = err;
  __syncthreads();
  bool bad = false;
#pragma unroll
  for (int ww = 0; ww < NWV; ++ww) bad |= s_err[ww] != 0;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * NWV) {
    const int h = idx / D, d = idx - h * D;
    float mn = -__builtin_inff();
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) mn = fmaxf(mn, s_ml[(ww * G + h) * 2]);
    float ls = 0.f, os = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) {
      const float mw = s_ml[(ww * G + h) * 2];
      const float f = mw == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mw - mn);
      ls += s_ml[(ww * G + h) * 2 + 1] * f;
      os += s_o[(ww * G + h) * D + d] * f;
    }
    if (a.n_split == 1) {  // the whole context in one split: normalise here, no merge launch
      const float r = (!bad && ls > 0.f) ? os / ls * a.v_scale[g] : __builtin_nanf("");
      a.out[(size_t)(b * a.Hq + g * G + h) * D + d] = (f16)r;
      continue;
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

namespace phi {

// ---- K16/V8 cache write ----------------------------------------------------
// One decode step appends one token per sequence: its binary16 key goes into
// the page slot as is, its value becomes the E4M3 code of the fp32 quotient
// v / v_scale[g], rounded to nearest-even and saturated to +-448 (NaN keeps a
// NaN code).  A group of 16 lanes owns one (sequence, KV head) row; lane j
// moves dims 8 j .. 8 j + 7: a 16-byte key store and an 8-byte value store.

struct KvAppendArgs {
  const f16* k_new;   // [B][Hkv][128]
  const f16* v_new;   // [B][Hkv][128]
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* positions;
  f16* k_pool;        // [n_pages][Hkv][16][128]
  uint8_t* v_pool;    // [n_pages][Hkv][16][128]
  int B, Hkv, n_pages, max_pages;
};

// Quotient ready for the hardware conversion: clamped into [-448, 448] so the
// conversion saturates instead of overflowing; NaN passes through.
__device__ __forceinline__ float e4m3_operand(float v, float s) {
  const float x = v / s;
  return x != x ? x : fminf(fmaxf(x, -448.f), 448.f);
}

// Four values to four E4M3 bytes (byte i = value i), NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_pack4(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  uint32_t u = static_cast<uint32_t>(w);
  const float x[4] = {x0, x1, x2, x3};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (x[i] != x[i]) u = (u & ~(0xFFu << (8 * i))) | (0x7Fu << (8 * i));
  return u;
}

__global__ __launch_bounds__(256) void phi_kv_append_kernel(KvAppendArgs a) {
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  if (row >= a.B * a.Hkv) return;
  const int b = row / a.Hkv, g = row - b * a.Hkv;
  const int t = a.positions[b];
  if (t < 0 || t >= a.max_pages * 16) return;
  const int page = a.block_table[(size_t)b * a.max_pages + (t >> 4)];
  if (page < 0 || page >= a.n_pages) return;
  const size_t src = (size_t)row * 128 + j * 8;
  const size_t dst = (((size_t)page * a.Hkv + g) * 16 + (t & 15)) * 128 + j * 8;
  *reinterpret_cast<uint4*>(a.k_pool + dst) = *reinterpret_cast<const uint4*>(a.k_new + src);
  const uint4 vv = *reinterpret_cast<const uint4*>(a.v_new + src);
  const f16* vh = reinterpret_cast<const f16*>(&vv);
  const float s = a.v_scale[g];
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = e4m3_operand(static_cast<float>(vh[i]), s);
  uint2 out;
  out.x = e4m3_pack4(x[0], x[1], x[2], x[3]);
  out.y = e4m3_pack4(x[4], x[5], x[6], x[7]);
  *reinterpret_cast<uint2*>(a.v_pool + dst) = out;
}

}  // namespace phi

namespace phi {

// ---- K16/V8 cache fill from a prefill ---------------------------------------
// The prefill's post-RoPE keys [B][Hkv][S][128] and transposed values
// V^T [B][Hkv][128][s_pad] (binary16, as the QKV GEMM leaves them) go to the
// pages of every sequence, token t of sequence b at block_table[b][t / 16],
// slot t % 16, with the value encoding of the single-token cache write.  One
// thread moves 8 dims of one token: a 16-byte key copy and an 8-byte value
// store (the 8 values are a column of V^T: 8 strided 2-byte loads).

struct KvFillArgs {
  const f16* k;       // [B][Hkv][S][128]
  const f16* vt;      // [B][Hkv][128][s_pad]
  const float* v_scale;
  const int32_t* block_table;
  f16* k_pool;
  uint8_t* v_pool;
  int B, Hkv, S, s_pad, n_pages, max_pages;
};

__global__ __launch_bounds__(256) void phi_kv_fill_kernel(KvFillArgs a) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)a.B * a.Hkv * a.S * 16;
  if (idx >= total) return;
  const int c = (int)(idx & 15);
  const size_t row = idx >> 4;             // (b, g, t)
  const int t = (int)(row % a.S);
  const int bg = (int)(row / a.S);
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  if (t >= a.max_pages * 16) return;
  const int page = a.block_table[(size_t)b * a.max_pages + (t >> 4)];
  if (page < 0 || page >= a.n_pages) return;
  const size_t dst = (((size_t)page * a.Hkv + g) * 16 + (t & 15)) * 128 + c * 8;
  *reinterpret_cast<uint4*>(a.k_pool + dst) = *reinterpret_cast<const uint4*>(a.k + row * 128 + c * 8);
  const f16* vcol = a.vt + ((size_t)bg * 128 + c * 8) * a.s_pad + t;
  const float s = a.v_scale[g];
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = e4m3_operand(static_cast<float>(vcol[(size_t)e * a.s_pad]), s);
  uint2 out;
  out.x = e4m3_pack4(x[0], x[1], x[2], x[3]);
  out.y = e4m3_pack4(x[4], x[5], x[6], x[7]);
  *reinterpret_cast<uint2*>(a.v_pool + dst) = out;
}

// ctx[b] = pos[b] + 1: the cache length a decode step attends over once its
// token is appended.  A position outside [0, max_ctx) gives length 0, which
// the attention kernel turns into a NaN output for that sequence.
__global__ void phi_ctx_from_pos_kernel(const int32_t* pos, int32_t* ctx, int B, int max_ctx) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) {
    const int p = pos[b];
    ctx[b] = (p >= 0 && p < max_ctx) ? p + 1 : 0;
  }
}

}  // namespace phi
