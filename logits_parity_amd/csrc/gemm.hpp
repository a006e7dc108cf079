// Prefill GEMMs: y[M][N] = a[M][K] w[N][K]^T with fused epilogues.
//
// Two cores share one set of epilogues:
//  - phi_gemm_mfma_kernel: binary16 activations, binary16 or int8 weights,
//    v_mfma_f32_32x32x16_f16 on 64-wide waves, fp32 accumulation.  Tiles are
//    staged through LDS in 16-byte chunks with an XOR swizzle (chunk c of row
//    r sits at c ^ (r & 7)) so each MFMA operand read is one conflict-free
//    ds_read_b128.  The K loop double-buffers LDS and overlaps the next tile's
//    global loads with the current tile's MFMAs.  int8 weights are widened to
//    binary16 exactly (|q| <= 127) on their way into LDS; the per-row scale
//    multiplies the fp32 accumulator, since it factors out of the K sum.
//  - phi_gemm_simt_f32_kernel: fp32 FMA core for the float32 model.
// After the K loop the accumulator tile is written to LDS (fp32) and the
// epilogue reads it row-wise, so every global store is a 16-byte vector:
//  EPI_F32    logits: out[m][n] = acc
//  EPI_RESID  residual: x[m][n] += acc
//  EPI_SILU   fused gate/up: the tile's first half holds gate rows, the second
//             half the matching up rows; act[m][n] = silu(gate) * up
//  EPI_QKV    fused Q/K/V: tiles cover whole heads; RoPE rotates pairs
//             (d, d + hd/2) of Q and K heads by angle pos * theta^(-2d/hd)
//             (tables precomputed); Q, K go to [B][heads][S][hd], V to
//             V^T [B][kv_heads][hd][s_pad].
#pragma once
#include "common.hpp"

namespace phi {

enum { EPI_F32 = 0, EPI_RESID = 1, EPI_SILU = 2, EPI_QKV = 3 };

struct GemmArgs {
  const void* A;      // [M][K] activations
  const void* W;      // [N][K] weights (f16, int8 or f32)
  const void* scale;  // binary16 [N] (int8 weights)
  int M, N, K;        // N = rows of W (2 I for the fused gate/up)
  int tiles_m, tiles_n;
  float* out;         // EPI_F32: [M][ldo]
  int ldo;
  float* x;           // EPI_RESID: [M][ldx]
  int ldx;
  void* act;          // EPI_SILU: [M][ld_act]
  int ld_act;
  void* q;            // EPI_QKV
  void* k;
  void* vt;
  const float* rope_cos;  // [max_pos][hd/2]
  const float* rope_sin;
  int S, s_pad, nh, nkv, hd;
};

// Row of W that local row r of N-tile tn reads.
template <int EPI, int BN>
__device__ __forceinline__ int w_row(const GemmArgs& a, int tn, int r) {
  if constexpr (EPI == EPI_SILU) {
    constexpr int H2 = BN / 2;
    const int I = a.N >> 1;
    return r < H2 ? tn * H2 + r : I + tn * H2 + (r - H2);
  } else {
    const int n = tn * BN + r;
    return n < a.N ? n : a.N - 1;
  }
}

template <class AT>
__device__ __forceinline__ void store8(AT* p, const float* v);
template <>
__device__ __forceinline__ void store8<f16>(f16* p, const float* v) {
  *reinterpret_cast<f16x8*>(p) =
      f16x8{(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3], (f16)v[4], (f16)v[5], (f16)v[6], (f16)v[7]};
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float* v) {
  reinterpret_cast<f32x4*>(p)[0] = f32x4{v[0], v[1], v[2], v[3]};
  reinterpret_cast<f32x4*>(p)[1] = f32x4{v[4], v[5], v[6], v[7]};
}

// Epilogue over an fp32 tile sC[BM][ldc] whose origin is row m0, N-tile tn.
template <int EPI, class AT, int BM, int BN>
__device__ void gemm_epilogue(const float* sC, int ldc, int m0, int tn, const GemmArgs& a, int tid, int nt) {
  if constexpr (EPI == EPI_F32 || EPI == EPI_RESID) {
    const int n0 = tn * BN;
    for (int u = tid; u < BM * (BN / 4); u += nt) {
      const int r = u / (BN / 4), c = (u % (BN / 4)) * 4;
      const int m = m0 + r, n = n0 + c;
      if (m >= a.M || n >= a.N) continue;
      const f32x4 v = *reinterpret_cast<const f32x4*>(sC + r * ldc + c);
      if constexpr (EPI == EPI_F32) {
        vec4<float>::store(a.out + (size_t)m * a.ldo + n, v);
      } else {
        float* px = a.x + (size_t)m * a.ldx + n;
        vec4<float>::store(px, vec4<float>::load(px) + v);
      }
    }
  } else if constexpr (EPI == EPI_SILU) {
    constexpr int H2 = BN / 2;
    const int n0 = tn * H2;
    AT* act = reinterpret_cast<AT*>(a.act);
    for (int u = tid; u < BM * (H2 / 4); u += nt) {
      const int r = u / (H2 / 4), c = (u % (H2 / 4)) * 4;
      const int m = m0 + r;
      if (m >= a.M) continue;
      const f32x4 g = *reinterpret_cast<const f32x4*>(sC + r * ldc + c);
      const f32x4 up = *reinterpret_cast<const f32x4*>(sC + r * ldc + H2 + c);
      f32x4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = g[e] / (1.0f + __expf(-g[e])) * up[e];
      vec4<AT>::store(act + (size_t)m * a.ld_act + n0 + c, y);
    }
  } else {  // EPI_QKV
    const int hd = a.hd, half = hd >> 1;
    const int n0 = tn * BN;
    constexpr int kHeads = BN / 96;  // head_dim 96: tiles hold whole heads
    const int q_end = a.nh * hd, k_end = (a.nh + a.nkv) * hd;
    AT* qo = reinterpret_cast<AT*>(a.q);
    AT* ko = reinterpret_cast<AT*>(a.k);
    AT* vo = reinterpret_cast<AT*>(a.vt);
    const int per_row = kHeads * (half / 4);
    for (int u = tid; u < BM * per_row; u += nt) {
      const int r = u / per_row, rest = u % per_row;
      const int hh = rest / (half / 4), d = (rest % (half / 4)) * 4;
      const int m = m0 + r, col0 = n0 + hh * hd;
      if (m >= a.M || col0 >= k_end) continue;
      AT* dst;
      int head, nheads;
      if (col0 < q_end) { dst = qo; head = col0 / hd; nheads = a.nh; }
      else { dst = ko; head = (col0 - q_end) / hd; nheads = a.nkv; }
      const int b = m / a.S, s = m - b * a.S;
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(sC + r * ldc + hh * hd + d);
      const f32x4 x2 = *reinterpret_cast<const f32x4*>(sC + r * ldc + hh * hd + half + d);
      const f32x4 cs = vec4<float>::load(a.rope_cos + (size_t)s * half + d);
      const f32x4 sn = vec4<float>::load(a.rope_sin + (size_t)s * half + d);
      AT* base = dst + ((size_t)(b * nheads + head) * a.S + s) * hd;
      vec4<AT>::store(base + d, x1 * cs - x2 * sn);
      vec4<AT>::store(base + half + d, x2 * cs + x1 * sn);
    }
    // V heads, transposed: each unit writes 8 consecutive positions of one d.
    const int per_head = hd * (BM / 8);
    for (int u = tid; u < kHeads * per_head; u += nt) {
      const int hh = u / per_head, rest = u % per_head;
      const int d = rest / (BM / 8), rg = (rest % (BM / 8)) * 8;
      const int col0 = n0 + hh * hd;
      if (col0 < k_end || col0 >= a.N) continue;
      const int head = (col0 - k_end) / hd;
      const int mf = m0 + rg;
      if (mf >= a.M) continue;
      const int bf = mf / a.S, sf = mf - bf * a.S;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = sC[(rg + e) * ldc + hh * hd + d];
      if (mf + 7 < a.M && sf + 7 < a.S && (sf & 7) == 0) {
        store8<AT>(vo + ((size_t)(bf * a.nkv + head) * hd + d) * a.s_pad + sf, v);
      } else {
        for (int e = 0; e < 8; ++e) {
          const int m = mf + e;
          if (m >= a.M) break;
          const int b = m / a.S, s = m - b * a.S;
          vo[((size_t)(b * a.nkv + head) * hd + d) * a.s_pad + s] = from_f32<AT>(v[e]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- MFMA core
__device__ __forceinline__ int swz(int r, int c) { return r * 64 + ((c ^ (r & 7)) << 3); }

__device__ __forceinline__ f16x8 i8x8_to_f16x8(uint32_t lo, uint32_t hi) {
  f16x8 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = (f16)(float)(int8_t)(lo >> (8 * e));
    o[4 + e] = (f16)(float)(int8_t)(hi >> (8 * e));
  }
  return o;
}

template <int BM, int BN, int WGM, int WGN, bool W8, int EPI>
__global__ __launch_bounds__(WGM* WGN * 64) void phi_gemm_mfma_kernel(GemmArgs a) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int BK = 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int STAGE = (BM + BN) * BK;  // f16 elements per stage
  constexpr int LDC = BN + 4;
  constexpr int SMEM = (2 * STAGE * 2 > BM * LDC * 4) ? 2 * STAGE * 2 : BM * LDC * 4;
  constexpr int CA = BM * 8 / NT;                      // A chunks per thread
  constexpr int CB = W8 ? BN * 4 / NT : BN * 8 / NT;   // W chunks per thread
  static_assert(CA * NT == BM * 8 && (W8 ? CB * NT == BN * 4 : CB * NT == BN * 8), "tile/threads");
  static_assert(TM * 32 == WM && TN * 32 == WN, "wave tile");

  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  f16* stage0 = reinterpret_cast<f16*>(smem);

  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  if (tile >= a.tiles_m * a.tiles_n) return;
  const int tm = tile % a.tiles_m, tn = tile / a.tiles_m;
  const int m0 = tm * BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  const f16* A = reinterpret_cast<const f16*>(a.A);
  const int K = a.K;

  // per-thread global sources (row pointers fixed over the K loop)
  const f16* a_src[CA];
  int a_dst[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int q = tid + i * NT, r = q >> 3, c = q & 7;
    const int gm = m0 + r < a.M ? m0 + r : a.M - 1;
    a_src[i] = A + (size_t)gm * K + c * 8;
    a_dst[i] = swz(r, c);
  }
  const char* w_src[CB];
  int w_dst[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int q = tid + i * NT;
    if constexpr (W8) {
      const int r = q >> 2, c = q & 3;
      w_src[i] = reinterpret_cast<const char*>(a.W) + (size_t)w_row<EPI, BN>(a, tn, r) * K + c * 16;
      w_dst[i] = BM * BK + swz(r, 2 * c);  // second chunk at swz(r, 2c + 1)
    } else {
      const int r = q >> 3, c = q & 7;
      w_src[i] = reinterpret_cast<const char*>(a.W) + ((size_t)w_row<EPI, BN>(a, tn, r) * K + c * 8) * 2;
      w_dst[i] = BM * BK + swz(r, c);
    }
  }

  i32x4 ra[CA], rw[CB];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CA; ++i) ra[i] = *reinterpret_cast<const i32x4*>(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < CB; ++i)
      rw[i] = *reinterpret_cast<const i32x4*>(w_src[i] + (W8 ? k0 : k0 * 2));
  };
  auto lstore = [&](f16* st) {
#pragma unroll
    for (int i = 0; i < CA; ++i) *reinterpret_cast<i32x4*>(st + a_dst[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      if constexpr (W8) {
        const int q = tid + i * NT, r = q >> 2, c = q & 3;
        *reinterpret_cast<f16x8*>(st + BM * BK + swz(r, 2 * c)) = i8x8_to_f16x8(rw[i][0], rw[i][1]);
        *reinterpret_cast<f16x8*>(st + BM * BK + swz(r, 2 * c + 1)) = i8x8_to_f16x8(rw[i][2], rw[i][3]);
      } else {
        *reinterpret_cast<i32x4*>(st + w_dst[i]) = rw[i];
      }
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  const int nk = K / BK;
  gload(0);
  lstore(stage0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    f16* cur = stage0 + (kt & 1) * STAGE;
    f16* nxt = stage0 + ((kt + 1) & 1) * STAGE;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      f16x8 af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WM + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const f16x8*>(cur + swz(r, c));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * WN + j * 32 + (lane & 31);
        bf[j] = *reinterpret_cast<const f16x8*>(cur + BM * BK + swz(r, c));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(nxt);
    __syncthreads();
  }

  // accumulators -> LDS tile (row = 8 (v / 4) + 4 (lane / 32) + v % 4, col = lane % 32)
  float* sC = reinterpret_cast<float*>(smem);
  const f16* sc16 = reinterpret_cast<const f16*>(a.scale);
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = wn * WN + j * 32 + (lane & 31);
    float s = 1.0f;
    if constexpr (W8) s = (float)sc16[w_row<EPI, BN>(a, tn, col)];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        sC[row * LDC + col] = acc[i][j][v] * s;
      }
    }
  }
  __syncthreads();
  gemm_epilogue<EPI, f16, BM, BN>(sC, LDC, m0, tn, a, tid, NT);
}

// ---------------------------------------------------------------- fp32 core
template <int BN, int EPI>
__global__ __launch_bounds__(256) void phi_gemm_simt_f32_kernel(GemmArgs a) {
  constexpr int BM = 32, BK = 32, NT = 256;
  constexpr int LDC = BN + 4;
  __shared__ float sA[BM][BK + 1];
  __shared__ float sW[BN][BK + 1];
  __shared__ __attribute__((aligned(16))) float sC[BM * LDC];
  const int tile = blockIdx.x;
  if (tile >= a.tiles_m * a.tiles_n) return;
  const int tm = tile % a.tiles_m, tn = tile / a.tiles_m;
  const int m0 = tm * BM;
  const int tid = threadIdx.x;
  const int r = tid >> 3, cl = tid & 7;
  const float* A = reinterpret_cast<const float*>(a.A);
  const float* W = reinterpret_cast<const float*>(a.W);
  float acc[BN / 8];
#pragma unroll
  for (int j = 0; j < BN / 8; ++j) acc[j] = 0.f;
  for (int k0 = 0; k0 < a.K; k0 += BK) {
    {
      const int ra = tid >> 3, ca = (tid & 7) * 4;
      const int gm = m0 + ra < a.M ? m0 + ra : a.M - 1;
      const f32x4 v = vec4<float>::load(A + (size_t)gm * a.K + k0 + ca);
#pragma unroll
      for (int e = 0; e < 4; ++e) sA[ra][ca + e] = v[e];
    }
    for (int q = tid; q < BN * 8; q += NT) {
      const int rw = q >> 3, cw = (q & 7) * 4;
      const f32x4 v = vec4<float>::load(W + (size_t)w_row<EPI, BN>(a, tn, rw) * a.K + k0 + cw);
#pragma unroll
      for (int e = 0; e < 4; ++e) sW[rw][cw + e] = v[e];
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < BK; ++kk) {
      const float av = sA[r][kk];
#pragma unroll
      for (int j = 0; j < BN / 8; ++j) acc[j] = fmaf(av, sW[cl + 8 * j][kk], acc[j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < BN / 8; ++j) sC[r * LDC + cl + 8 * j] = acc[j];
  __syncthreads();
  gemm_epilogue<EPI, float, BM, BN>(sC, LDC, m0, tn, a, tid, NT);
}

}  // namespace phi
