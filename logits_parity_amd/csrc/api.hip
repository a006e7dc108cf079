// C ABI of libphi: argument checks, workspace planning and the stream-ordered
// launch sequence of the prefill forward and of the decode attention.
#include <hip/hip_ext.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/phi.h"
#include "attention.hpp"
#include "common.hpp"
#include "decode.hpp"
#include "gemm.hpp"
#include "norm.hpp"

using namespace phi;

// Event pairs bracketing the launches of recorded forwards.
struct PhiProfile {
  bool enabled = false;
  std::vector<hipEvent_t> ev;  // 2 per launch slot
  std::vector<int> stage;      // stage of each used slot
  size_t used = 0;
};

struct phi_model {
  phi_config cfg;
  PhiProfile prof;
  std::vector<phi_layer_weights> layers;
  const void* embed;
  const void* final_norm;
  phi_linear lm_head;
  const float* rope_cos;  // [max_pos][head_dim / 2], in the caller's state buffer
  const float* rope_sin;
};

namespace {

constexpr int kMaxPos = 4096;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

phi_status launched() { return hipGetLastError() == hipSuccess ? PHI_OK : PHI_E_HIP; }

// ---------------------------------------------------------------- GEMM plans
// 8 waves, wave tile 128 x 64: twice the waves issuing the tile's copies of
// a 4-wave 128 x 128 layout (gate/up at 4096 tokens 12.6 -> 12.1 ms per
// forward, int8 13.3 -> 12.3 ms)
using CfgL = TileCfg<256, 256, 2, 4>;
// 8 compute waves of 64 x 64 (with 4 copy waves: 12 waves, 99 registers):
// two compute waves per SIMD, so one issues MFMAs while the other waits on
// LDS.  At 512 tokens, against 4 compute waves of 128 x 64: o_proj 0.585 ->
// 0.527, down 1.029 -> 0.977, gate/up 1.723 -> 1.692 ms per forward; 8 copy
// waves instead of 4 measured slower (0.544 / 1.018 / 1.712).
using CfgM = TileCfg<256, 128, 4, 2>;
using CfgS = TileCfg<128, 128, 2, 2>;   // wave tile 64 x 64
// 256 x 192 and 128 x 192 tiles run 8 waves (wave tiles 64 x 96 and 32 x 96,
// still one head per wave for the QKV epilogue): twice the waves issuing the
// tile's copies.  binary16 at 4096 tokens: o_proj 4.21 -> 3.36 ms, down
// 7.87 -> 7.05 ms, QKV 8.60 -> 8.08 ms per forward; 512 tokens: QKV 1.75 ->
// 1.64 ms.  int8 at 4 x 1024 (register-staged copies, 44 per stage padded to
// 6 per wave): o_proj 4.34 -> 3.62 ms, down 8.48 -> 7.83 ms.
using CfgQL8 = TileCfg<256, 192, 4, 2>;  // 8 waves, wave tile 64 x 96
using CfgQS8 = TileCfg<128, 192, 4, 2>;  // 8 waves, wave tile 32 x 96
using CfgQ128 = TileCfg<128, 256, 2, 2>;  // wave tile 64 x 128 (one 128-wide head per wave)
using CfgQ64 = TileCfg<128, 128, 2, 2>;   // wave tile 64 x 64 (one 64-wide head per wave)
// QKV below 1024 tokens with as many query as KV heads of width 96: a tile is
// one Q or K head plus half a V head (144 rows), so the tiles number
// nh + nkv per 128 tokens (256 at 512 tokens for 32 + 32 heads, one per CU,
// against 192 of 128 x 192), and move 15% fewer operand bytes each
using CfgQH = TileCfg<128, 144, 4, 1>;    // wave tile 32 x 144
using CfgR96 = TileCfg<256, 96, 4, 2>;    // wave tile 64 x 48 (short split-K residual GEMMs)
enum CfgId { C_L, C_M, C_S, C_QL, C_QS, C_Q128, C_Q64, C_QH, C_R96 };

struct GemmPlan {
  int cfg, tiles_m, tiles_n, splits, kpt, group_m;
};

// M-tiles per tile group when there are more M-tiles than that: the 32
// workgroups that run together on an XCD then cover a block of 8 x 4 tiles
// (12 distinct A and W tiles in its L2) instead of a column of all M-tiles.
constexpr int kGemmGroupM = 8;

constexpr int kCUs = 256;

inline void cfg_dims(int cfg, int& bm, int& bn) {
  switch (cfg) {
    case C_L: bm = 256; bn = 256; break;
    case C_M: bm = 256; bn = 128; break;
    case C_S: bm = 128; bn = 128; break;
    case C_QL: bm = 256; bn = 192; break;
    case C_Q128: bm = 128; bn = 256; break;
    case C_Q64: bm = 128; bn = 128; break;
    case C_QH: bm = 128; bn = 144; break;
    case C_R96: bm = 256; bn = 96; break;
    default: bm = 128; bn = 192; break;
  }
}

// Tile shape per GEMM role and token count: large wave tiles keep LDS traffic
// per MFMA low; at small M the residual GEMMs (N = hidden) have too few tiles
// for 256 CUs, so K is split into as many ranges as give one even round of
// workgroups (any count: at 512 tokens down takes 5, 240 workgroups of
// 256 x 128, and o_proj 4, 256 workgroups of 256 x 96).  int8 and binary16
// weights share the plans (binary16 copies go global -> LDS by DMA, int8
// through registers), except the head-and-a-half QKV tiles and the 256 x 96
// residual tiles (binary16 only, as measured).
GemmPlan plan_gemm(int epi, int M, int N, int K, bool w8, int hd = 96, int nh = 0, int nkv = 0) {
  GemmPlan p{};
  if (epi == EPI_QKV) {
    p.cfg = hd == 128 ? C_Q128 : (hd == 64 ? C_Q64 : (M >= 1024 ? C_QL : C_QS));
    // head-and-a-half tiles when they make one round of at most 256 workgroups
    if (p.cfg == C_QS && !w8 && nh == nkv && nh > 0 && (long)((M + 127) / 128) * (nh + nkv) <= kCUs) p.cfg = C_QH;
  } else if (epi == EPI_SILU) p.cfg = M >= 1024 ? C_L : C_M;
  else if (epi == EPI_F32) p.cfg = C_L;
  else {
    // 256 x 192 when the output width divides and it gives whole rounds of
    // 256 workgroups without splitting K (384 tiles of 256 x 128 would leave
    // the second round half empty); 256 x 128 otherwise
    p.cfg = C_M;
    const long t192 = (long)((M + 255) / 256) * (N / 192);
    if (N % 192 == 0 && t192 >= kCUs && t192 % kCUs == 0) p.cfg = C_QL;
    else if (!w8 && N % 96 == 0) {
      // K ranges shorter than 16 k-steps (o_proj at 512 tokens: 9.6 k-steps
      // on 240 workgroups of 256 x 128) lose more to each range's pipeline
      // fill and drain than 256 x 96 tiles lose to their 22% more operand
      // bytes per flop; those give one full round (4 splits of 64 tiles, 12
      // k-steps each at 512 tokens).  Measured per forward at 1 x 512:
      // o_proj 0.540 -> 0.505 ms; down (25.6 k-steps) keeps 256 x 128,
      // where 256 x 96 measured 0.943 -> 0.968 ms.
      const int tm = (M + 255) / 256, nk = K / 64;
      const int s128 = std::max(1, std::min(kCUs / (tm * ((N + 127) / 128)), nk / 4));
      if (s128 > 1 && nk / s128 < 16) p.cfg = C_R96;
    }
  }
  int bm, bn;
  cfg_dims(p.cfg, bm, bn);
  p.tiles_m = (M + bm - 1) / bm;
  p.tiles_n = epi == EPI_SILU ? (N / 2) / (bn / 2) : (p.cfg == C_QH ? nh + nkv : (N + bn - 1) / bn);
  const int nk = K / 64;
  int s = 1;
  // residual GEMMs: as many K splits as keep one round of at most 256
  // workgroups (one per CU) and at least 4 k-steps per split
  if (epi == EPI_RESID) s = std::max(1, std::min(kCUs / (p.tiles_m * p.tiles_n), nk / 4));
  p.kpt = (nk + s - 1) / s;
  p.splits = (nk + p.kpt - 1) / p.kpt;
  p.group_m = std::min(p.tiles_m, kGemmGroupM);
  return p;
}

// LDS stages of a tile.  Tiles whose two stages leave room for a second
// workgroup per CU keep 2 (the other workgroup covers the load latency);
// larger tiles take 3 when they fit in 152 KB.  int8 weights stage their
// copies in registers (two register sets over two LDS stages).
template <class C, bool W8>
constexpr int gemm_stages() {
  if (W8) return 2;
  constexpr int stage_bytes = C::BM * 64 * 2 + C::BN * 64 * (W8 ? 1 : 2);
  if (2 * stage_bytes <= 64 * 1024) return 2;
  return 3 * stage_bytes <= 152 * 1024 ? 3 : 2;
}

// Copy waves (4 extra waves that issue all global -> LDS copies) for the
// binary16 4-wave tiles of at most 128 x 64 per wave (measured 5% faster
// on the gate/up and residual GEMMs at 512 tokens), the 8-wave 256 x 128
// and 256 x 96 tiles, and the 8-wave
// 128 x 192 QKV tile (144 registers, so 12 waves fit): QKV at 512 tokens
// 1.595 -> 1.49 ms per forward.  Not for the 4-wave QKV tiles (their RoPE
// factors spill at 256 registers per lane), nor the other 8-wave tiles (the
// 256 x 192 residual tile spills at 168 registers and measured 19% slower).
// The 128 x 144 QKV tile gets 2: its 16 + 18 copies per stage split evenly
// only over two waves.
template <class C, bool W8, int EPI>
constexpr int gemm_copy_waves() {
  return ((!W8 && EPI != EPI_QKV && C::NW == 4 && C::WM * C::WN <= 8192) ||
          (!W8 && EPI != EPI_QKV && C::BM == 256 && (C::BN == 128 || C::BN == 96) && C::NW == 8) ||
          (!W8 && EPI == EPI_QKV && C::NW == 8 && C::BM == 128 && C::WN == 96)) ? 4
         : (!W8 && EPI == EPI_QKV && C::BN == 144) ? 2   // 34 copies per stage: 17 each
         : 0;
}

// Kernel launch.  With profiling events (ev non-null) the two events ride on
// the dispatch itself (hipExtLaunchKernelGGL), so their elapsed time is the
// kernel's own run time, as a kernel trace reports it; otherwise a plain launch.
#define PHI_LAUNCH(ev, kernel, grid, block, st, ...)                                                \
  do {                                                                                              \
    if (ev) hipExtLaunchKernelGGL(kernel, grid, block, 0, st, (ev)[0], (ev)[1], 0, __VA_ARGS__);   \
    else hipLaunchKernelGGL(kernel, grid, block, 0, st, __VA_ARGS__);                              \
  } while (0)

template <class C, bool W8, int EPI>
void launch_mfma(GemmArgs a, hipStream_t st, const hipEvent_t* ev) {
  const int units = a.tiles_m * a.tiles_n * a.splits;
  const int grid = (units + 7) / 8 * 8;
  constexpr int HW = gemm_copy_waves<C, W8, EPI>();
  PHI_LAUNCH(ev, (phi_gemm_mfma_kernel<C, W8, EPI, gemm_stages<C, W8>(), HW>), dim3(grid), dim3(C::NT + 64 * HW), st,
             a);
}

template <bool W8, int EPI>
void launch_cfg(int cfg, GemmArgs a, hipStream_t st, const hipEvent_t* ev) {
  using QL = CfgQL8;
  using QS = CfgQS8;
  if constexpr (EPI == EPI_QKV) {
    // the head width picks the kernel family first: a QKV kernel writes Q, K
    // and V^T with its own head width, so it never runs on another model's
    if (a.hd == 128) launch_mfma<CfgQ128, W8, EPI>(a, st, ev);
    else if (a.hd == 64) launch_mfma<CfgQ64, W8, EPI>(a, st, ev);
    else if (cfg == C_QL) launch_mfma<QL, W8, EPI>(a, st, ev);
    else if (cfg == C_QH && !W8 && a.nh == a.nkv && a.tiles_n == a.nh + a.nkv) launch_mfma<CfgQH, false, EPI>(a, st, ev);
    else launch_mfma<QS, W8, EPI>(a, st, ev);
  } else if constexpr (EPI == EPI_SILU) {
    if (cfg == C_L) launch_mfma<CfgL, W8, EPI>(a, st, ev);
    else launch_mfma<CfgM, W8, EPI>(a, st, ev);
  } else if constexpr (EPI == EPI_F32) {
    launch_mfma<CfgL, W8, EPI>(a, st, ev);
  } else {
    if (cfg == C_M) launch_mfma<CfgM, W8, EPI>(a, st, ev);
    else if (cfg == C_R96 && !W8) launch_mfma<CfgR96, false, EPI>(a, st, ev);
    else if (cfg == C_QL) launch_mfma<QL, W8, EPI>(a, st, ev);
    else launch_mfma<CfgS, W8, EPI>(a, st, ev);
  }
}

// ---------------------------------------------------------------- workspace
struct PrefillPlan {
  int T, S, s_pad;
  GemmPlan qkv, o, gu, down, lm;
  size_t off_x, off_xn, off_q, off_k, off_vt, off_attn, off_act, off_part, off_ids, total;
};

PrefillPlan plan_prefill(const phi_config& c, int batch, int seq) {
  PrefillPlan p;
  const size_t as = c.wtype == PHI_WT_F32 ? 4 : 2;
  p.T = batch * seq;
  p.S = seq;
  p.s_pad = (int)round_up((size_t)seq, 64);
  const int H = c.hidden, hd = c.head_dim, I = c.intermediate;
  const bool w8 = c.wtype == PHI_WT_I8;
  p.qkv = plan_gemm(EPI_QKV, p.T, (c.n_heads + 2 * c.n_kv_heads) * hd, H, w8, hd, c.n_heads, c.n_kv_heads);
  p.o = plan_gemm(EPI_RESID, p.T, H, c.n_heads * hd, w8);
  p.gu = plan_gemm(EPI_SILU, p.T, 2 * I, H, w8);
  p.down = plan_gemm(EPI_RESID, p.T, H, I, w8);
  p.lm = plan_gemm(EPI_F32, p.T, c.vocab, H, w8);
  const size_t T = (size_t)p.T;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = round_up(o + bytes, 256); return r; };
  p.off_x = take(T * H * 4);
  p.off_xn = take(T * H * as);
  p.off_q = take((size_t)batch * c.n_heads * seq * hd * as);
  p.off_k = take((size_t)batch * c.n_kv_heads * seq * hd * as);
  p.off_vt = take((size_t)batch * c.n_kv_heads * hd * p.s_pad * as);
  p.off_attn = take(T * c.n_heads * hd * as);
  p.off_act = take(T * (size_t)I * as);
  const int max_split = c.wtype == PHI_WT_F32 ? 0 : std::max(p.o.splits, p.down.splits);
  p.off_part = take(max_split > 1 ? (size_t)max_split * T * H * 2 : 0);  // binary16 partials
  p.off_ids = take(T * 4);  // the device copy of host ids (phi_prefill_logits_host_ids)
  p.total = o;
  return p;
}

// Token rows times the widest GEMM operand row (hidden, intermediate or
// attention width) stay within int32 element offsets.
bool rows_fit(const phi_config& c, long long rows) {
  const long long w = std::max({(long long)c.hidden, (long long)c.intermediate, (long long)c.n_heads * c.head_dim});
  return rows >= 1 && rows * w < (1ll << 31) && rows * c.vocab < (1ll << 40);
}

// The GEMM kernels form operand offsets (row * K + column) in int32: every
// weight's rows x K, and the activation rows x K of a call, must stay below 2^31.
constexpr long long kMaxElems = 1ll << 31;
inline bool elems_fit(long long rows, long long k) { return rows >= 1 && k >= 1 && rows * k < kMaxElems; }

// head_dim 64 and 128 run on the MFMA paths only (binary16 and int8 weights).
// Every product below is formed in 64 bits from fields bounded first.
bool check_config(const phi_config* c) {
  const bool hd_ok = c->head_dim == 96 || ((c->head_dim == 64 || c->head_dim == 128) && c->wtype != PHI_WT_F32);
  if (!(c->n_layers >= 1 && c->hidden >= 64 && c->hidden % 64 == 0 && hd_ok && c->n_heads >= 1 &&
        c->n_kv_heads >= 1 && c->n_heads <= (1 << 16) && c->n_heads % c->n_kv_heads == 0 &&
        c->intermediate >= 128 && c->intermediate % 128 == 0 && c->hidden <= kNormMaxChunks * 4 * kNormThreads &&
        c->vocab >= 4 && c->vocab % 4 == 0 && c->max_pos >= 1 && c->max_pos <= kMaxPos))
    return false;
  const long long H = c->hidden, hd = c->head_dim, I = c->intermediate;
  const long long attn_w = (long long)c->n_heads * hd, qkv_rows = ((long long)c->n_heads + 2ll * c->n_kv_heads) * hd;
  return attn_w % 64 == 0 && elems_fit(qkv_rows, H) && elems_fit(H, attn_w) && elems_fit(2 * I, H) &&
         elems_fit(H, I) && elems_fit(c->vocab, H);
}

// ---------------------------------------------------------------- GEMM dispatch
template <int EPI>
struct SimtCfg { static constexpr int BN = 64; };
template <>
struct SimtCfg<EPI_QKV> { static constexpr int BN = 96; };

// Runs one GEMM; returns the number of K splits whose partials the caller
// must reduce (0 when the epilogue completed the result).
template <int EPI>
phi_status gemm(int wtype, GemmArgs a, const GemmPlan& p, hipStream_t st, int* partials = nullptr,
                const hipEvent_t* ev = nullptr) {
  if (partials) *partials = 0;
  if (wtype == PHI_WT_F32) {
    constexpr int BN = SimtCfg<EPI>::BN;
    a.tiles_m = (a.M + 31) / 32;
    a.tiles_n = EPI == EPI_SILU ? (a.N / 2) / (BN / 2) : (a.N + BN - 1) / BN;
    a.splits = 1;
    const int tiles = a.tiles_m * a.tiles_n;
    PHI_LAUNCH(ev, (phi_gemm_simt_f32_kernel<BN, EPI>), dim3(tiles), dim3(256), st, a);
    return launched();
  }
  a.tiles_m = p.tiles_m;
  a.tiles_n = p.tiles_n;
  a.splits = p.splits;
  a.kt_per_split = p.kpt;
  a.group_m = p.group_m;
  const bool w8 = wtype == PHI_WT_I8;
  if constexpr (EPI == EPI_RESID) {
    if (p.splits > 1) {
      if (partials) *partials = p.splits;
      if (w8) launch_cfg<true, EPI_PARTIAL>(p.cfg, a, st, ev);
      else launch_cfg<false, EPI_PARTIAL>(p.cfg, a, st, ev);
      return launched();
    }
  }
  if (w8) launch_cfg<true, EPI>(p.cfg, a, st, ev);
  else launch_cfg<false, EPI>(p.cfg, a, st, ev);
  return launched();
}

// Workgroups of the shared-key-block attention at which it beats the split
// kernel (measured: 448 and more win at head_dim 64 to 128, 256 lose).
constexpr long kAttnSharedMinWorkgroups = 384;
// The shared-key-block kernel on 8 waves (256 queries per workgroup): from
// S = 2048 with at least 256 workgroups.  At 1 x 4096: 4.75 -> 4.55-4.60 ms
// of attention per forward; at 4 x 1024 the 4-wave form stays faster (a
// 256-query block wastes more of the causal diagonal at short S).
constexpr long kAttnShared8MinWorkgroups = 256;
constexpr int kAttnShared8MinSeq = 2048;

phi_status attention(bool f32, AttnArgs a, int batch, int hd, hipStream_t st, const hipEvent_t* ev = nullptr) {
  a.scale_log2 = kLog2e / sqrtf((float)hd);
  if (f32) {
    PHI_LAUNCH(ev, (phi_attn_prefill_f32_kernel), dim3((a.S + 63) / 64, a.nh, batch), dim3(64), st, a);
    return launched();
  }
  // Shared key blocks (128 queries per workgroup) once there are enough
  // workgroups to fill the chip at two per CU; split keys (32 queries per
  // workgroup, four times the workgroups) below that.
  const int heads = a.nh * batch;
  if (a.S >= kAttnShared8MinSeq && (long)heads * ((a.S + 255) / 256) >= kAttnShared8MinWorkgroups) {
    const dim3 grid(heads, (a.S + 255) / 256);
    if (hd == 128) PHI_LAUNCH(ev, (phi_attn_prefill_lds_kernel<128, 8>), grid, dim3(512), st, a);
    else if (hd == 64) PHI_LAUNCH(ev, (phi_attn_prefill_lds_kernel<64, 8>), grid, dim3(512), st, a);
    else PHI_LAUNCH(ev, (phi_attn_prefill_lds_kernel<96, 8>), grid, dim3(512), st, a);
    return launched();
  }
  if ((long)heads * ((a.S + 127) / 128) >= kAttnSharedMinWorkgroups) {
    const dim3 grid(heads, (a.S + 127) / 128);
    if (hd == 128) PHI_LAUNCH(ev, (phi_attn_prefill_lds_kernel<128>), grid, dim3(256), st, a);
    else if (hd == 64) PHI_LAUNCH(ev, (phi_attn_prefill_lds_kernel<64>), grid, dim3(256), st, a);
    else PHI_LAUNCH(ev, (phi_attn_prefill_lds_kernel<96>), grid, dim3(256), st, a);
    return launched();
  }
  const dim3 grid(heads, (a.S + 31) / 32);
  if (hd == 128) PHI_LAUNCH(ev, (phi_attn_prefill_f16_kernel<128, 4>), grid, dim3(256), st, a);
  else if (hd == 64) PHI_LAUNCH(ev, (phi_attn_prefill_f16_kernel<64, 4>), grid, dim3(256), st, a);
  else PHI_LAUNCH(ev, (phi_attn_prefill_f16_kernel<96, 4>), grid, dim3(256), st, a);
  return launched();
}

template <class ET, class AT>
phi_status norm(bool embed, NormArgs a, hipStream_t st, const hipEvent_t* ev = nullptr) {
  // chunks per thread: hidden <= kNormMaxChunks * 1024 is checked at load
  switch ((a.H + 4 * kNormThreads - 1) / (4 * kNormThreads)) {
#define PHI_NORM_CASE(CH)                                                                                      \
  case CH:                                                                                                     \
    if (embed) PHI_LAUNCH(ev, (phi_norm_kernel<ET, AT, true, CH>), dim3(a.T), dim3(kNormThreads), st, a);       \
    else if (a.nsplit == 0) PHI_LAUNCH(ev, (phi_norm_kernel<ET, AT, false, CH, 0>), dim3(a.T), dim3(kNormThreads), st, a); \
    else if (a.nsplit == 5) PHI_LAUNCH(ev, (phi_norm_kernel<ET, AT, false, CH, 5>), dim3(a.T), dim3(kNormThreads), st, a); \
    else if (a.nsplit == 4) PHI_LAUNCH(ev, (phi_norm_kernel<ET, AT, false, CH, 4>), dim3(a.T), dim3(kNormThreads), st, a); \
    else PHI_LAUNCH(ev, (phi_norm_kernel<ET, AT, false, CH>), dim3(a.T), dim3(kNormThreads), st, a);            \
    break;
    PHI_NORM_CASE(1) PHI_NORM_CASE(2) PHI_NORM_CASE(3) PHI_NORM_CASE(4)
    PHI_NORM_CASE(5) PHI_NORM_CASE(6) PHI_NORM_CASE(7) PHI_NORM_CASE(8)
#undef PHI_NORM_CASE
    default: return PHI_E_SHAPE;
  }
  return launched();
}

// Records the start event of a launch slot when profiling (no-op otherwise).
struct StageTimer {
  PhiProfile* p;
  hipStream_t st;
  size_t slot = 0;
  bool on = false;
  void begin(int stage) {
    on = p->enabled;
    if (!on) return;
    slot = p->used++;
    p->stage[slot] = stage;
    (void)hipEventRecord(p->ev[2 * slot], st);
  }
  void end() {
    if (on) (void)hipEventRecord(p->ev[2 * slot + 1], st);
  }
  // A stage of one kernel: its events go to the dispatch (PHI_LAUNCH) and
  // time the kernel alone; nullptr when profiling is off.
  const hipEvent_t* dispatch(int stage) {
    on = false;
    if (!p->enabled) return nullptr;
    slot = p->used++;
    p->stage[slot] = stage;
    return &p->ev[2 * slot];
  }
};

// Launch slots of one forward: embed + per layer (qkv, attn, o, norm, gate_up, down, norm) + lm_head.
inline size_t launches_per_forward(const phi_config& c) { return 2 + 7 * (size_t)c.n_layers; }

// Cache fill of layer l from the QKV outputs in the prefill workspace.
phi_status kv_fill(const phi_kv_cache* cache, int l, const void* k, const void* vt, int batch, int seq, int s_pad,
                   int n_kv_heads, hipStream_t st) {
  KvFillArgs f{};
  f.k = reinterpret_cast<const f16*>(k);
  f.vt = reinterpret_cast<const f16*>(vt);
  f.v_scale = cache->v_scale + (size_t)l * n_kv_heads;
  f.block_table = cache->block_table;
  f.k_pool = reinterpret_cast<f16*>(cache->k_pools[l]);
  f.v_pool = reinterpret_cast<uint8_t*>(cache->v_pools[l]);
  f.B = batch;
  f.Hkv = n_kv_heads;
  f.S = seq;
  f.s_pad = s_pad;
  f.n_pages = cache->n_pages;
  f.max_pages = cache->max_pages;
  const size_t threads = (size_t)batch * n_kv_heads * seq * 16;
  hipLaunchKernelGGL(phi_kv_fill_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, f);
  return launched();
}

template <class AT>
phi_status forward(const phi_model* m, const int32_t* ids, int batch, int seq, float* logits, char* ws,
                   hipStream_t st, const phi_kv_cache* cache = nullptr) {
  StageTimer tm{const_cast<PhiProfile*>(&m->prof), st};
  const phi_config& c = m->cfg;
  const PrefillPlan p = plan_prefill(c, batch, seq);
  const int T = p.T, H = c.hidden, I = c.intermediate, hd = c.head_dim;
  float* x = reinterpret_cast<float*>(ws + p.off_x);
  void* xn = ws + p.off_xn;
  void* attn = ws + p.off_attn;
  void* act = ws + p.off_act;
  float* part = reinterpret_cast<float*>(ws + p.off_part);
  const int wt = c.wtype;

  NormArgs na{};
  na.ids = ids;
  na.embed = m->embed;
  na.x = x;
  na.xn = xn;
  na.part = reinterpret_cast<const f16*>(part);
  na.T = T;
  na.H = H;
  na.V = c.vocab;
  na.eps = c.rms_eps;
  na.gain = m->layers[0].ln1;
  phi_status s = norm<AT, AT>(true, na, st, tm.dispatch(PHI_PROF_EMBED));
  if (s) return s;

  GemmArgs base{};
  base.M = T;
  base.S = seq;
  base.s_pad = p.s_pad;
  base.nh = c.n_heads;
  base.nkv = c.n_kv_heads;
  base.hd = hd;
  base.rope_cos = m->rope_cos;
  base.rope_sin = m->rope_sin;
  base.max_pos = c.max_pos;

  AttnArgs aa{};
  aa.q = ws + p.off_q;
  aa.k = ws + p.off_k;
  aa.vt = ws + p.off_vt;
  aa.out = attn;
  aa.S = seq;
  aa.s_pad = p.s_pad;
  aa.nh = c.n_heads;
  aa.nkv = c.n_kv_heads;

  for (int l = 0; l < c.n_layers; ++l) {
    const phi_layer_weights& L = m->layers[l];
    GemmArgs g = base;
    g.A = xn;
    g.W = L.qkv.w;
    g.scale = L.qkv.scale;
    g.N = (c.n_heads + 2 * c.n_kv_heads) * hd;
    g.K = H;
    g.q = const_cast<void*>(aa.q);
    g.k = const_cast<void*>(aa.k);
    g.vt = const_cast<void*>(aa.vt);
    g.bias = reinterpret_cast<const f16*>(L.qkv_bias);
    if (cache) {  // the stage also fills the cache: events around both launches
      tm.begin(PHI_PROF_QKV);
      s = gemm<EPI_QKV>(wt, g, p.qkv, st);
      if (!s) s = kv_fill(cache, l, aa.k, aa.vt, batch, seq, p.s_pad, c.n_kv_heads, st);
      tm.end();
    } else {
      s = gemm<EPI_QKV>(wt, g, p.qkv, st, nullptr, tm.dispatch(PHI_PROF_QKV));
    }
    if (s) return s;

    s = attention(wt == PHI_WT_F32, aa, batch, hd, st, tm.dispatch(PHI_PROF_ATTN));
    if (s) return s;

    g = base;
    g.A = attn;
    g.W = L.o.w;
    g.scale = L.o.scale;
    g.N = H;
    g.K = c.n_heads * hd;
    g.x = x;
    g.ldx = H;
    g.out = part;
    s = gemm<EPI_RESID>(wt, g, p.o, st, &na.nsplit, tm.dispatch(PHI_PROF_O));
    if (s) return s;

    na.gain = L.ln2;
    s = norm<AT, AT>(false, na, st, tm.dispatch(PHI_PROF_NORM));
    if (s) return s;

    g = base;
    g.A = xn;
    g.W = L.gate_up.w;
    g.scale = L.gate_up.scale;
    g.N = 2 * I;
    g.K = H;
    g.act = act;
    g.ld_act = I;
    s = gemm<EPI_SILU>(wt, g, p.gu, st, nullptr, tm.dispatch(PHI_PROF_GATE_UP));
    if (s) return s;

    g = base;
    g.A = act;
    g.W = L.down.w;
    g.scale = L.down.scale;
    g.N = H;
    g.K = I;
    g.x = x;
    g.ldx = H;
    g.out = part;
    s = gemm<EPI_RESID>(wt, g, p.down, st, &na.nsplit, tm.dispatch(PHI_PROF_DOWN));
    if (s) return s;

    na.gain = l + 1 < c.n_layers ? m->layers[l + 1].ln1 : m->final_norm;
    s = norm<AT, AT>(false, na, st, tm.dispatch(PHI_PROF_NORM));
    if (s) return s;
  }

  GemmArgs g = base;
  g.A = xn;
  g.W = m->lm_head.w;
  g.scale = m->lm_head.scale;
  g.N = c.vocab;
  g.K = H;
  g.out = logits;
  g.ldo = c.vocab;
  return gemm<EPI_F32>(wt, g, p.lm, st, nullptr, tm.dispatch(PHI_PROF_LM_HEAD));
}

// ---------------------------------------------------------------- decode plan
struct DecodePlan {
  int n_split, pages_per_split, waves;
  size_t off_ml, total;
};

// Pages per split: the largest of 256, 128, 64, 32, 16 that still gives at
// least 320 workgroups (more than one per CU); 16 below that.  Long splits
// amortise each workgroup's start-up (table and query loads, the first
// page's latency) and the merge; one split per sequence skips the merge
// launch.  (At most 256 pages per split on 4 waves: 64 per wave, one table
// entry per lane.)  Where that takes several splits, one split on 8 waves
// (up to 512 pages) keeps the pages per wave and needs no merge launch:
// 16 x 8192 tokens 94.2-95.6 -> 88.7 us (160 workgroups of 512 pages).
// One split per sequence on 8-wave workgroups replaces a multi-split plan
// when the context fits one split (<= 512 pages: 64 per wave) and the
// (sequence, KV head) pairs fill at least half the CUs.  Measured at 40/10
// heads: 16 x 4096 51-53 -> 47-48 us, 24 x 8192 132-134 -> 130 us; below the
// cut the split plan wins (12 x 8192: 72 against 82 us, 8 x 8192: 53 against 77).
constexpr long kDecode8MinUnits = 128;
DecodePlan plan_decode(int batch, int n_q_heads, int n_kv_heads, int max_ctx) {
  DecodePlan p;
  const int np = (max_ctx + 15) / 16;
  const long units = (long)batch * n_kv_heads;
  int pps = 16;
  for (int cand : {256, 128, 64, 32}) {
    if (units * ((np + cand - 1) / cand) >= 320) {
      pps = cand;
      break;
    }
  }
  p.pages_per_split = pps;
  p.n_split = (np + pps - 1) / pps;
  p.waves = 4;
  if (p.n_split > 1 && np <= 512 && units >= kDecode8MinUnits) {
    p.pages_per_split = np;
    p.n_split = 1;
    p.waves = 8;
  }
  const size_t parts = (size_t)batch * n_q_heads * p.n_split;
  p.off_ml = round_up(parts * 128 * 4, 256);
  p.total = p.off_ml + round_up(parts * 2 * 4, 256);
  return p;
}


// Launch of split-KV decode attention + merge (arguments already checked).
phi_status decode_attention(const void* q, const void* k_pool, const void* v_pool, const float* v_scale,
                            const int32_t* block_table, const int32_t* ctx_lens, int batch, int n_q_heads,
                            int n_kv_heads, int n_pages, int max_pages, int max_ctx, float sm_scale, void* out,
                            void* workspace, const DecodePlan& p, hipStream_t st) {
  DecodeArgs a{};
  a.q = reinterpret_cast<const f16*>(q);
  a.k_pool = reinterpret_cast<const f16*>(k_pool);
  a.v_pool = reinterpret_cast<const uint8_t*>(v_pool);
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.ctx_lens = ctx_lens;
  a.part_o = reinterpret_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + p.off_ml);
  a.out = reinterpret_cast<f16*>(out);
  a.B = batch;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.n_pages = n_pages;
  a.max_pages = max_pages;
  a.n_split = p.n_split;
  a.pages_per_split = p.pages_per_split;
  a.max_ctx = max_ctx;
  a.scale_log2 = sm_scale * kLog2e;
  const dim3 grid(p.n_split, n_kv_heads, batch);
  if (p.waves == 8) {
    switch (n_q_heads / n_kv_heads) {
      case 1: hipLaunchKernelGGL((phi_decode_stream_kernel<1, 2, 8>), grid, dim3(512), 0, st, a); break;
      case 2: hipLaunchKernelGGL((phi_decode_stream_kernel<2, 2, 8>), grid, dim3(512), 0, st, a); break;
      case 4: hipLaunchKernelGGL((phi_decode_stream_kernel<4, 2, 8>), grid, dim3(512), 0, st, a); break;
      default: hipLaunchKernelGGL((phi_decode_stream_kernel<8, 2, 8>), grid, dim3(512), 0, st, a); break;
    }
  } else {
    switch (n_q_heads / n_kv_heads) {
      case 1: hipLaunchKernelGGL((phi_decode_stream_kernel<1, 2>), grid, dim3(256), 0, st, a); break;
      case 2: hipLaunchKernelGGL((phi_decode_stream_kernel<2, 2>), grid, dim3(256), 0, st, a); break;
      case 4: hipLaunchKernelGGL((phi_decode_stream_kernel<4, 2>), grid, dim3(256), 0, st, a); break;
      default: hipLaunchKernelGGL((phi_decode_stream_kernel<8, 2>), grid, dim3(256), 0, st, a); break;
    }
  }
  if (hipGetLastError() != hipSuccess) return PHI_E_HIP;
  if (p.n_split > 1) hipLaunchKernelGGL(phi_decode_merge_kernel, dim3(batch * n_q_heads), dim3(128), 0, st, a);
  return launched();
}

// Launch of the one-token cache write (arguments already checked, batch >= 1).
phi_status kv_append(const void* k_new, const void* v_new, const float* v_scale, const int32_t* block_table,
                     const int32_t* positions, int batch, int n_kv_heads, int n_pages, int max_pages, void* k_pool,
                     void* v_pool, hipStream_t st) {
  KvAppendArgs a{};
  a.k_new = reinterpret_cast<const f16*>(k_new);
  a.v_new = reinterpret_cast<const f16*>(v_new);
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.positions = positions;
  a.k_pool = reinterpret_cast<f16*>(k_pool);
  a.v_pool = reinterpret_cast<uint8_t*>(v_pool);
  a.B = batch;
  a.Hkv = n_kv_heads;
  a.n_pages = n_pages;
  a.max_pages = max_pages;
  const int rows = batch * n_kv_heads;
  hipLaunchKernelGGL(phi_kv_append_kernel, dim3((rows + 15) / 16), dim3(256), 0, st, a);
  return launched();
}

// ---------------------------------------------------------------- decode step
struct DecodeStepPlan {
  GemmPlan qkv, o, gu, down, lm;
  DecodePlan att;
  size_t off_x, off_xn, off_q, off_k, off_v, off_attn, off_act, off_part, off_ctx, off_att, total;
};

DecodeStepPlan plan_decode_step(const phi_config& c, int batch, int max_ctx) {
  DecodeStepPlan p;
  const int B = batch, H = c.hidden, hd = c.head_dim, I = c.intermediate;
  const bool w8 = c.wtype == PHI_WT_I8;
  p.qkv = plan_gemm(EPI_QKV, B, (c.n_heads + 2 * c.n_kv_heads) * hd, H, w8, hd);
  p.o = plan_gemm(EPI_RESID, B, H, c.n_heads * hd, w8);
  p.gu = plan_gemm(EPI_SILU, B, 2 * I, H, w8);
  p.down = plan_gemm(EPI_RESID, B, H, I, w8);
  p.lm = plan_gemm(EPI_F32, B, c.vocab, H, w8);
  p.att = plan_decode(B, c.n_heads, c.n_kv_heads, max_ctx);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = round_up(o + bytes, 256); return r; };
  p.off_x = take((size_t)B * H * 4);
  p.off_xn = take((size_t)B * H * 2);
  p.off_q = take((size_t)B * c.n_heads * hd * 2);
  p.off_k = take((size_t)B * c.n_kv_heads * hd * 2);
  p.off_v = take((size_t)B * c.n_kv_heads * hd * 2);
  p.off_attn = take((size_t)B * c.n_heads * hd * 2);
  p.off_act = take((size_t)B * I * 2);
  const int max_split = std::max(p.o.splits, p.down.splits);
  p.off_part = take(max_split > 1 ? (size_t)max_split * B * H * 2 : 0);  // binary16 partials
  p.off_ctx = take((size_t)B * 4);
  p.off_att = take(p.att.total);
  p.total = o;
  return p;
}

// One token per sequence through every layer with the K16/V8 cache.  The
// QKV GEMM sees S = 1 (each row its own sequence) and s_pad = 1, so its
// V^T output is the row-major [B][n_kv_heads][hd] that the cache write takes.
phi_status decode_step(const phi_model* m, const int32_t* ids, const int32_t* positions, int batch, int max_ctx,
                       const phi_kv_cache* cache, float* logits, char* ws, hipStream_t st) {
  const phi_config& c = m->cfg;
  const DecodeStepPlan p = plan_decode_step(c, batch, max_ctx);
  const int B = batch, H = c.hidden, I = c.intermediate, hd = c.head_dim;
  float* x = reinterpret_cast<float*>(ws + p.off_x);
  void* xn = ws + p.off_xn;
  void* q = ws + p.off_q;
  void* k = ws + p.off_k;
  void* v = ws + p.off_v;
  void* attn = ws + p.off_attn;
  void* act = ws + p.off_act;
  float* part = reinterpret_cast<float*>(ws + p.off_part);
  int32_t* ctx = reinterpret_cast<int32_t*>(ws + p.off_ctx);
  const int wt = c.wtype;

  hipLaunchKernelGGL(phi_ctx_from_pos_kernel, dim3((B + 255) / 256), dim3(256), 0, st, positions, ctx, B, max_ctx);
  phi_status s = launched();
  if (s) return s;

  NormArgs na{};
  na.ids = ids;
  na.embed = m->embed;
  na.x = x;
  na.xn = xn;
  na.part = reinterpret_cast<const f16*>(part);
  na.T = B;
  na.H = H;
  na.V = c.vocab;
  na.eps = c.rms_eps;
  na.gain = m->layers[0].ln1;
  if ((s = norm<f16, f16>(true, na, st))) return s;

  GemmArgs base{};
  base.M = B;
  base.S = 1;
  base.s_pad = 1;
  base.nh = c.n_heads;
  base.nkv = c.n_kv_heads;
  base.hd = hd;
  base.rope_cos = m->rope_cos;
  base.rope_sin = m->rope_sin;
  base.pos = positions;
  base.max_pos = c.max_pos;
  const float sm_scale = 1.0f / sqrtf((float)hd);

  for (int l = 0; l < c.n_layers; ++l) {
    const phi_layer_weights& L = m->layers[l];
    GemmArgs g = base;
    g.A = xn;
    g.W = L.qkv.w;
    g.scale = L.qkv.scale;
    g.N = (c.n_heads + 2 * c.n_kv_heads) * hd;
    g.K = H;
    g.q = q;
    g.k = k;
    g.vt = v;
    g.bias = reinterpret_cast<const f16*>(L.qkv_bias);
    if ((s = gemm<EPI_QKV>(wt, g, p.qkv, st))) return s;
    const float* vs = cache->v_scale + (size_t)l * c.n_kv_heads;
    if ((s = kv_append(k, v, vs, cache->block_table, positions, B, c.n_kv_heads, cache->n_pages,
                       cache->max_pages, cache->k_pools[l], cache->v_pools[l], st)))
      return s;
    if ((s = decode_attention(q, cache->k_pools[l], cache->v_pools[l], vs, cache->block_table, ctx, B, c.n_heads,
                              c.n_kv_heads, cache->n_pages, cache->max_pages, max_ctx, sm_scale, attn,
                              ws + p.off_att, p.att, st)))
      return s;

    g = base;
    g.A = attn;
    g.W = L.o.w;
    g.scale = L.o.scale;
    g.N = H;
    g.K = c.n_heads * hd;
    g.x = x;
    g.ldx = H;
    g.out = part;
    if ((s = gemm<EPI_RESID>(wt, g, p.o, st, &na.nsplit))) return s;
    na.gain = L.ln2;
    if ((s = norm<f16, f16>(false, na, st))) return s;

    g = base;
    g.A = xn;
    g.W = L.gate_up.w;
    g.scale = L.gate_up.scale;
    g.N = 2 * I;
    g.K = H;
    g.act = act;
    g.ld_act = I;
    if ((s = gemm<EPI_SILU>(wt, g, p.gu, st))) return s;

    g = base;
    g.A = act;
    g.W = L.down.w;
    g.scale = L.down.scale;
    g.N = H;
    g.K = I;
    g.x = x;
    g.ldx = H;
    g.out = part;
    if ((s = gemm<EPI_RESID>(wt, g, p.down, st, &na.nsplit))) return s;
    na.gain = l + 1 < c.n_layers ? m->layers[l + 1].ln1 : m->final_norm;
    if ((s = norm<f16, f16>(false, na, st))) return s;
  }

  GemmArgs g = base;
  g.A = xn;
  g.W = m->lm_head.w;
  g.scale = m->lm_head.scale;
  g.N = c.vocab;
  g.K = H;
  g.out = logits;
  g.ldo = c.vocab;
  return gemm<EPI_F32>(wt, g, p.lm, st);
}

// Model and cache checks shared by the cached entry points.
phi_status check_cache(const phi_model* m, const phi_kv_cache* cache) {
  const phi_config& c = m->cfg;
  const int G = c.n_heads / c.n_kv_heads;
  if (c.head_dim != 128 || c.wtype == PHI_WT_F32 || (G != 1 && G != 2 && G != 4 && G != 8)) return PHI_E_SHAPE;
  if (!cache->k_pools || !cache->v_pools || !cache->v_scale || !cache->block_table) return PHI_E_NULL;
  if (cache->page_size != 16 || cache->n_pages < 1 || cache->max_pages < 1) return PHI_E_SHAPE;
  if ((long long)cache->n_pages * c.n_kv_heads * 16 * 128 * 2 > (1ll << 40)) return PHI_E_SHAPE;
  for (int l = 0; l < c.n_layers; ++l) {
    if (!cache->k_pools[l] || !cache->v_pools[l]) return PHI_E_NULL;
    if (!aligned16(cache->k_pools[l]) || !aligned16(cache->v_pools[l])) return PHI_E_ALIGN;
  }
  return PHI_OK;
}
}  // namespace

// Split partials of attn_decode_k16v8_noalloc: a fixed device array, one copy
// per GPU, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: only its per-device address from
// hipGetSymbolAddress (decode_scratch below) is ever passed to a kernel.
static __device__ __attribute__((aligned(256))) char scratch[PHI_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, resolved once per device
// (with that device current) on its first use.
phi_status decode_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PHI_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PHI_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PHI_OK;
}

// Host checks shared by the decode-attention entry points; on success *plan
// holds the split plan.
phi_status check_decode_args(const void* q, const void* k_pool, const void* v_pool, const float* v_scale,
                             const int32_t* block_table, const int32_t* ctx_lens, const void* out, int32_t batch,
                             int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                             int32_t n_pages, int32_t max_pages, int32_t max_ctx, float sm_scale, DecodePlan* plan) {
  if (!q || !k_pool || !v_pool || !v_scale || !block_table || !ctx_lens || !out) return PHI_E_NULL;
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || head_dim != 128 ||
      page_size != 16 || n_pages < 1 || max_pages < 1 || batch > (1 << 20) || n_q_heads > (1 << 12))
    return PHI_E_SHAPE;
  const int G = n_q_heads / n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PHI_E_SHAPE;
  if (max_ctx < 1 || (long long)max_ctx > (long long)max_pages * page_size || !(sm_scale > 0.f)) return PHI_E_RANGE;
  if ((long long)n_pages * n_kv_heads * 16 * 128 * 2 > (1ll << 40)) return PHI_E_SHAPE;
  *plan = plan_decode(batch, n_q_heads, n_kv_heads, max_ctx);
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out)) return PHI_E_ALIGN;
  return PHI_OK;
}

}  // namespace

extern "C" {

const char* phi_strerror(int32_t s) {
  switch (s) {
    case PHI_OK: return "ok";
    case PHI_E_NULL: return "null pointer argument";
    case PHI_E_SHAPE: return "unsupported shape";
    case PHI_E_DTYPE: return "unsupported weight type";
    case PHI_E_RANGE: return "value out of range";
    case PHI_E_WORKSPACE: return "workspace or state buffer too small";
    case PHI_E_ALIGN: return "device pointer not 16-byte aligned";
    case PHI_E_HIP: return "HIP call or kernel launch failed";
    default: return "unknown status";
  }
}

size_t phi_state_bytes(const phi_config* cfg) {
  if (!cfg || cfg->max_pos < 1 || cfg->head_dim < 2) return 0;
  return 2 * (size_t)cfg->max_pos * (cfg->head_dim / 2) * sizeof(float);
}

phi_status phi_load_fused(const phi_config* cfg, const phi_weights* w, void* state, size_t state_bytes,
                          void* stream, phi_model** out) {
  if (!cfg || !w || !state || !out || !w->layers || !w->embed || !w->final_norm || !w->lm_head.w)
    return PHI_E_NULL;
  if (cfg->wtype != PHI_WT_F32 && cfg->wtype != PHI_WT_F16 && cfg->wtype != PHI_WT_I8) return PHI_E_DTYPE;
  if (!check_config(cfg)) return PHI_E_SHAPE;
  if (!(cfg->rms_eps > 0.f) || !(cfg->rope_theta > 0.f)) return PHI_E_RANGE;
  if (state_bytes < phi_state_bytes(cfg)) return PHI_E_WORKSPACE;
  const bool i8 = cfg->wtype == PHI_WT_I8;
  auto lin_ok = [&](const phi_linear& l) { return l.w && (i8 ? l.scale != nullptr : l.scale == nullptr); };
  if (!lin_ok(w->lm_head)) return PHI_E_NULL;
  if (!aligned16(state) || !aligned16(w->embed) || !aligned16(w->final_norm) || !aligned16(w->lm_head.w) ||
      !aligned16(w->lm_head.scale))
    return PHI_E_ALIGN;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const phi_layer_weights& L = w->layers[l];
    if (!L.ln1 || !L.ln2 || !lin_ok(L.qkv) || !lin_ok(L.o) || !lin_ok(L.gate_up) || !lin_ok(L.down))
      return PHI_E_NULL;
    if (L.qkv_bias && cfg->wtype == PHI_WT_F32) return PHI_E_DTYPE;  // the float32 path has no bias
    if (!aligned16(L.qkv_bias)) return PHI_E_ALIGN;
    const void* ps[] = {L.ln1, L.ln2, L.qkv.w, L.qkv.scale, L.o.w, L.o.scale,
                        L.gate_up.w, L.gate_up.scale, L.down.w, L.down.scale};
    for (const void* p : ps)
      if (!aligned16(p)) return PHI_E_ALIGN;
  }

  phi_model* m = new (std::nothrow) phi_model;
  if (!m) return PHI_E_HIP;
  m->cfg = *cfg;
  m->layers.assign(w->layers, w->layers + cfg->n_layers);
  m->embed = w->embed;
  m->final_norm = w->final_norm;
  m->lm_head = w->lm_head;

  // RoPE tables: angle(p, i) = p * theta^(-2 i / head_dim), in double, stored fp32.
  const int half = cfg->head_dim / 2;
  const size_t n = (size_t)cfg->max_pos * half;
  std::vector<float> tab(2 * n);
  for (int p = 0; p < cfg->max_pos; ++p)
    for (int i = 0; i < half; ++i) {
      const double ang = (double)p * pow((double)cfg->rope_theta, -2.0 * i / cfg->head_dim);
      tab[(size_t)p * half + i] = (float)cos(ang);
      tab[n + (size_t)p * half + i] = (float)sin(ang);
    }
  hipStream_t st = as_stream(stream);
  if (hipMemcpyAsync(state, tab.data(), 2 * n * sizeof(float), hipMemcpyHostToDevice, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    delete m;
    return PHI_E_HIP;
  }
  m->rope_cos = reinterpret_cast<const float*>(state);
  m->rope_sin = m->rope_cos + n;
  *out = m;
  return PHI_OK;
}

size_t phi_workspace_bytes(const phi_model* m, int32_t batch, int32_t seq) {
  if (!m || batch < 1 || seq < 1) return 0;
  return plan_prefill(m->cfg, batch, seq).total;
}

phi_status phi_prefill_logits(const phi_model* m, const int32_t* ids, int32_t batch, int32_t seq, float* logits,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!m || !ids || !logits || !workspace) return PHI_E_NULL;
  if (batch < 1 || seq < 1) return PHI_E_SHAPE;
  if (seq > m->cfg.max_pos) return PHI_E_RANGE;
  if (!rows_fit(m->cfg, (long long)batch * seq)) return PHI_E_SHAPE;
  if (workspace_bytes < plan_prefill(m->cfg, batch, seq).total) return PHI_E_WORKSPACE;
  if (!aligned16(ids) || !aligned16(logits) || !aligned16(workspace)) return PHI_E_ALIGN;
  hipStream_t st = as_stream(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  const PhiProfile& pr = m->prof;
  if (pr.enabled && pr.used + launches_per_forward(m->cfg) > pr.stage.size()) return PHI_E_RANGE;
  if (m->cfg.wtype == PHI_WT_F32) return forward<float>(m, ids, batch, seq, logits, ws, st);
  return forward<f16>(m, ids, batch, seq, logits, ws, st);
}

phi_status phi_prefill_logits_host_ids(const phi_model* m, const int32_t* ids_host, int32_t batch, int32_t seq,
                                       float* logits, void* workspace, size_t workspace_bytes, void* stream) {
  if (!m || !ids_host || !logits || !workspace) return PHI_E_NULL;
  if (batch < 1 || seq < 1) return PHI_E_SHAPE;
  if (seq > m->cfg.max_pos) return PHI_E_RANGE;
  if (!rows_fit(m->cfg, (long long)batch * seq)) return PHI_E_SHAPE;
  const PrefillPlan p = plan_prefill(m->cfg, batch, seq);
  if (workspace_bytes < p.total) return PHI_E_WORKSPACE;
  if (!aligned16(logits) || !aligned16(workspace)) return PHI_E_ALIGN;
  const size_t T = (size_t)batch * seq;
  for (size_t t = 0; t < T; ++t)
    if (ids_host[t] < 0 || ids_host[t] >= m->cfg.vocab) return PHI_E_RANGE;
  const PhiProfile& pr = m->prof;
  if (pr.enabled && pr.used + launches_per_forward(m->cfg) > pr.stage.size()) return PHI_E_RANGE;
  int32_t* ids_dev = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(workspace) + p.off_ids);
  if (hipMemcpyAsync(ids_dev, ids_host, T * sizeof(int32_t), hipMemcpyHostToDevice, as_stream(stream)) != hipSuccess)
    return PHI_E_HIP;
  return phi_prefill_logits(m, ids_dev, batch, seq, logits, workspace, workspace_bytes, stream);
}

void phi_free(phi_model* m) {
  if (!m) return;
  for (hipEvent_t e : m->prof.ev) (void)hipEventDestroy(e);
  delete m;
}

phi_status phi_profile_enable(phi_model* m, int32_t enable) {
  if (!m) return PHI_E_NULL;
  PhiProfile& p = m->prof;
  if (enable && p.ev.empty()) {
    const size_t slots = 16 * launches_per_forward(m->cfg);
    p.ev.resize(2 * slots);
    p.stage.assign(slots, 0);
    for (hipEvent_t& e : p.ev)
      if (hipEventCreate(&e) != hipSuccess) return PHI_E_HIP;
  }
  p.enabled = enable != 0;
  return PHI_OK;
}

phi_status phi_profile_read(phi_model* m, double* ms_out, int64_t* launches_out) {
  if (!m || !ms_out || !launches_out) return PHI_E_NULL;
  PhiProfile& p = m->prof;
  for (int i = 0; i < PHI_PROF_N; ++i) {
    ms_out[i] = 0.0;
    launches_out[i] = 0;
  }
  if (p.used && hipEventSynchronize(p.ev[2 * p.used - 1]) != hipSuccess) return PHI_E_HIP;
  for (size_t i = 0; i < p.used; ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, p.ev[2 * i], p.ev[2 * i + 1]) != hipSuccess) return PHI_E_HIP;
    ms_out[p.stage[i]] += ms;
    launches_out[p.stage[i]] += 1;
  }
  p.used = 0;
  return PHI_OK;
}

phi_status phi_linear_f32out(int32_t wtype, const void* a, const void* w, const void* scale, float* y, int32_t M,
                             int32_t N, int32_t K, void* stream) {
  if (!a || !w || !y) return PHI_E_NULL;
  if (wtype != PHI_WT_F32 && wtype != PHI_WT_F16 && wtype != PHI_WT_I8) return PHI_E_DTYPE;
  if ((wtype == PHI_WT_I8) != (scale != nullptr)) return PHI_E_NULL;
  if (M < 1 || N < 4 || K < 64 || K % 64 || N % 4) return PHI_E_SHAPE;
  if (!elems_fit(M, K) || !elems_fit(N, K)) return PHI_E_SHAPE;
  if (!aligned16(a) || !aligned16(w) || !aligned16(y) || !aligned16(scale)) return PHI_E_ALIGN;
  GemmArgs g{};
  g.A = a;
  g.W = w;
  g.scale = scale;
  g.M = M;
  g.N = N;
  g.K = K;
  g.out = y;
  g.ldo = N;
  return gemm<EPI_F32>(wtype, g, plan_gemm(EPI_F32, M, N, K, wtype == PHI_WT_I8), as_stream(stream));
}

phi_status phi_gate_up_silu(int32_t wtype, const void* a, const void* w, const void* scale, void* act, int32_t M,
                            int32_t I, int32_t K, void* stream) {
  if (!a || !w || !act) return PHI_E_NULL;
  if (wtype != PHI_WT_F32 && wtype != PHI_WT_F16 && wtype != PHI_WT_I8) return PHI_E_DTYPE;
  if ((wtype == PHI_WT_I8) != (scale != nullptr)) return PHI_E_NULL;
  if (M < 1 || I < 128 || K < 64 || K % 64 || I % 128) return PHI_E_SHAPE;
  if (!elems_fit(M, K) || !elems_fit(2ll * I, K)) return PHI_E_SHAPE;
  if (!aligned16(a) || !aligned16(w) || !aligned16(act) || !aligned16(scale)) return PHI_E_ALIGN;
  GemmArgs g{};
  g.A = a;
  g.W = w;
  g.scale = scale;
  g.M = M;
  g.N = 2 * I;
  g.K = K;
  g.act = act;
  g.ld_act = I;
  return gemm<EPI_SILU>(wtype, g, plan_gemm(EPI_SILU, M, 2 * I, K, wtype == PHI_WT_I8), as_stream(stream));
}

size_t phi_attention_vt_stride(int32_t seq) { return seq < 1 ? 0 : round_up((size_t)seq, 64); }

phi_status phi_attention_prefill(int32_t act_f32, const void* q, const void* k, const void* vt, void* out,
                                 int32_t batch, int32_t seq, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                 void* stream) {
  if (!q || !k || !vt || !out) return PHI_E_NULL;
  if (batch < 1 || seq < 1 || n_heads < 1 || n_kv_heads < 1 || n_heads % n_kv_heads ||
      (head_dim != 96 && !((head_dim == 64 || head_dim == 128) && !act_f32)))
    return PHI_E_SHAPE;
  if (seq > kMaxPos) return PHI_E_RANGE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(out)) return PHI_E_ALIGN;
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.vt = vt;
  a.out = out;
  a.S = seq;
  a.s_pad = (int)round_up((size_t)seq, 64);
  a.nh = n_heads;
  a.nkv = n_kv_heads;
  return attention(act_f32 != 0, a, batch, head_dim, as_stream(stream));
}

size_t attn_decode_k16v8_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                         int32_t max_ctx) {
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim != 128 || max_ctx < 1) return 0;
  return plan_decode(batch, n_q_heads, n_kv_heads, max_ctx).total;
}

phi_status attn_decode_k16v8(const void* q, const void* k_pool, const void* v_pool, const float* v_scale,
                             const int32_t* block_table, const int32_t* ctx_lens, int32_t batch, int32_t n_q_heads,
                             int32_t n_kv_heads, int32_t head_dim, int32_t page_size, int32_t n_pages,
                             int32_t max_pages, int32_t max_ctx, float sm_scale, void* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!workspace) return PHI_E_NULL;
  DecodePlan p;
  const phi_status s = check_decode_args(q, k_pool, v_pool, v_scale, block_table, ctx_lens, out, batch, n_q_heads,
                                         n_kv_heads, head_dim, page_size, n_pages, max_pages, max_ctx, sm_scale, &p);
  if (s) return s;
  if (workspace_bytes < p.total) return PHI_E_WORKSPACE;
  if (!aligned16(workspace)) return PHI_E_ALIGN;
  return decode_attention(q, k_pool, v_pool, v_scale, block_table, ctx_lens, batch, n_q_heads, n_kv_heads,
                          n_pages, max_pages, max_ctx, sm_scale, out, workspace, p, as_stream(stream));
}

phi_status attn_decode_k16v8_noalloc(const void* q, const void* k_pool, const void* v_pool, const float* v_scale,
                                     const int32_t* block_table, const int32_t* ctx_lens, int32_t batch,
                                     int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                     int32_t n_pages, int32_t max_pages, int32_t max_ctx, float sm_scale, void* out,
                                     void* stream) {
  DecodePlan p;
  phi_status s = check_decode_args(q, k_pool, v_pool, v_scale, block_table, ctx_lens, out, batch, n_q_heads,
                                   n_kv_heads, head_dim, page_size, n_pages, max_pages, max_ctx, sm_scale, &p);
  if (s) return s;
  if (p.total > (size_t)PHI_DECODE_SCRATCH_BYTES) return PHI_E_WORKSPACE;
  // the stream must belong to the current device, whose scratch copy is used
  hipStream_t st = as_stream(stream);
  if (st) {
    int cur = -1, sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(st, &sdev) != hipSuccess) return PHI_E_HIP;
    if (cur != sdev) return PHI_E_RANGE;
  }
  void* ws = nullptr;
  if ((s = decode_scratch(&ws))) return s;
  return decode_attention(q, k_pool, v_pool, v_scale, block_table, ctx_lens, batch, n_q_heads, n_kv_heads,
                          n_pages, max_pages, max_ctx, sm_scale, out, ws, p, st);
}

phi_status kv_append_k16v8(const void* k_new, const void* v_new, const float* v_scale, const int32_t* block_table,
                           const int32_t* positions, int32_t batch, int32_t n_kv_heads, int32_t head_dim,
                           int32_t page_size, int32_t n_pages, int32_t max_pages, void* k_pool, void* v_pool,
                           void* stream) {
  if (batch == 0) return PHI_OK;
  if (!k_new || !v_new || !v_scale || !block_table || !positions || !k_pool || !v_pool) return PHI_E_NULL;
  if (batch < 0 || n_kv_heads < 1 || head_dim != 128 || page_size != 16 || n_pages < 1 || max_pages < 1)
    return PHI_E_SHAPE;
  if ((long long)n_pages * n_kv_heads * 16 * 128 * 2 > (1ll << 40) || (long long)batch * n_kv_heads > (1 << 26))
    return PHI_E_SHAPE;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool)) return PHI_E_ALIGN;
  return kv_append(k_new, v_new, v_scale, block_table, positions, batch, n_kv_heads, n_pages, max_pages, k_pool,
                   v_pool, as_stream(stream));
}


phi_status phi_prefill_fill_k16v8(const phi_model* m, const int32_t* ids, int32_t batch, int32_t seq,
                                  float* logits, const phi_kv_cache* cache, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!m || !ids || !logits || !workspace || !cache) return PHI_E_NULL;
  phi_status s = check_cache(m, cache);
  if (s) return s;
  if (batch < 1 || seq < 1) return PHI_E_SHAPE;
  if (seq > m->cfg.max_pos || seq > cache->max_pages * 16) return PHI_E_RANGE;
  if (!rows_fit(m->cfg, (long long)batch * seq)) return PHI_E_SHAPE;
  if (workspace_bytes < plan_prefill(m->cfg, batch, seq).total) return PHI_E_WORKSPACE;
  if (!aligned16(ids) || !aligned16(logits) || !aligned16(workspace)) return PHI_E_ALIGN;
  const PhiProfile& pr = m->prof;
  if (pr.enabled && pr.used + launches_per_forward(m->cfg) > pr.stage.size()) return PHI_E_RANGE;
  return forward<f16>(m, ids, batch, seq, logits, reinterpret_cast<char*>(workspace), as_stream(stream), cache);
}

size_t phi_decode_workspace_bytes(const phi_model* m, int32_t batch, int32_t max_ctx) {
  if (!m || batch < 1 || max_ctx < 1 || m->cfg.head_dim != 128) return 0;
  return plan_decode_step(m->cfg, batch, max_ctx).total;
}

phi_status phi_decode_step_k16v8(const phi_model* m, const int32_t* ids, const int32_t* positions, int32_t batch,
                                 int32_t max_ctx, const phi_kv_cache* cache, float* logits, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!m || !ids || !positions || !logits || !workspace || !cache) return PHI_E_NULL;
  phi_status s = check_cache(m, cache);
  if (s) return s;
  if (batch < 1 || batch > (1 << 16) || !rows_fit(m->cfg, batch)) return PHI_E_SHAPE;
  if (max_ctx < 1 || max_ctx > cache->max_pages * 16 || max_ctx > m->cfg.max_pos) return PHI_E_RANGE;
  if (workspace_bytes < plan_decode_step(m->cfg, batch, max_ctx).total) return PHI_E_WORKSPACE;
  if (!aligned16(ids) || !aligned16(positions) || !aligned16(logits) || !aligned16(workspace)) return PHI_E_ALIGN;
  return decode_step(m, ids, positions, batch, max_ctx, cache, logits, reinterpret_cast<char*>(workspace),
                     as_stream(stream));
}

int64_t phi_kv_pool_slots(int64_t budget_bytes, int32_t n_layers, int32_t n_kv_heads, int32_t head_dim,
                          int32_t k_bytes, int32_t v_bytes, int32_t page_size) {
  if (budget_bytes <= 0 || n_layers <= 0 || n_kv_heads <= 0 || head_dim <= 0 || k_bytes <= 0 || v_bytes <= 0 ||
      page_size <= 0)
    return -1;
  const int64_t per_token = (int64_t)n_kv_heads * head_dim * (k_bytes + v_bytes);
  const int64_t slots = budget_bytes / n_layers / per_token;
  return slots / page_size * page_size;
}

}  // extern "C"
