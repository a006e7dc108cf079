// Prefill GEMMs: y[M][N] = a[M][K] w[N][K]^T with fused epilogues.
//
// MFMA core (binary16 activations; binary16 or int8 weights):
//  - 4 or 8 compute waves of 64 lanes, each owning a WM x WN sub-tile built
//    from v_mfma_f32_16x16x32_f16 blocks with fp32 accumulators, plus
//    optional copy waves that only issue the global -> LDS copies.  The
//    16x16x32 form does the same flops per cycle as 32x32x16 but moves half
//    the accumulator bytes per flop; under sustained load the chip's clock is
//    set by its power limit, and with it the GEMMs ran at a higher shader
//    clock (1.52 -> 1.75 GHz at 512 tokens, 1.78 -> 2.0 GHz at 4096, read from
//    the shader-cycle and 100 MHz counters inside the kernel) and faster.
//  - K is walked in steps of 64 through a ring of NS LDS stages, NS - 1 of
//    them in flight while one is consumed, so the DMA of a k-step has NS - 1
//    k-steps of MFMA work to arrive.  binary16 operands go global -> LDS
//    directly (buffer_load_dwordx4 ... lds, no VGPR staging): one wave
//    instruction fills 1 KB = 8 rows of 128 B.  int8 weights are staged
//    through registers (16 codes per lane and load) and widened exactly to
//    binary16 (|q| <= 127) as they are written to LDS, once per element, so
//    both weight types share one LDS layout (the 256 x 256 tiles, short of
//    registers for that, keep codes in LDS and widen B fragments as they are
//    read); the per-row scale multiplies the fp32 accumulator (it factors out
//    of the K sum).
//  - Rows are stored with an XOR swizzle of their 16-byte chunks,
//    chunk' = chunk ^ ((row >> 1) & 7): 16 lanes reading 16 consecutive rows
//    at one logical chunk touch 16 distinct 16-byte bank groups of the
//    256-byte LDS bank row, so fragment reads are conflict free (int8 code
//    rows: chunk' = chunk ^ ((row >> 1) & 3) over their four chunks).
//  - A k-step is two k32 sub-steps.  The reads for sub-step s + 1 run behind
//    the MFMAs of sub-step s: the operand with more blocks per wave is
//    streamed (block o of the next sub-step is read into the registers of
//    block o right after its last MFMA), the other one is double-buffered,
//    and scheduling barriers keep the compiler from re-serialising them.  The
//    stage barrier of k-step kt + 1 sits between the two sub-steps of kt, so
//    the next stage's first reads also run under MFMAs.
//  - Split-K: a launch may cut K into `splits` ranges; each writes a binary16
//    partial tile (saturating, NaN kept) that the next kernel (the residual +
//    RMSNorm) sums into the fp32 residual in a fixed order, so results do not
//    depend on scheduling.
//  - Workgroups map to tiles so that consecutive tiles of one weight column
//    block run on the same XCD (workgroups go round-robin over the 8 XCDs),
//    sharing that XCD's L2 for the weight tile.
// Epilogues work on the accumulator registers (lane l of a 16x16 block holds
// column l % 16 and rows 4 (l / 16) + v, v < 4):
//  EPI_F32      logits: out[m][n] = acc
//  EPI_RESID    residual: x[m][n] += acc (fp32, staged through LDS)
//  EPI_PARTIAL  split-K: part[split][m][n] = acc, binary16 (staged through LDS
//               for full-line stores)
//  EPI_SILU     fused gate/up: the tile reads weight rows in 16-row blocks
//               alternating gate, up for the same outputs, so a lane holds
//               gate and up of one output: act = silu(gate) * up
//  EPI_QKV      fused Q/K/V, one head (64, 96 or 128 wide) per wave (or, on
//               the 128 x 144 tiles, one Q or K head of 96 plus half a V
//               head per tile), plus an optional per-row bias before RoPE.  With 16-wide blocks in
//               natural d order, RoPE partners (d, d + HD / 2) sit in blocks
//               j and j + HD / 32 of the same lane.  The RoPE position is the
//               row's index within its sequence, or a per-row position
//               (decode steps).  RoPE runs on the fp32 accumulator; the head
//               tile is staged through LDS and written with 16-byte stores:
//               Q, K to [B][heads][S][HD], V to V^T [B][kv_heads][HD][s_pad].
// fp32 core (float32 model): a SIMT kernel with an LDS-staged epilogue.
#pragma once
#include <type_traits>

#include "common.hpp"

namespace phi {

enum { EPI_F32 = 0, EPI_RESID = 1, EPI_SILU = 2, EPI_QKV = 3, EPI_PARTIAL = 4 };

struct GemmArgs {
  const void* A;      // [M][K] activations
  const void* W;      // [N][K] weights (f16, int8 or f32)
  const void* scale;  // binary16 [N] (int8 weights)
  int M, N, K;        // N = rows of W (2 I for the fused gate/up)
  int tiles_m, tiles_n, splits, kt_per_split;
  int group_m;        // M-tiles per tile group (1 <= group_m <= tiles_m)
  float* out;         // EPI_F32: [M][ldo]; EPI_PARTIAL: [splits][M][N]
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
  const int32_t* pos;     // EPI_QKV: RoPE position of each token row (nullptr: row mod S)
  const f16* bias;        // EPI_QKV: optional per-row bias of the fused product (nullptr: none)
  int max_pos;
  int S, s_pad, nh, nkv, hd;
};

// ---------------------------------------------------------------- row maps
// Weight row read by tile-local row r of N-tile tn (MFMA core).
template <int EPI, int BN>
__device__ __forceinline__ int w_row_mfma(const GemmArgs& a, int tn, int r) {
  if constexpr (EPI == EPI_SILU) {
    // 16-row blocks alternate gate / up; block pair p covers outputs tn*BN/2 + 16p ..
    const int blk = r >> 4, p = blk >> 1;
    const int out = tn * (BN / 2) + p * 16 + (r & 15);
    return (blk & 1) ? (a.N >> 1) + out : out;
  } else if constexpr (EPI == EPI_QKV && BN == 144) {
    // head-and-a-half tiles: Q or K head tn (96 rows), then V rows 48 (tn % 2) ..
    // of V head tn / 2 (tiles cover nh + nkv heads with nh = nkv)
    const int n = r < 96 ? tn * 96 + r : (a.nh + a.nkv) * 96 + tn * 48 + (r - 96);
    return n < a.N ? n : a.N - 1;
  } else {
    const int n = tn * BN + r;
    return n < a.N ? n : a.N - 1;
  }
}

// ---------------------------------------------------------------- MFMA core
__device__ __forceinline__ int swz(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 7)) << 3); }

// Eight int8 codes (two dwords) -> binary16, exactly: with the sign bit
// flipped a code q is the byte u = q + 128, and the binary16 with high byte
// 0x64 and low byte u is 1024 + u; subtracting 1152 leaves q.
__device__ __forceinline__ f16x8 i8x8_to_f16x8(uint32_t lo, uint32_t hi) {
  const uint32_t x0 = lo ^ 0x80808080u, x1 = hi ^ 0x80808080u;
  const uint32_t k = 0x64646464u;
  f16x8 o;
  const uint32_t w[4] = {__builtin_amdgcn_perm(k, x0, 0x04010400u), __builtin_amdgcn_perm(k, x0, 0x04030402u),
                         __builtin_amdgcn_perm(k, x1, 0x04010400u), __builtin_amdgcn_perm(k, x1, 0x04030402u)};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = __builtin_bit_cast(f16x2, w[i]) - f16x2{(f16)1152.f, (f16)1152.f};
    o[2 * i] = h[0];
    o[2 * i + 1] = h[1];
  }
  return o;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

template <int BM_, int BN_, int WGM_, int WGN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr int NT = WGM * WGN * 64, NW = WGM * WGN;
  static constexpr int WM = BM / WGM, WN = BN / WGN, TM = WM / 16, TN = WN / 16;  // 16x16 blocks per wave
};

// HW > 0 adds HW copy waves to the workgroup: they issue every global -> LDS
// copy of the tile and take part in the k-step barriers, while the C::NW
// compute waves only read fragments and run MFMAs.  A direct-to-LDS load
// holds its wave at issue until the copy path takes it (tens of cycles
// each), so copies issued by the compute waves leave their MFMA pipes idle.
template <class C, bool W8, int EPI, int NS, int HW = 0>
__global__ __launch_bounds__(C::NT + 64 * HW) void phi_gemm_mfma_kernel(GemmArgs a) {
  // int8 weights take the register-staged copy (their 64-byte rows measured
  // faster that way, and the registers are where they are widened);
  // binary16 operands go global -> LDS by DMA
  constexpr bool VG = W8;
  static_assert(!W8 || VG, "int8 codes are widened on their way into LDS (register staging only)");
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN, TM = C::TM, TN = C::TN;
  constexpr int NT = C::NT, NW = C::NW, BK = 64;
  static_assert(NS >= 2 && NS <= 4, "stages");
  // An LDS stage holds A [BM][64] then W [BN][64], binary16 with 128-byte
  // rows of eight 16-byte chunks (or int8 codes in 64-byte rows, see WIDEN).
  // A copy instruction moves 1 KB from HBM: 8 binary16 rows, or 16 rows of
  // int8 codes (64 bytes each).
  constexpr int WB = W8 ? 1 : 2;                     // bytes per weight element in HBM
  // WIDEN: int8 codes are widened to binary16 once, as their registers are
  // written to LDS, and share the binary16 LDS layout.  The 256 x 256 tiles
  // keep them as codes in LDS (64-byte rows, chunk' = chunk ^ ((row >> 1) & 3))
  // and widen them as fragments are read: widening on the way in spills
  // there (128 bytes per lane; gate/up at 4 x 1024 13.9 -> 19.3 ms per
  // forward), while on the 256 x 192 tiles it took QKV 9.36 -> 8.38, o_proj
  // 3.75 -> 3.48 and down 8.26 -> 7.42 ms (each B fragment was widened by
  // every wave of its column before).
  constexpr bool WIDEN = W8 && !(BM == 256 && BN == 256);
  constexpr int WLB = W8 && !WIDEN ? 1 : 2;          // bytes per weight element in LDS
  constexpr int STAGE = (BM * BK * 2 + BN * BK * WLB) / 2;  // f16 elements per LDS stage
  constexpr int INS_A = BM * 8 / 64;                 // 1 KB DMA instructions for A per stage
  constexpr int INS_W = BN * BK * WB / 1024;
  static_assert(HW == 0 || !VG, "copy waves only on the DMA path");
  constexpr int NDW = HW > 0 ? HW : NW;               // waves that issue the copies
  // copies per copying wave and stage; where they do not divide evenly (int8
  // weights on 8 waves: 44 per stage) the surplus ones repeat the last copy,
  // writing the same bytes to the same LDS slot
  constexpr int LPW = (INS_A + INS_W + NDW - 1) / NDW;
  constexpr bool PAD = LPW * NDW != INS_A + INS_W;
  constexpr int JMAX = INS_A + INS_W - 1;             // last copy of a stage
  static_assert(LPW * NDW == INS_A + INS_W || VG, "stage split (binary16 DMA tiles divide evenly)");
  static_assert(TM * 16 == WM && TN * 16 == WN, "wave tile");
  // QH: 144-wide QKV tiles of one Q or K head plus half a V head (head_dim 96,
  // as many query as KV heads), the whole tile width in every wave
  constexpr bool QH = EPI == EPI_QKV && BN == 144;
  static_assert(!QH || WN == 144, "QKV head-and-a-half tile: one wave column");
  static_assert(EPI != EPI_QKV || QH || WN == 64 || WN == 96 || WN == 128, "QKV: one head (64, 96 or 128 wide) per wave");
  constexpr int HD = EPI == EPI_QKV ? (QH ? 96 : WN) : 96;
  static_assert(EPI != EPI_SILU || TN % 2 == 0, "SILU: gate/up block pairs");

  // the QKV epilogue stages each wave's head tile in the same LDS
  constexpr int QKV_REG = EPI == EPI_QKV ? ((WM * (HD + 8) > HD * (WM + 8)) ? WM * (HD + 8) : HD * (WM + 8)) : 0;
  constexpr int SMEM = NS * STAGE > NW * QKV_REG ? NS * STAGE : NW * QKV_REG;
  __shared__ __attribute__((aligned(1024))) f16 smem[SMEM];

  const int n_units = a.tiles_m * a.tiles_n * a.splits;
  const int unit = xcd_swizzle(blockIdx.x, gridDim.x);
  if (unit >= n_units) return;
  // units walk group_m M-tiles fastest, then the N-tiles, then the next group
  // of M-tiles: the workgroups running together on one XCD cover a block of
  // group_m x (32 / group_m) tiles and share its A and W tiles in L2
  const int per_split = a.tiles_m * a.tiles_n;
  const int split = unit / per_split;
  const int u = unit - split * per_split;
  const int tgroup = u / (a.group_m * a.tiles_n);
  const int rem = u - tgroup * a.group_m * a.tiles_n;
  const int gm = min(a.group_m, a.tiles_m - tgroup * a.group_m);
  const int tm = tgroup * a.group_m + rem % gm;
  const int tn = rem / gm;
  const int m0 = tm * BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool copies = HW == 0 || wave >= NW;            // this wave issues copies
  const int dw = HW > 0 ? (copies ? wave - NW : 0) : wave;  // its index among the copying waves
  const int wm = min(wave, NW - 1) / C::WGN, wn = min(wave, NW - 1) % C::WGN;
  const int K = a.K;
  const f16* A = reinterpret_cast<const f16*>(a.A);

  // DMA sources (element offsets in the operand's own type; the host keeps
  // rows x K within int32): instruction j = wave + NW * t fills LDS bytes
  // [1024 j, 1024 j + 1024) of the stage; the lane's 16-byte slot holds a
  // swizzled chunk of one row
  // A stage's first INS_A instructions are A rows, the rest W rows; with
  // INS_A a multiple of NW, instruction t of every wave is of one kind.
  static_assert(INS_A % NDW == 0, "A / W split of the DMA instructions");
  constexpr int TA_ = INS_A / NDW;  // instructions t < TA_ load A
  int src_off[LPW > 0 ? LPW : 1];
#pragma unroll
  for (int t = 0; t < LPW; ++t) {
    const int j = PAD ? min(dw + NDW * t, JMAX) : dw + NDW * t;
    const int s = j * 64 + lane;
    const bool is_w = t >= TA_;
    if (!is_w) {
      const int r = s >> 3, c = (s & 7) ^ ((r >> 1) & 7);
      src_off[t] = (m0 + r < a.M ? m0 + r : a.M - 1) * K + c * 8;
    } else if constexpr (WIDEN) {
      // 16 codes (k = 16 c4 .. + 15) of row r; swizzled when written to LDS
      const int sw = s - INS_A * 64, r = sw >> 2, c4 = sw & 3;
      src_off[t] = w_row_mfma<EPI, BN>(a, tn, r) * K + c4 * 16;
    } else if constexpr (W8) {
      // the slot's swizzled 16-code chunk of row r (codes stay codes in LDS)
      const int sw = s - INS_A * 64, r = sw >> 2, c = (sw & 3) ^ ((r >> 1) & 3);
      src_off[t] = w_row_mfma<EPI, BN>(a, tn, r) * K + c * 16;
    } else {
      const int sw = s - INS_A * 64, r = sw >> 3, c = (sw & 7) ^ ((r >> 1) & 7);
      src_off[t] = w_row_mfma<EPI, BN>(a, tn, r) * K + c * 8;
    }
  }
  // Buffer loads into LDS (MUBUF) rather than global ones (FLAT): the
  // compiler counts a FLAT load into LDS as an LDS access in flight too, and
  // then makes the first use of every later fragment read wait for
  // lgkmcnt(0).  Byte offsets fit the 32-bit voffset: the host keeps each
  // operand under 2^31 elements of at most 2 bytes.
  const f16* Wf = reinterpret_cast<const f16*>(a.W);
  const int8_t* W8p = reinterpret_cast<const int8_t*>(a.W);
  constexpr int WBY = W8 ? 1 : 2;
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.A), 0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.W), 0, -1, 0x00020000);

  auto issue = [&](int kt, f16* st) {
    const int k0 = kt * BK;
#pragma unroll
    for (int t = 0; t < LPW; ++t) {
      const int j = PAD ? min(dw + NDW * t, JMAX) : dw + NDW * t;
      lds_ptr_t dst = (lds_ptr_t)(reinterpret_cast<char*>(st) + j * 1024);
      // weights are streamed once per tile row: non-temporal, so that they do
      // not push the activation tiles (re-read by every N-tile) out of L2
      const unsigned off = (unsigned)(src_off[t] + k0) * (t < TA_ ? 2u : (unsigned)WBY);
      if (t < TA_) __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, dst, 16, off, 0, 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, dst, 16, off, 0, 0, kCacheNT);
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{};
  // QH: the compute waves load the RoPE factors of their rows (position of
  // row 4 (l / 16) + v of each 16-row block, dims l % 16 + 16 q of the 48
  // pairs) before the main loop, so that the last wave to finish it does not
  // wait for them after the final barrier (QKV 1.212 -> 1.198 ms per forward
  // at 1 x 512); the other QKV tiles have no registers to spare for them
  float qh_cs[QH ? TM : 1][4][3], qh_sn[QH ? TM : 1][4][3];
  if constexpr (QH) {
    if (HW == 0 || !copies) {
      const int grp0 = lane >> 4, col0 = lane & 15;
      const int mw0 = m0 + wm * WM;
      const int s_base = mw0 - (mw0 / a.S) * a.S;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = i * 16 + 4 * grp0 + v;
          int sp;
          if (a.pos) {
            sp = a.pos[min(mw0 + r, a.M - 1)];
            sp = sp < 0 ? 0 : (sp >= a.max_pos ? a.max_pos - 1 : sp);
          } else {
            sp = s_base + r;
            while (sp >= a.S) sp -= a.S;
          }
          const size_t t = (size_t)sp * 48;
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            qh_cs[i][v][q] = a.rope_cos[t + q * 16 + col0];
            qh_sn[i][v][q] = a.rope_sin[t + q * 16 + col0];
          }
        }
    }
  }

  // Fragments of k32 sub-step kk (k = 32 kk .. 32 kk + 31 of the stage): A
  // block i is 16 rows x 32 k, B block j 16 columns x 32 k; lane l holds row
  // (column) l % 16 and k = 32 kk + 8 (l / 16) .. + 8.
  auto ldA = [&](const f16* cur, int kk, int i) __attribute__((always_inline)) -> f16x8 {
    const int r = wm * WM + i * 16 + (lane & 15);
    return *reinterpret_cast<const f16x8*>(cur + swz(r, kk * 4 + (lane >> 4)));
  };
  auto ldB = [&](const f16* cur, int kk, int j) __attribute__((always_inline)) -> f16x8 {
    const int r = wn * WN + j * 16 + (lane & 15);
    if constexpr (W8 && !WIDEN) {
      // the lane's 8 codes: 16-code chunk 2 kk + g / 2, half g % 2 (g = l / 16)
      const uint8_t* curw = reinterpret_cast<const uint8_t*>(cur + BM * BK);
      const int g = lane >> 4;
      const uint2 q = *reinterpret_cast<const uint2*>(curw + r * 64 + 16 * ((kk * 2 + (g >> 1)) ^ ((r >> 1) & 3)) +
                                                      8 * (g & 1));
      return i8x8_to_f16x8(q.x, q.y);
    } else {
      return *reinterpret_cast<const f16x8*>(cur + BM * BK + swz(r, kk * 4 + (lane >> 4)));
    }
  };
  // The operand with more blocks per wave is streamed in place (so[o]), the
  // other one double-buffered (di[b][n]).  ROWS: A streams (TM >= TN).
  constexpr bool ROWS = TM >= TN;
  constexpr int NO = ROWS ? TM : TN, NI = ROWS ? TN : TM;
  f16x8 so[NO], di[2][NI];
  auto ld_o = [&](const f16* cur, int kk, int o) __attribute__((always_inline)) { return ROWS ? ldA(cur, kk, o) : ldB(cur, kk, o); };
  auto ld_i = [&](const f16* cur, int kk, int n) __attribute__((always_inline)) { return ROWS ? ldB(cur, kk, n) : ldA(cur, kk, n); };
  // One k32 sub-step: the MFMAs on so[] and di[b], outer block by outer
  // block; with reads, the fragments of sub-step kkr of stage rd follow each
  // outer block's MFMAs (its own streamed block, and the inner blocks spread
  // evenly over the outer ones, into di[b ^ 1]).  MFMAs go first: a read ahead of them would make
  // the first MFMA wait for it too (lgkmcnt(0)), a full LDS latency.
  auto sub = [&](const f16* rd, int kkr, int b, auto reads) __attribute__((always_inline)) {
#pragma unroll
    for (int o = 0; o < NO; ++o) {
#pragma unroll
      for (int n = 0; n < NI; ++n) {
        if constexpr (ROWS) acc[o][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(so[o], di[b][n], acc[o][n], 0, 0, 0);
        else acc[n][o] = __builtin_amdgcn_mfma_f32_16x16x32_f16(di[b][n], so[o], acc[n][o], 0, 0, 0);
      }
      if constexpr (decltype(reads)::value) {
#pragma unroll
        for (int n = o * NI / NO; n < (o + 1) * NI / NO; ++n) di[b ^ 1][n] = ld_i(rd, kkr, n);
        so[o] = ld_o(rd, kkr, o);
      }
    }
#pragma unroll
    for (int o = 0; o < NO; ++o) {
      __builtin_amdgcn_sched_group_barrier(0x008, NI, 0);
      if constexpr (decltype(reads)::value) {
        const int nr = 1 + (o + 1) * NI / NO - o * NI / NO;  // reads after this outer block
        if (nr == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        else if (nr == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else if (nr == 3) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        else __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // sub-step 0 of a stage into so[] and di[0]
  auto ld_first = [&](const f16* cur) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < NI; ++n) di[0][n] = ld_i(cur, 0, n);  // (row 0 needs all of these first)
#pragma unroll
    for (int o = 0; o < NO; ++o) so[o] = ld_o(cur, 0, o);
  };
  // One k-step on stage `cur` (register-staged path)
  auto kstep = [&](const f16* cur) __attribute__((always_inline)) {
    ld_first(cur);
    sub(cur, 1, 0, std::true_type{});
    sub(cur, 0, 1, std::false_type{});
  };

  const int kt0 = split * a.kt_per_split;
  const int kt1 = min(K / BK, kt0 + a.kt_per_split);
  if constexpr (VG) {
    // Register-staged copies, two stages of registers over two LDS stages:
    // k-step kt computes on LDS stage kt % 2 while the loads of kt + 2 are in
    // flight into one register set and the other set (k-step kt + 1, loaded
    // a step earlier) is written to LDS stage (kt + 1) % 2 at its end.
    static_assert(NS == 2, "register staging: two LDS stages");
    i32x4 r0[LPW], r1[LPW];
    auto gload = [&](int kt, i32x4* r) {
      const int k0 = kt * BK;
#pragma unroll
      for (int t = 0; t < LPW; ++t) {
        if (t < TA_) r[t] = *reinterpret_cast<const i32x4*>(A + src_off[t] + k0);
        else if constexpr (W8) r[t] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(W8p + src_off[t] + k0));
        else r[t] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(Wf + src_off[t] + k0));
      }
    };
    auto lput = [&](f16* st, const i32x4* r) {
#pragma unroll
      for (int t = 0; t < LPW; ++t) {
        const int j = PAD ? min(wave + NW * t, JMAX) : wave + NW * t;
        if (!WIDEN || t < TA_) {
          *reinterpret_cast<i32x4*>(reinterpret_cast<char*>(st) + j * 1024 + 16 * lane) = r[t];
        } else {
          // 16 int8 codes of row rw -> binary16 chunks 2 c4 and 2 c4 + 1 of
          // its 128-byte LDS row (the binary16 layout and swizzle)
          const int sw = (j - INS_A) * 64 + lane, rw = sw >> 2, c4 = sw & 3;
          const f16x8 h0 = i8x8_to_f16x8((uint32_t)r[t][0], (uint32_t)r[t][1]);
          const f16x8 h1 = i8x8_to_f16x8((uint32_t)r[t][2], (uint32_t)r[t][3]);
          f16* wrow = st + BM * BK;
          *reinterpret_cast<f16x8*>(wrow + swz(rw, 2 * c4)) = h0;
          *reinterpret_cast<f16x8*>(wrow + swz(rw, 2 * c4 + 1)) = h1;
        }
      }
    };
    if (kt0 < kt1) {
      gload(kt0, r0);
      if (kt0 + 1 < kt1) gload(kt0 + 1, r1);
      lput(smem, r0);
    }
    lds_barrier();
    for (int kt = kt0; kt < kt1; kt += 2) {
      // even step: LDS stage 0 holds kt, r1 holds kt + 1
      if (kt + 2 < kt1) gload(kt + 2, r0);
      // (always true: the block boundary keeps the register copies out of
      // the MFMA region; without it the int8 tiles run out of registers)
      __builtin_amdgcn_sched_barrier(0);
      if (wave < NW) kstep(smem);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < kt1) lput(smem + STAGE, r1);
      lds_barrier();
      if (kt + 1 >= kt1) break;
      // odd step: LDS stage 1 holds kt + 1, r0 holds kt + 2
      if (kt + 3 < kt1) gload(kt + 3, r1);
      __builtin_amdgcn_sched_barrier(0);
      if (wave < NW) kstep(smem + STAGE);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 2 < kt1) lput(smem, r0);
      lds_barrier();
    }
  } else {
    // The stage barrier of k-step kt + 1 sits between the two sub-steps of
    // k-step kt: every fragment of stage kt is in registers by then, so the
    // next stage's first fragment reads run under kt's second sub-step
    // instead of in front of the next k-step's first MFMAs.  Barrier B(j)
    // (stage j has landed, every read of stage j - 1 is done) lets the
    // copying waves refill the stage of k-step j - 1 with k-step j + NS - 1.
    auto wait_stage = [&](int j) {  // this wave's DMA of stage j; newer stages stay in flight
      const int newer = min(NS - 2, kt1 - 1 - j);
      if (newer <= 0) PHI_WAIT_VMCNT(0);
      else if (newer == 1) PHI_WAIT_VMCNT(LPW);
      else PHI_WAIT_VMCNT(2 * LPW);
    };
    auto stage_of = [&](int j) { return smem + ((j - kt0) % NS) * STAGE; };
    if (kt0 < kt1) {
      if (copies) {
#pragma unroll
        for (int i = 0; i < NS - 1; ++i)
          if (kt0 + i < kt1) issue(kt0 + i, smem + i * STAGE);
        wait_stage(kt0);
      }
      lds_barrier();  // B(kt0)
      if (copies && kt0 + NS - 1 < kt1) issue(kt0 + NS - 1, stage_of(kt0 + NS - 1));
      if (HW > 0 && copies) {
        for (int j = kt0 + 1; j < kt1; ++j) {
          wait_stage(j);
          lds_barrier();  // B(j)
          if (j + NS - 1 < kt1) issue(j + NS - 1, stage_of(j + NS - 1));
        }
      } else {
        ld_first(smem);
        for (int kt = kt0; kt < kt1; ++kt) {
          const f16* cur = stage_of(kt);
          sub(cur, 1, 0, std::true_type{});
          const bool more = kt + 1 < kt1;
          if (more) {
            if (copies) wait_stage(kt + 1);
            lds_barrier();  // B(kt + 1): this wave's reads of stage kt are done
            if (copies && kt + NS < kt1) issue(kt + NS, stage_of(kt + NS));
          }
          // (the last k-step re-reads its own stage into the unused buffers: no
          // branch around the MFMAs, which keeps the accumulators in place)
          sub(more ? stage_of(kt + 1) : cur, 0, 1, std::true_type{});
        }
      }
    }
  }

  // ---------------------------------------------------------------- epilogue
  if (HW > 0 && wave >= NW) {
    if constexpr (EPI != EPI_SILU) __syncthreads();  // the one barrier of the epilogue (all but SiLU)
    return;
  }
  const int grp = lane >> 4, col_l = lane & 15;
  auto row_of = [&](int i, int v) { return m0 + wm * WM + i * 16 + 4 * grp + v; };
  float sc[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    sc[j] = 1.0f;
    if constexpr (W8) sc[j] = (float)reinterpret_cast<const f16*>(a.scale)[w_row_mfma<EPI, BN>(a, tn, wn * WN + j * 16 + col_l)];
  }

  if constexpr (EPI == EPI_PARTIAL || EPI == EPI_F32 || EPI == EPI_RESID) {
    // The tile goes through the wave's own LDS rows, 16 rows at a time, and
    // leaves as 4-column vectors, so 16 lanes cover one row segment of 64
    // columns in full cache lines: binary16 split-K partials (8-byte
    // stores), fp32 logits or the fp32 residual update (16-byte stores).
    // Against per-lane 4-byte stores (4 rows of 64 bytes per instruction),
    // measured at 4096 tokens: o_proj 2.98 -> 2.61, down 6.30 -> 5.97,
    // lm_head 0.74 -> 0.70 ms per forward.
    constexpr int SLD = WN + 4;  // staging row stride (floats)
    static_assert(NW * 16 * SLD * 4 <= SMEM * 2, "epilogue staging fits");
    constexpr int CPR = WN / 4;         // 4-column chunks per row
    constexpr int NQ = 16 * CPR / 64;   // chunks per lane per 16-row block
    static_assert(16 * CPR % 64 == 0, "whole chunks per lane");
    const int n0 = tn * BN + wn * WN;
    // The residual rows of the wave's tile are loaded before the staging
    // barrier, all in flight at once.  Loaded next to its store, each
    // load-add-store waited for its own load (the compiler cannot prove a
    // store and the next load apart): one memory latency per 4 columns.
    f32x4 xres[EPI == EPI_RESID ? TM : 1][EPI == EPI_RESID ? NQ : 1];
    if constexpr (EPI == EPI_RESID) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int idx = lane + 64 * q, r = idx / CPR, c = idx - r * CPR;
          const int m = m0 + wm * WM + i * 16 + r, n = n0 + 4 * c;
          // (clamped into the tile's valid rows and columns instead of a
          // branch per load; the store below keeps the bounds check)
          xres[i][q] = vec4<float>::load(a.x + (size_t)min(m, a.M - 1) * a.ldx + min(n, a.N - 4));
        }
      lds_barrier();  // every wave is done with the k-stages (LDS only: the loads stay in flight)
    } else {
      __syncthreads();  // every wave is done with the k-stages
    }
    float* stg = reinterpret_cast<float*>(smem) + wave * 16 * SLD;
    f16* po = reinterpret_cast<f16*>(a.out);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) stg[(4 * grp + v) * SLD + j * 16 + col_l] = acc[i][j][v] * sc[j];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int idx = lane + 64 * q;
        const int r = idx / CPR, c = idx - r * CPR;
        const int m = m0 + wm * WM + i * 16 + r, n = n0 + 4 * c;
        f32x4 y = *reinterpret_cast<const f32x4*>(stg + r * SLD + 4 * c);
        // saturate instead of overflowing to inf (a partial of a finite sum
        // beyond the binary16 range is not expected on real activations); a
        // NaN stays NaN, so bad rows still come out NaN
        if constexpr (EPI == EPI_PARTIAL) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = y[e] > 65504.f ? 65504.f : (y[e] < -65504.f ? -65504.f : y[e]);
        }
        if (m < a.M && n < a.N) {
          if constexpr (EPI == EPI_PARTIAL) vec4<f16>::store(po + ((size_t)split * a.M + m) * a.N + n, y);
          else if constexpr (EPI == EPI_F32) vec4<float>::store(a.out + (size_t)m * a.ldo + n, y);
          else vec4<float>::store(a.x + (size_t)m * a.ldx + n, xres[EPI == EPI_RESID ? i : 0][EPI == EPI_RESID ? q : 0] + y);
        }
      }
    }
  } else if constexpr (EPI == EPI_SILU) {
    f16* act = reinterpret_cast<f16*>(a.act);
#pragma unroll
    for (int p = 0; p < TN / 2; ++p) {
      const int n = tn * (BN / 2) + wn * (WN / 2) + p * 16 + col_l;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = row_of(i, v);
          if (m >= a.M) continue;
          act[(size_t)m * a.ld_act + n] = (f16)silu_mul(acc[i][2 * p][v] * sc[2 * p], acc[i][2 * p + 1][v] * sc[2 * p + 1]);
        }
    }
  } else if constexpr (QH) {
    // Q or K head tn with RoPE (blocks 0..5, partners j and j + 3), then V^T
    // dims 48 (tn % 2) .. + 48 of V head tn / 2 (blocks 6..8); each part goes
    // through the wave's LDS region and leaves as 16-byte stores
    constexpr int HALF = 48, NP = 3;
    constexpr int QLD = HD + 8, VLD = WM + 8;
    constexpr int REG = QKV_REG;
    static_assert(WM * QLD <= REG && HALF * VLD <= REG && NW * REG <= SMEM, "QKV staging");
    const bool is_q = tn < a.nh;
    const int head = is_q ? tn : tn - a.nh, nheads = is_q ? a.nh : a.nkv;
    const int vh = tn >> 1, vd0 = (tn & 1) * HALF;
    const int mw0 = m0 + wm * WM;
    static_assert(HALF == 48 && NP == 3, "RoPE factors loaded before the main loop");
    float bj[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) bj[j] = a.bias ? (float)a.bias[w_row_mfma<EPI, BN>(a, tn, j * 16 + col_l)] : 0.f;
    __syncthreads();                      // every wave is done with the k-stages
    f16* tile = smem + wave * REG;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = i * 16 + 4 * grp + v;
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          const float y0 = acc[i][q][v] * sc[q] + bj[q], y1 = acc[i][q + NP][v] * sc[q + NP] + bj[q + NP];
          const int d = q * 16 + col_l;
          tile[r * QLD + d] = (f16)(y0 * qh_cs[i][v][q] - y1 * qh_sn[i][v][q]);
          tile[r * QLD + d + HALF] = (f16)(y1 * qh_cs[i][v][q] + y0 * qh_sn[i][v][q]);
        }
      }
    // the wave reads back only what it wrote: its own LDS operations are ordered
    {
      f16* dst = reinterpret_cast<f16*>(is_q ? a.q : a.k);
      constexpr int CR = HD / 8;
      for (int idx = lane; idx < WM * CR; idx += 64) {
        const int r = idx / CR, c = idx - r * CR;
        const int m = mw0 + r;
        if (m >= a.M) continue;
        const int b = m / a.S, s = m - b * a.S;
        *reinterpret_cast<f16x8*>(dst + ((size_t)(b * nheads + head) * a.S + s) * HD + c * 8) =
            *reinterpret_cast<const f16x8*>(tile + r * QLD + c * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = i * 16 + 4 * grp + v;
#pragma unroll
        for (int j = 2 * NP; j < TN; ++j) tile[((j - 2 * NP) * 16 + col_l) * VLD + r] = (f16)(acc[i][j][v] * sc[j] + bj[j]);
      }
    {
      f16* vt = reinterpret_cast<f16*>(a.vt);
      constexpr int CPR = WM / 8;  // 8-token chunks per V^T row segment
      const bool aligned = (a.S & 7) == 0 && (a.s_pad & 7) == 0;
      for (int idx = lane; idx < HALF * CPR; idx += 64) {
        const int dl = idx / CPR, c = idx - dl * CPR;
        const int d = vd0 + dl;
        const int m = mw0 + c * 8;
        if (m >= a.M) continue;
        if (aligned) {
          const int b = m / a.S, s = m - b * a.S;
          *reinterpret_cast<f16x8*>(vt + ((size_t)(b * a.nkv + vh) * HD + d) * a.s_pad + s) =
              *reinterpret_cast<const f16x8*>(tile + dl * VLD + c * 8);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (m + e >= a.M) break;
            const int b = (m + e) / a.S, s = m + e - b * a.S;
            vt[((size_t)(b * a.nkv + vh) * HD + d) * a.s_pad + s] = tile[dl * VLD + c * 8 + e];
          }
        }
      }
    }
  } else {  // EPI_QKV
    // RoPE on the accumulators, then the wave's WM x HD head tile goes through
    // LDS in natural d order and leaves as 16-byte stores: rows of Q / K, and
    // rows of V^T (8-token chunks of one d row).
    constexpr int HALF = HD / 2;
    constexpr int QLD = HD + 8;           // Q/K staging row stride (conflict-free writes)
    constexpr int VLD = WM + 8;           // V^T staging row stride
    constexpr int REG = QKV_REG;
    static_assert(REG == ((WM * QLD > HD * VLD) ? WM * QLD : HD * VLD) && NW * REG <= SMEM, "QKV staging");
    const int col0 = tn * BN + wn * HD;   // first fused row of this wave's head
    const int q_end = a.nh * HD, k_end = (a.nh + a.nkv) * HD;
    const bool is_v = col0 >= k_end;
    const int head = col0 < q_end ? col0 / HD : (col0 < k_end ? (col0 - q_end) / HD : (col0 - k_end) / HD);
    const int nheads = col0 < q_end ? a.nh : a.nkv;
    // block j < NP holds d = 16 j + l % 16 (frequency index f = d), block
    // j + NP its RoPE partner d + HD / 2
    constexpr int NP = HD / 32;
    const int mw0 = m0 + wm * WM;      // first token row of this wave
    // rotation factors of the lane's rows: all loads in flight at once, before
    // the barrier.  Position = pos[row] when given, else row mod S.
    float cs[TM][4][NP], sn[TM][4][NP];
    if (!is_v && col0 < a.N) {
      const int s_base = mw0 - (mw0 / a.S) * a.S;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = i * 16 + 4 * grp + v;
          int sp;
          if (a.pos) {
            sp = a.pos[min(mw0 + r, a.M - 1)];
            sp = sp < 0 ? 0 : (sp >= a.max_pos ? a.max_pos - 1 : sp);
          } else {
            sp = s_base + r;
            while (sp >= a.S) sp -= a.S;
          }
          const size_t t = (size_t)sp * HALF;
#pragma unroll
          for (int q = 0; q < NP; ++q) {
            cs[i][v][q] = a.rope_cos[t + q * 16 + col_l];
            sn[i][v][q] = a.rope_sin[t + q * 16 + col_l];
          }
        }
    }
    // per-row bias of the fused product (one value per lane and block)
    float bj[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bj[j] = (a.bias && col0 < a.N) ? (float)a.bias[w_row_mfma<EPI, BN>(a, tn, wn * WN + j * 16 + col_l)] : 0.f;
    __syncthreads();                      // every wave is done with the k-stages
    if (col0 >= a.N) return;
    f16* tile = smem + wave * REG;
    if (is_v) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = i * 16 + 4 * grp + v;
#pragma unroll
          for (int j = 0; j < TN; ++j) tile[(j * 16 + col_l) * VLD + r] = (f16)(acc[i][j][v] * sc[j] + bj[j]);
        }
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = i * 16 + 4 * grp + v;
#pragma unroll
          for (int q = 0; q < NP; ++q) {
            const float y0 = acc[i][q][v] * sc[q] + bj[q], y1 = acc[i][q + NP][v] * sc[q + NP] + bj[q + NP];
            const int d = q * 16 + col_l;
            tile[r * QLD + d] = (f16)(y0 * cs[i][v][q] - y1 * sn[i][v][q]);
            tile[r * QLD + d + HALF] = (f16)(y1 * cs[i][v][q] + y0 * sn[i][v][q]);
          }
        }
    }
    // the wave reads back only what it wrote: its own LDS operations are ordered
    if (!is_v) {
      f16* dst = reinterpret_cast<f16*>(col0 < q_end ? a.q : a.k);
      constexpr int CR = HD / 8;  // 16-byte chunks per row
      for (int idx = lane; idx < WM * CR; idx += 64) {
        const int r = idx / CR, c = idx - r * CR;
        const int m = mw0 + r;
        if (m >= a.M) continue;
        const int b = m / a.S, s = m - b * a.S;
        *reinterpret_cast<f16x8*>(dst + ((size_t)(b * nheads + head) * a.S + s) * HD + c * 8) =
            *reinterpret_cast<const f16x8*>(tile + r * QLD + c * 8);
      }
    } else {
      f16* vt = reinterpret_cast<f16*>(a.vt);
      constexpr int CPR = WM / 8;  // 8-token chunks per V^T row segment
      const bool aligned = (a.S & 7) == 0 && (a.s_pad & 7) == 0;  // chunks never straddle sequences
      for (int idx = lane; idx < HD * CPR; idx += 64) {
        const int d = idx / CPR, c = idx - d * CPR;
        const int m = mw0 + c * 8;
        if (m >= a.M) continue;
        if (aligned) {
          const int b = m / a.S, s = m - b * a.S;
          *reinterpret_cast<f16x8*>(vt + ((size_t)(b * a.nkv + head) * HD + d) * a.s_pad + s) =
              *reinterpret_cast<const f16x8*>(tile + d * VLD + c * 8);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (m + e >= a.M) break;
            const int b = (m + e) / a.S, s = m + e - b * a.S;
            vt[((size_t)(b * a.nkv + head) * HD + d) * a.s_pad + s] = tile[d * VLD + c * 8 + e];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- fp32 core
template <int BN>
__device__ __forceinline__ int w_row_simt(const GemmArgs& a, int tn, int r, int epi) {
  if (epi == EPI_SILU) {
    constexpr int H2 = BN / 2;
    const int I = a.N >> 1;
    return r < H2 ? tn * H2 + r : I + tn * H2 + (r - H2);
  }
  const int n = tn * BN + r;
  return n < a.N ? n : a.N - 1;
}

template <class AT>
__device__ __forceinline__ void store8(AT* p, const float* v);
template <>
__device__ __forceinline__ void store8<float>(float* p, const float* v) {
  reinterpret_cast<f32x4*>(p)[0] = f32x4{v[0], v[1], v[2], v[3]};
  reinterpret_cast<f32x4*>(p)[1] = f32x4{v[4], v[5], v[6], v[7]};
}

// Epilogue over an fp32 tile sC[BM][ldc] (origin row m0, N-tile tn), float32 model.
template <int EPI, int BM, int BN>
__device__ void simt_epilogue(const float* sC, int ldc, int m0, int tn, const GemmArgs& a, int tid, int nt) {
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
    float* act = reinterpret_cast<float*>(a.act);
    for (int u = tid; u < BM * (H2 / 4); u += nt) {
      const int r = u / (H2 / 4), c = (u % (H2 / 4)) * 4;
      const int m = m0 + r;
      if (m >= a.M) continue;
      const f32x4 g = *reinterpret_cast<const f32x4*>(sC + r * ldc + c);
      const f32x4 up = *reinterpret_cast<const f32x4*>(sC + r * ldc + H2 + c);
      f32x4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = silu_mul(g[e], up[e]);
      vec4<float>::store(act + (size_t)m * a.ld_act + n0 + c, y);
    }
  } else {  // EPI_QKV, one 96-wide head per tile
    const int hd = 96, half = 48;
    const int col0 = tn * BN;
    const int q_end = a.nh * hd, k_end = (a.nh + a.nkv) * hd;
    if (col0 >= a.N) return;
    float* qo = reinterpret_cast<float*>(a.q);
    float* ko = reinterpret_cast<float*>(a.k);
    float* vo = reinterpret_cast<float*>(a.vt);
    if (col0 < k_end) {
      float* dst = col0 < q_end ? qo : ko;
      const int head = col0 < q_end ? col0 / hd : (col0 - q_end) / hd;
      const int nheads = col0 < q_end ? a.nh : a.nkv;
      for (int u = tid; u < BM * (half / 4); u += nt) {
        const int r = u / (half / 4), d = (u % (half / 4)) * 4;
        const int m = m0 + r;
        if (m >= a.M) continue;
        const int b = m / a.S, s = m - b * a.S;
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(sC + r * ldc + d);
        const f32x4 x2 = *reinterpret_cast<const f32x4*>(sC + r * ldc + half + d);
        const f32x4 cs = vec4<float>::load(a.rope_cos + (size_t)s * half + d);
        const f32x4 sn = vec4<float>::load(a.rope_sin + (size_t)s * half + d);
        float* base = dst + ((size_t)(b * nheads + head) * a.S + s) * hd;
        vec4<float>::store(base + d, x1 * cs - x2 * sn);
        vec4<float>::store(base + half + d, x2 * cs + x1 * sn);
      }
    } else {
      const int head = (col0 - k_end) / hd;
      for (int u = tid; u < hd * (BM / 8); u += nt) {
        const int d = u / (BM / 8), rg = (u % (BM / 8)) * 8;
        const int mf = m0 + rg;
        if (mf >= a.M) continue;
        const int bf = mf / a.S, sf = mf - bf * a.S;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = sC[(rg + e) * ldc + d];
        if (mf + 7 < a.M && sf + 7 < a.S && (sf & 7) == 0) {
          store8<float>(vo + ((size_t)(bf * a.nkv + head) * hd + d) * a.s_pad + sf, v);
        } else {
          for (int e = 0; e < 8; ++e) {
            const int m = mf + e;
            if (m >= a.M) break;
            const int b = m / a.S, s = m - b * a.S;
            vo[((size_t)(b * a.nkv + head) * hd + d) * a.s_pad + s] = v[e];
          }
        }
      }
    }
  }
}

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
      const f32x4 v = vec4<float>::load(W + (size_t)w_row_simt<BN>(a, tn, rw, EPI) * a.K + k0 + cw);
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
  simt_epilogue<EPI, BM, BN>(sC, LDC, m0, tn, a, tid, NT);
}

}  // namespace phi
