/*
 * phi.h - C ABI of an MI355X (gfx950) engine for Phi-3-style prefill logits
 * and for K16/V8 paged decode attention.
 *
 * What is computed comes from three pages:
 *   [P1] "Phi-3-mini: fused-tensor direct loading in a sovereign inference
 *        engine" - a dense Phi-3-mini-4k forward that loads the fused Q/K/V
 *        and gate/up projections as single tensors (section 1, Contribution;
 *        section 5, "Loading path"), head_dim 96 and an untied lm_head
 *        (section 2, Methods table), plain RoPE up to 4k positions (Abstract;
 *        section 4), f16 and 8-bit precision paths (section 2, "Precision"),
 *        no BOS prepended (section 2, "Stimulus / inputs").
 *   [P2] "The direct HF-logits parity harness" - the engine emits logits for
 *        every token position (section 1; section 5, "Engine dump").
 *   [P3] "Phi-4: quality transfer and interrupted throughput studies" -
 *        FP16 keys with E4M3 FP8 values in a paged KV pool, 40 query heads
 *        over 10 KV heads at head dimension 128 (setup paragraph), pool sizes
 *        in token slots per layer (pool paragraph), attention plus merge
 *        kernels on the decode path (matched diagnostic profiles).
 *
 * Conventions for every entry point
 *  - All tensors are device memory owned by the caller, row-major, densely
 *    packed, 16-byte aligned.  Linear weights are [out, in] and a linear layer
 *    computes y = x W^T.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    work on it and return; results are ready when the stream is synchronised.
 *    Faults inside kernels surface at that synchronisation.
 *  - Every argument check runs on the host before any HIP call; a failed check
 *    returns its status and enqueues nothing.  PHI_E_HIP means a HIP call or a
 *    kernel launch failed (hipGetLastError) after checks passed.
 *  - No entry point allocates device memory; scratch comes from the caller's
 *    `workspace` of at least the size the matching *_workspace_bytes returns.
 *    Two calls in flight at once need two workspaces.
 */
#ifndef PHI_H
#define PHI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum phi_status {
  PHI_OK = 0,
  PHI_E_NULL = 1,      /* a required pointer is NULL                          */
  PHI_E_SHAPE = 2,     /* a size is outside the supported set                 */
  PHI_E_DTYPE = 3,     /* unknown weight type                                 */
  PHI_E_RANGE = 4,     /* a value is out of range (seq > max_pos, ...)        */
  PHI_E_WORKSPACE = 5, /* workspace or state buffer smaller than required     */
  PHI_E_ALIGN = 6,     /* a device pointer is not 16-byte aligned             */
  PHI_E_HIP = 7        /* a HIP call or kernel launch failed                  */
} phi_status;

/* Weight storage types ([P1] section 2, "Precision": f16 primary, 8-bit
 * quantised check).  F32 stores every weight as float32 and computes in fp32.
 * F16 stores every weight as IEEE binary16; activations are rounded to f16 at
 * GEMM inputs, accumulation is fp32, the residual stream stays fp32.
 * I8 stores each linear weight (fused qkv, o, fused gate_up, down, lm_head) as
 * int8 codes q[N][K] plus one binary16 scale s[N] per output row, meaning
 * W[n][k] = q[n][k] * s[n]; embedding and norm gains are binary16. */
typedef enum phi_wtype { PHI_WT_F32 = 0, PHI_WT_F16 = 1, PHI_WT_I8 = 2 } phi_wtype;

typedef struct phi_config {
  int32_t n_layers;
  int32_t hidden;       /* H; multiple of 64, at most 8192                    */
  int32_t n_heads;      /* query heads                                        */
  int32_t n_kv_heads;   /* divides n_heads (n_kv_heads == n_heads: MHA)       */
  int32_t head_dim;     /* 96 ([P1] section 2); 64 or 128 on the binary16 and
                           int8 paths (other dense families, [P3]'s Phi-4)   */
  int32_t intermediate; /* I; multiple of 128                                 */
  int32_t vocab;        /* V; multiple of 4                                   */
  int32_t max_pos;      /* longest sequence; at most 4096 ([P1] section 4)   */
  float rms_eps;
  float rope_theta;
  int32_t wtype;        /* phi_wtype                                          */
} phi_config;

/* One linear weight: w is [N][K] of the weight type; scale is binary16 [N]
 * for PHI_WT_I8 and must be NULL otherwise. */
typedef struct phi_linear {
  const void* w;
  const void* scale;
} phi_linear;

/* Per-layer weights.  qkv is the fused [Wq; Wk; Wv] tensor of
 * (n_heads + 2 n_kv_heads) * head_dim rows, in that row order; gate_up is the
 * fused [Wgate; Wup] tensor of 2 I rows, gate rows first ([P1] section 1).
 * ln1 / ln2 are the RMSNorm gains [H] before attention and before the MLP. */
typedef struct phi_layer_weights {
  const void* ln1;
  phi_linear qkv;
  phi_linear o;
  const void* ln2;
  phi_linear gate_up;
  phi_linear down;
  const void* qkv_bias; /* optional [(n_heads + 2 n_kv_heads) head_dim] binary16
                           added to the fused QKV product before RoPE
                           (Qwen2-style families, [P2] section 3); NULL: none.
                           Not on the float32 path.                          */
} phi_layer_weights;

typedef struct phi_weights {
  const void* embed;                /* [V][H]                                  */
  const phi_layer_weights* layers;  /* host array of n_layers entries          */
  const void* final_norm;           /* [H]                                     */
  phi_linear lm_head;               /* [V][H], untied from embed ([P1] sec. 2);
                                       a tied model passes embed here        */
} phi_weights;

typedef struct phi_model phi_model; /* opaque host object */

/* Bytes of device state phi_load_fused fills (RoPE cos/sin tables). */
size_t phi_state_bytes(const phi_config* cfg);

/* Direct load of the fused tensors ([P1] section 1 and section 5, "Loading
 * path"): records the caller's device pointers - the fused qkv and gate_up
 * tensors are each consumed whole by one GEMM, never split or copied - and
 * writes the RoPE tables into `state` (device, state_bytes >= phi_state_bytes).
 * Weight buffers and `state` are borrowed and must outlive the model; the
 * layers array is copied.  This call synchronises `stream` once (table upload).
 * On success *out holds a model to release with phi_free. */
phi_status phi_load_fused(const phi_config* cfg, const phi_weights* w, void* state, size_t state_bytes,
                          void* stream, phi_model** out);

/* Workspace bytes phi_prefill_logits needs for `batch` sequences of `seq` ids. */
size_t phi_workspace_bytes(const phi_model* m, int32_t batch, int32_t seq);

/* Prefill forward, ids -> logits at every position ([P1] section 1; [P2]
 * section 1, per-token logit dump):
 *   x = embed[ids]; per layer: x += o(attn(rope(qkv(rmsnorm(x))))),
 *   x += down(silu(gate) * up (gate_up(rmsnorm(x)))); logits = lm_head(rmsnorm(x)).
 * ids: device int32 [batch][seq]; position s of each sequence is s (no BOS,
 * [P1] section 2).  logits: device float32 [batch][seq][V].
 * Requires 1 <= seq <= max_pos, batch >= 1.  An id outside [0, V) is not a
 * host-checkable error (ids live on the device): its row of x is set to NaN,
 * so that position's logits - and, through attention, later positions of the
 * same sequence - come out NaN; no memory outside the tensors is touched. */
phi_status phi_prefill_logits(const phi_model* m, const int32_t* ids, int32_t batch, int32_t seq,
                              float* logits, void* workspace, size_t workspace_bytes, void* stream);

/* phi_prefill_logits with the ids in host memory (the per-token logit dump
 * of [P2] section 1 takes token ids from the caller's file).  Every id is
 * checked on the host first: one outside [0, V) returns PHI_E_RANGE, as do
 * the checks of phi_prefill_logits, before anything is enqueued.  The ids are
 * then copied on `stream` into a region of the same workspace
 * (phi_workspace_bytes covers it), so ids_host must stay valid and unchanged
 * until the stream has run that copy, as for any asynchronous host-to-device
 * copy (from pageable memory HIP has read it before returning).  The result
 * is identical to phi_prefill_logits on the same ids. */
phi_status phi_prefill_logits_host_ids(const phi_model* m, const int32_t* ids_host, int32_t batch, int32_t seq,
                                       float* logits, void* workspace, size_t workspace_bytes, void* stream);

void phi_free(phi_model* m);

/* Static text for a status code. */
const char* phi_strerror(int32_t status);

/* ---- per-stage device timing of phi_prefill_logits ------------------------
 * Off by default.  When enabled, every stage of phi_prefill_logits gets two
 * HIP events on the call's stream.  A stage of one kernel passes them to that
 * kernel's dispatch (hipExtLaunchKernelGGL), so they time the kernel itself,
 * as a kernel trace does; the QKV stage with a KV cache (two launches) records
 * them around both.  A stage's time is the device time of its own launches
 * inside real forwards.  phi_profile_read
 * waits for the recorded events, writes per-stage total milliseconds and
 * launch counts (arrays of PHI_PROF_N), and clears the record.  Events are
 * created on the first enabled call; at most 16 forwards may be recorded
 * between reads (PHI_E_RANGE otherwise, checked before anything is enqueued).
 * Not for concurrent use of one model from several threads. */
enum {
  PHI_PROF_EMBED = 0,   /* embedding gather + first RMSNorm */
  PHI_PROF_QKV = 1,     /* fused QKV GEMM + RoPE */
  PHI_PROF_ATTN = 2,    /* causal attention */
  PHI_PROF_O = 3,       /* o_proj GEMM (+ residual or split partials) */
  PHI_PROF_NORM = 4,    /* RMSNorm (+ split-K reduce) after o_proj and down */
  PHI_PROF_GATE_UP = 5, /* fused gate/up GEMM + SiLU*up */
  PHI_PROF_DOWN = 6,    /* down GEMM (+ residual or split partials) */
  PHI_PROF_LM_HEAD = 7, /* lm_head GEMM */
  PHI_PROF_N = 8
};
phi_status phi_profile_enable(phi_model* m, int32_t enable);
phi_status phi_profile_read(phi_model* m, double* ms_out, int64_t* launches_out);

/* ---- building blocks, exposed for kernel-level checks ------------------- */

/* y[M][N] (float32) = a[M][K] w[N][K]^T with the prefill GEMM kernel.
 * wtype PHI_WT_F16: a, w binary16.  PHI_WT_I8: a binary16, w int8 with
 * binary16 row scales `scale` [N].  PHI_WT_F32: a, w float32.
 * K must be a multiple of 64, N a multiple of 4. */
phi_status phi_linear_f32out(int32_t wtype, const void* a, const void* w, const void* scale, float* y,
                             int32_t M, int32_t N, int32_t K, void* stream);

/* act[M][I] = silu(a w_gate^T) * (a w_up^T), the fused gate/up projection with
 * its SiLU(gate) * up epilogue, where w = [w_gate; w_up] is the single fused
 * tensor of 2 I rows, gate rows first ([P1] section 1).  Same kernel as the
 * prefill's MLP step.  Types as in phi_linear_f32out; act is float32 for
 * PHI_WT_F32 and binary16 otherwise.  I must be a multiple of 128 and K of 64. */
phi_status phi_gate_up_silu(int32_t wtype, const void* a, const void* w, const void* scale, void* act,
                            int32_t M, int32_t I, int32_t K, void* stream);

/* Causal softmax attention of the prefill ([P1] section 2: head_dim 96):
 * out[b][s][h][d] = sum_{t <= s} softmax_t(q[b][h][s] . k[b][g][t] / sqrt(96)) v[b][g][t][d],
 * g = h / (n_heads / n_kv_heads).  Layouts: q [B][n_heads][S][96],
 * k [B][n_kv_heads][S][96], vt [B][n_kv_heads][96][s_pad] (V transposed, row
 * stride s_pad = S rounded up to a multiple of 64; columns >= S are ignored),
 * out [B][S][n_heads * 96].  act_f32 = 0: all binary16; 1: all float32. */
size_t phi_attention_vt_stride(int32_t seq);
phi_status phi_attention_prefill(int32_t act_f32, const void* q, const void* k, const void* vt, void* out,
                                 int32_t batch, int32_t seq, int32_t n_heads, int32_t n_kv_heads,
                                 int32_t head_dim, void* stream);

/* ---- K16/V8 paged decode attention ([P3]) ---------------------------------
 * One decode step of one layer: for sequence b and query head h, with
 * g = h / (n_q_heads / n_kv_heads) and L = ctx_lens[b],
 *   out[b][h] = v_scale[g] * sum_{t < L} softmax_t(sm_scale * q[b][h] . K_t) dec(V_t)
 * where token t of sequence b sits in physical page block_table[b][t / 16],
 * slot t % 16; K_t = k_pool[page][g][slot][:] (binary16) and V_t =
 * v_pool[page][g][slot][:] (OCP E4M3FN bytes, decoded exactly).  Keys FP16 and
 * values E4M3 with a per-KV-head float32 scale follow [P3]'s K16/V8 cache.
 *   q        binary16 [B][n_q_heads][D]
 *   k_pool   binary16 [n_pages][n_kv_heads][16][D]
 *   v_pool   uint8    [n_pages][n_kv_heads][16][D]
 *   v_scale  float32  [n_kv_heads]
 *   block_table int32 [B][max_pages], ctx_lens int32 [B] (device)
 *   out      binary16 [B][n_q_heads][D]
 * Supported: D = 128, page_size = 16, n_q_heads / n_kv_heads <= 8 and
 * dividing.  The work is split over the context (split-KV); partial results
 * are combined by a log-sum-exp merge kernel ([P3], "attention and merge").
 * When one split per sequence suffices (the context fits one split and the
 * (sequence, KV head) pairs fill the GPU) the split kernel normalises the
 * output itself and no merge runs; the workspace size follows the plan.
 * max_ctx is the longest context of the call (1 <= max_ctx <= max_pages *
 * 16, PHI_E_RANGE otherwise): it sizes the split plan and the workspace, so
 * the workspace query and the call must use the same value.
 * Device-side values are checked in the kernel: a ctx_len outside
 * [1, max_ctx] or a page id outside [0, n_pages) makes that sequence's
 * output NaN instead of reading outside the pool or dropping the pages past
 * the plan. */
size_t attn_decode_k16v8_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                         int32_t head_dim, int32_t max_ctx);
phi_status attn_decode_k16v8(const void* q, const void* k_pool, const void* v_pool, const float* v_scale,
                             const int32_t* block_table, const int32_t* ctx_lens, int32_t batch,
                             int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                             int32_t n_pages, int32_t max_pages, int32_t max_ctx, float sm_scale, void* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---- decode attention without a workspace ---------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, checks, kernels and results as attn_decode_k16v8, without the
 * workspace: the split partials go to a fixed scratch array inside the
 * library, PHI_DECODE_SCRATCH_BYTES on each GPU the library runs on, held
 * from the first call on that GPU until the process ends.  A call whose plan
 * needs more (attn_decode_k16v8_workspace_bytes tells) returns
 * PHI_E_WORKSPACE before any HIP call.  `stream` must belong to the current
 * device (PHI_E_RANGE otherwise), whose scratch copy the call uses.  The call
 * allocates nothing: no hipMalloc, no library allocation.  Every call on one
 * GPU shares that GPU's scratch array, which keeps the last call's partials:
 * calls that overlap in time on one GPU (other streams, other threads) race
 * and must be serialised by the caller.  Nothing needs clearing between
 * calls: every partial a call reads is written earlier in the same call. */
#define PHI_DECODE_SCRATCH_BYTES (16u << 20)
phi_status attn_decode_k16v8_noalloc(const void* q, const void* k_pool, const void* v_pool, const float* v_scale,
                                     const int32_t* block_table, const int32_t* ctx_lens, int32_t batch,
                                     int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                                     int32_t n_pages, int32_t max_pages, int32_t max_ctx, float sm_scale, void* out,
                                     void* stream);

/* ---- K16/V8 cache write ([P3]) --------------------------------------------
 * The step before decode attention: append one token per sequence to the
 * paged pool ([P3] names the write of the compressed cache in its
 * candidate-kernel description).  For sequence b and KV head g, with
 * t = positions[b], page = block_table[b][t / 16] and slot = t % 16:
 *   k_pool[page][g][slot][:] = k_new[b][g][:]            (binary16, copied)
 *   v_pool[page][g][slot][d] = E4M3(v_new[b][g][d] / v_scale[g])
 * where the quotient is an IEEE fp32 division and E4M3 rounds it to the
 * nearest OCP E4M3FN value, ties to even, saturating magnitudes above 448 to
 * +-448 and mapping NaN to 0x7F.  Nothing else in the pools changes.
 *   k_new, v_new binary16 [B][n_kv_heads][D]
 *   v_scale  float32 [n_kv_heads]
 *   block_table int32 [B][max_pages], positions int32 [B] (device)
 *   k_pool binary16 / v_pool uint8 [n_pages][n_kv_heads][16][D], updated in place
 * Supported: D = 128, page_size = 16.  batch = 0 returns PHI_OK before any
 * other check (the per-sequence pointers may then be NULL).  Two
 * sequences must not name the same (page, slot).  Device-side values are
 * checked in the kernel: a sequence whose position lies outside
 * [0, max_pages * 16) or whose page id lies outside [0, n_pages) is not
 * written. */
phi_status kv_append_k16v8(const void* k_new, const void* v_new, const float* v_scale, const int32_t* block_table,
                           const int32_t* positions, int32_t batch, int32_t n_kv_heads, int32_t head_dim,
                           int32_t page_size, int32_t n_pages, int32_t max_pages, void* k_pool, void* v_pool,
                           void* stream);

/* ---- K16/V8 cached decoding of a loaded model ([P3]) ------------------------
 * A paged cache for every layer: keys binary16, values E4M3 with a float32
 * scale per (layer, KV head) ([P3] setup paragraph), 16-token pages shared by
 * the sequences of a batch through one block table.  All device memory is
 * the caller's; the two pointer arrays are host arrays.
 *   k_pools[l]  binary16 [n_pages][n_kv_heads][16][head_dim], layer l
 *   v_pools[l]  uint8    [n_pages][n_kv_heads][16][head_dim], layer l
 *   v_scale     float32  [n_layers][n_kv_heads] (device)
 *   block_table int32    [batch][max_pages] (device): token t of sequence b
 *               is in page block_table[b][t / 16], slot t % 16
 * Models: head_dim 128, n_heads / n_kv_heads in {1, 2, 4, 8}, binary16 or
 * int8 weights. */
typedef struct {
  void* const* k_pools;
  void* const* v_pools;
  const float* v_scale;
  const int32_t* block_table;
  int32_t n_pages, max_pages, page_size;
} phi_kv_cache;

/* phi_prefill_logits, and in addition every layer's keys and values of
 * tokens 0..seq-1 of each sequence are written into the cache with the
 * encoding of kv_append_k16v8 (the prefill's own attention uses them
 * unquantised).  seq <= max_pages * 16 (PHI_E_RANGE otherwise).  Workspace:
 * phi_workspace_bytes(m, batch, seq). */
phi_status phi_prefill_fill_k16v8(const phi_model* m, const int32_t* ids, int32_t batch, int32_t seq,
                                  float* logits, const phi_kv_cache* cache, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* One decode step: sequence b's token ids[b] at position positions[b] (its
 * cache length; both device int32 [batch]) goes through every layer - RMSNorm,
 * fused QKV with RoPE at that position, the cache write of its key and value
 * (kv_append_k16v8), decode attention over positions[b] + 1 cached tokens
 * (attn_decode_k16v8), o_proj, RMSNorm, fused gate/up, down - and the final
 * RMSNorm and lm_head give logits float32 [batch][vocab].  max_ctx bounds
 * positions[b] + 1 for every b (1 <= max_ctx <= max_pages * 16 and
 * <= max_pos; PHI_E_RANGE otherwise).  Device-side values are checked in the
 * kernels: a position whose slot lies outside the table or pool is not
 * written, and a position outside [0, max_ctx) makes that sequence's
 * attention output, and so its logits, NaN (its RoPE position is then
 * clamped into the table, which only affects that NaN row).  Workspace:
 * phi_decode_workspace_bytes(m, batch, max_ctx). */
size_t phi_decode_workspace_bytes(const phi_model* m, int32_t batch, int32_t max_ctx);
phi_status phi_decode_step_k16v8(const phi_model* m, const int32_t* ids, const int32_t* positions, int32_t batch,
                                 int32_t max_ctx, const phi_kv_cache* cache, float* logits, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Token slots per layer of a KV pool of budget_bytes split evenly over
 * n_layers, each token holding one key of k_bytes and one value of v_bytes per
 * element per KV head, rounded down to whole pages ([P3] pool paragraph:
 * 32 GiB, 40 layers, 10 KV heads x 128 gives 223,696 slots for 2 + 1 bytes
 * and 167,760 for 2 + 2 bytes with 16-token pages).  Returns -1 on a
 * non-positive argument. */
int64_t phi_kv_pool_slots(int64_t budget_bytes, int32_t n_layers, int32_t n_kv_heads, int32_t head_dim,
                          int32_t k_bytes, int32_t v_bytes, int32_t page_size);

#ifdef __cplusplus
}
#endif

#endif /* PHI_H */
