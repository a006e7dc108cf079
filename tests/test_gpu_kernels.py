"""Kernel-level parity of the GEMM and prefill-attention kernels (GPU).

Each kernel is called through the C ABI and compared element by element with
the oracle's definition in fp64 on the same input bytes.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import prefill

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


# Phi-3-mini GEMM shapes (N, K): fused QKV, o_proj, fused gate/up, down, lm_head
MINI_SHAPES = [(9216, 3072), (3072, 3072), (16384, 3072), (3072, 8192), (32064, 3072)]


def _gemm_bound(a64, w64, tol):
    """Elementwise bound tol * (|a| |w|^T): fp32 accumulation error of a K-term
    dot product of exactly representable products."""
    return tol * (np.abs(a64) @ np.abs(w64).T) + 1e-30


@pytest.mark.parametrize("N,K", MINI_SHAPES)
@pytest.mark.parametrize("M", [512, 300])
def test_gemm_f16_mini_shapes(phi, M, N, K):
    _say(f"gemm f16 M={M} N={N} K={K}")
    a16 = synth.normal(11, f"gemm.a.{M}.{K}", (M, K), 1.0, np.float16)
    w16 = synth.normal(12, f"gemm.w.{N}.{K}", (N, K), 0.02, np.float16)
    y = phi.phi_linear_f32out(torch.from_numpy(a16).cuda(), torch.from_numpy(w16).cuda())
    torch.cuda.synchronize()
    a64, w64 = a16.astype(np.float64), w16.astype(np.float64)
    ref = prefill.linear(a64, w16)
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= _gemm_bound(a64, w64, 2e-4)), err.max()


@pytest.mark.parametrize("N,K", [(9216, 3072), (3072, 8192), (32064, 3072)])
def test_gemm_int8_rowscale(phi, N, K):
    M = 384
    _say(f"gemm i8 M={M} N={N} K={K}")
    a16 = synth.normal(13, f"gemm.a8.{M}.{K}", (M, K), 1.0, np.float16)
    q, s = synth.quantize_rows_i8(synth.normal(14, f"gemm.w8.{N}.{K}", (N, K), 0.02, np.float16))
    y = phi.phi_linear_f32out(torch.from_numpy(a16).cuda(), torch.from_numpy(q).cuda(),
                              torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    a64 = a16.astype(np.float64)
    ref = prefill.linear(a64, (q, s))
    wabs = np.abs(q.astype(np.float64)) * s.astype(np.float64)[:, None]
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= _gemm_bound(a64, wabs, 2e-4)), err.max()


@pytest.mark.parametrize("M,N,K", [(16, 1152, 384), (37, 2048, 384), (16, 384, 1024), (16, 4096, 384)])
def test_gemm_f32_tiny_shapes(phi, M, N, K):
    _say(f"gemm f32 M={M} N={N} K={K}")
    a = synth.normal(15, "gemm.a32", (M, K), 1.0, np.float32)
    w = synth.normal(16, "gemm.w32", (N, K), 0.02, np.float32)
    y = phi.phi_linear_f32out(torch.from_numpy(a).cuda(), torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    a64 = a.astype(np.float64)
    ref = prefill.linear(a64, w)
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= _gemm_bound(a64, w.astype(np.float64), 1e-5)), err.max()


@pytest.mark.parametrize("wtype,M,I,K", [("f16", 512, 8192, 3072), ("f16", 77, 1024, 384),
                                         ("i8", 300, 8192, 3072), ("f32", 40, 1024, 384),
                                         # 256x256 tiles (1024 tokens and more) with a ragged last M-tile:
                                         # binary16 by direct-to-LDS copies, int8 register-staged
                                         ("f16", 1100, 2048, 1024), ("i8", 1100, 2048, 1024)])
def test_gate_up_silu_epilogue(phi, wtype, M, I, K):
    _say(f"gate_up silu {wtype} M={M} I={I} K={K}")
    adt = np.float32 if wtype == "f32" else np.float16
    a = synth.normal(17, "gu.a", (M, K), 1.0, adt)
    w = synth.normal(18, "gu.w", (2 * I, K), 0.02, adt)
    wt = synth.quantize_rows_i8(w) if wtype == "i8" else w
    dev = lambda x: torch.from_numpy(x).cuda()
    if wtype == "i8":
        got = phi.phi_gate_up_silu(dev(a), dev(wt[0]), dev(wt[1]))
    else:
        got = phi.phi_gate_up_silu(dev(a), dev(w))
    torch.cuda.synchronize()
    gu = prefill.linear(a.astype(np.float64), wt)
    ref = prefill.silu(gu[:, :I]) * gu[:, I:]
    got = got.cpu().numpy().astype(np.float64)
    tol = 1e-6 if wtype == "f32" else 2e-3
    assert np.all(np.abs(got - ref) <= tol * (1 + np.abs(ref))), np.abs(got - ref).max()


def _attn_inputs(B, S, nh, nkv, dtype, seed, scale=1.0, D=96):
    q = synth.normal(seed, "attn.q", (B, nh, S, D), scale, dtype)
    k = synth.normal(seed, "attn.k", (B, nkv, S, D), scale, dtype)
    v = synth.normal(seed, "attn.v", (B, nkv, S, D), 1.0, dtype)
    return q, k, v


def _attn_gpu(phi, q, k, v):
    B, nkv, S, D = v.shape
    sp = phi.phi_attention_vt_stride(S)
    vt = np.zeros((B, nkv, D, sp), dtype=v.dtype)
    vt[..., :S] = v.transpose(0, 1, 3, 2)
    # poison the padding columns: the kernel must ignore them
    if sp > S:
        vt[..., S:] = np.nan
    out = phi.phi_attention_prefill(torch.from_numpy(q).cuda(), torch.from_numpy(k).cuda(),
                                    torch.from_numpy(vt).cuda())
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _attn_ref(q, k, v):
    B, nh, S, D = q.shape
    out = np.empty((B, S, nh * D))
    for b in range(B):
        o = prefill.causal_attention(q[b].transpose(1, 0, 2).astype(np.float64),
                                     k[b].transpose(1, 0, 2).astype(np.float64),
                                     v[b].transpose(1, 0, 2).astype(np.float64), 1 / np.sqrt(D))
        out[b] = o.reshape(S, nh * D)
    return out


@pytest.mark.parametrize("B,S,nh,nkv", [(1, 1, 4, 4), (1, 5, 4, 2), (2, 64, 4, 4), (1, 100, 2, 1),
                                        (1, 300, 8, 8), (2, 512, 4, 2), (1, 1000, 2, 2)])
def test_attention_f16_peaked(phi, B, S, nh, nkv):
    _say(f"attention f16 B={B} S={S} nh={nh} nkv={nkv}")
    q, k, v = _attn_inputs(B, S, nh, nkv, np.float16, 21 + S, scale=1.5)
    got = _attn_gpu(phi, q, k, v)
    ref = _attn_ref(q, k, v)
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - ref) <= 2e-3 + 2e-3 * np.abs(ref)), np.abs(got - ref).max()


@pytest.mark.parametrize("B,S,nh,nkv", [(1, 1, 4, 1), (1, 31, 8, 2), (2, 100, 8, 2), (1, 513, 40, 10)])
def test_attention_f16_head_dim_128(phi, B, S, nh, nkv):
    _say(f"attention f16 D=128 B={B} S={S} nh={nh} nkv={nkv}")
    q, k, v = _attn_inputs(B, S, nh, nkv, np.float16, 41 + S, scale=1.5, D=128)
    got = _attn_gpu(phi, q, k, v)
    ref = _attn_ref(q, k, v)
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - ref) <= 2e-3 + 2e-3 * np.abs(ref)), np.abs(got - ref).max()


# Launches of at least 384 workgroups of 128 queries take the shared-key-block
# kernel: ragged sequences (a last query block with one query, so waves with
# no queries; a last key block with one key), grouped heads, every head width.
@pytest.mark.parametrize("B,S,nh,nkv,D", [(3, 1000, 16, 4, 96), (1, 1537, 32, 32, 96), (2, 777, 40, 10, 128),
                                          (4, 600, 24, 8, 64)])
def test_attention_f16_shared_key_blocks(phi, B, S, nh, nkv, D):
    assert B * nh * (-(-S // 128)) >= 384
    _say(f"attention f16 shared blocks D={D} B={B} S={S} nh={nh} nkv={nkv}")
    q, k, v = _attn_inputs(B, S, nh, nkv, np.float16, 51 + S, scale=1.5, D=D)
    got = _attn_gpu(phi, q, k, v)
    ref = _attn_ref(q, k, v)
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - ref) <= 2e-3 + 2e-3 * np.abs(ref)), np.abs(got - ref).max()


@pytest.mark.parametrize("direction", [1.0, -1.0], ids=["rising", "falling"])
def test_attention_shared_key_blocks_moving_max(phi, direction):
    """Scores that ramp along the keys by about 60 log2 units over the
    sequence (rising: every query's maximum is its most recent key, so the
    running maximum keeps moving by more than the kernel's lazy threshold;
    falling: the first block holds the maximum and later blocks contribute
    almost nothing), checked element by element against the oracle."""
    B, S, nh, nkv, D = 1, 1537, 32, 32, 96
    assert B * nh * (-(-S // 128)) >= 384
    _say(f"attention f16 shared blocks, moving max ({'rising' if direction > 0 else 'falling'})")
    rng = np.random.default_rng(77)
    u = rng.standard_normal((nh, D))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    ramp = direction * np.linspace(-1.0, 1.0, S)                  # g(t)
    amp = 30.0 * np.sqrt(D) / np.log2(np.e)                        # c * a * g spans about +-30 log2 units
    q = np.broadcast_to(u[None, :, None, :] * np.sqrt(amp), (B, nh, S, D))
    k = u[None, :, None, :] * (np.sqrt(amp) * ramp)[None, None, :, None]
    k = k + 0.05 * rng.standard_normal((B, nkv, S, D))
    v = synth.normal(91, "attn.v", (B, nkv, S, D), 1.0, np.float16)
    q, k = np.ascontiguousarray(q, dtype=np.float16), np.ascontiguousarray(k, dtype=np.float16)
    got = _attn_gpu(phi, q, k, v)
    ref = _attn_ref(q, k, v)
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - ref) <= 2e-3 + 2e-3 * np.abs(ref)), np.abs(got - ref).max()


def test_attention_shared_key_blocks_rows_sum_to_one(phi):
    q, k, v = _attn_inputs(1, 3001, 16, 2, np.float16, 6, scale=2.0)
    got = _attn_gpu(phi, q, k, np.ones_like(v))
    assert np.abs(got - 1).max() <= 2e-3


@pytest.mark.parametrize("B,S,nh,nkv", [(1, 16, 4, 4), (2, 70, 4, 2)])
def test_attention_f32(phi, B, S, nh, nkv):
    _say(f"attention f32 B={B} S={S}")
    q, k, v = _attn_inputs(B, S, nh, nkv, np.float32, 31 + S, scale=1.5)
    got = _attn_gpu(phi, q, k, v)
    ref = _attn_ref(q, k, v)
    assert np.abs(got - ref).max() <= 1e-5


def test_attention_rows_sum_to_one(phi):
    # V = 1 everywhere: every output is exactly a sum of softmax weights
    q, k, v = _attn_inputs(1, 257, 4, 4, np.float16, 5, scale=2.0)
    got = _attn_gpu(phi, q, k, np.ones_like(v))
    assert np.abs(got - 1).max() <= 2e-3
