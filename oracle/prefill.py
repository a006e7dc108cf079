"""fp64 oracle of the Phi-3-style decoder prefill: token ids -> logits.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed follows the page "Phi-3-mini: fused-tensor direct loading in
a sovereign inference engine": a dense Phi-3-mini-4k forward pass whose fused
Q/K/V and gate/up projections are single tensors (section 1, Contribution),
head_dim 96 and an untied lm_head (section 2, Methods table), plain RoPE in
the 4k regime (Abstract; section 4), no BOS prepended (Methods table,
"Stimulus / inputs"), logits at every position (page "The direct HF-logits
parity harness", section 1: per-token logit dump).  The page's oracle is the
HuggingFace Phi-3 model; where the page leaves a convention open (row order
inside the fused tensors, RoPE pairing) this follows that model, and the
tests pin the whole forward against it.

Weights enter as stored (float32, float16, or int8 codes with a float16 scale
per output row) and are widened to fp64; nothing is rounded afterwards.
"""
from __future__ import annotations

import numpy as np


def widen(w) -> np.ndarray:
    """Stored weight -> fp64.  An int8 weight is the pair (q [N, K], s [N]) and
    means q[n, k] * s[n] (symmetric per-output-row quantization)."""
    if isinstance(w, tuple):
        q, s = w
        return q.astype(np.float64) * s.astype(np.float64)[:, None]
    return np.asarray(w, dtype=np.float64)


def linear(x: np.ndarray, w) -> np.ndarray:
    """y = x W^T with W stored [out, in] (PyTorch Linear layout)."""
    return x @ widen(w).T


def rms_norm(x: np.ndarray, g, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * widen(g)


def rope_angles(positions: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """angle[p, i] = p * theta^(-2i / head_dim), i < head_dim / 2 (no scaling:
    plain RoPE, the 4k regime of P1)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    return np.outer(np.asarray(positions, dtype=np.float64), inv_freq)


def apply_rope(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate pairs (i, i + d/2) of every head: x [S, heads, d], angles [S, d/2].
    x'[i] = x[i] cos - x[i + d/2] sin ; x'[i + d/2] = x[i + d/2] cos + x[i] sin."""
    half = x.shape[-1] // 2
    c = np.cos(angles)[:, None, :]
    s = np.sin(angles)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """a[p, h] = sum_{t <= p} softmax_t(scale * q[p, h] . k[t, g]) v[t, g], with
    g = h // (heads / kv_heads).  q [S, heads, d]; k, v [S, kv_heads, d]."""
    S, nh, d = q.shape
    group = nh // k.shape[1]
    out = np.empty((S, nh, v.shape[-1]), dtype=np.float64)
    for h in range(nh):
        g = h // group
        scores = (q[:, h, :] @ k[:, g, :].T) * scale
        for p in range(S):
            s = scores[p, : p + 1]
            e = np.exp(s - s.max())
            out[p, h] = (e / e.sum()) @ v[: p + 1, g, :]
    return out


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x)."""
    return x / (1.0 + np.exp(-x))


def decoder_layer(x: np.ndarray, lw: dict, cfg, positions: np.ndarray) -> np.ndarray:
    """One Phi-3 decoder layer on one sequence, x [S, H] fp64 -> [S, H].

    Fused Q/K/V: one product with the concatenated [Wq; Wk; Wv], rows split in
    that order; fused gate/up: one product with [Wg; Wu], gate rows first
    (P1 section 1: the fused tensors are used as single tensors).  An optional
    qkv_bias is added to that product before RoPE: the Qwen2 family of the
    parity harness page (section 3) carries one, Phi-3 does not."""
    nh, nkv, hd, I = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate
    S = x.shape[0]
    xn = rms_norm(x, lw["ln1"], cfg.rms_eps)
    qkv = linear(xn, lw["qkv"])
    if "qkv_bias" in lw:
        qkv = qkv + widen(lw["qkv_bias"])
    q = qkv[:, : nh * hd].reshape(S, nh, hd)
    k = qkv[:, nh * hd : (nh + nkv) * hd].reshape(S, nkv, hd)
    v = qkv[:, (nh + nkv) * hd :].reshape(S, nkv, hd)
    ang = rope_angles(positions, hd, cfg.rope_theta)
    q = apply_rope(q, ang)
    k = apply_rope(k, ang)
    a = causal_attention(q, k, v, 1.0 / np.sqrt(hd)).reshape(S, nh * hd)
    x = x + linear(a, lw["o"])
    xn = rms_norm(x, lw["ln2"], cfg.rms_eps)
    gu = linear(xn, lw["gate_up"])
    m = silu(gu[:, :I]) * gu[:, I:]
    return x + linear(m, lw["down"])


def final_hidden(cfg, weights, ids: np.ndarray, n_layers: int | None = None) -> np.ndarray:
    """The normalised final hidden state rmsnorm(x) * g_final, fp64 [B, S, H],
    that the untied lm_head multiplies: every step of the forward except the
    last product.

    `weights` provides .embed, .layer(l) (dict: ln1, qkv, o, ln2, gate_up,
    down), .final_norm and .lm_head, each as stored.  Positions run 0..S-1 from
    the first id of each sequence (no BOS).  `n_layers` < cfg.n_layers runs
    only the first layers (used to time a bounded sample)."""
    ids = np.asarray(ids)
    B, S = ids.shape
    L = cfg.n_layers if n_layers is None else n_layers
    E = weights.embed
    xs = [widen(E[ids[b]]) for b in range(B)]
    pos = np.arange(S)
    for l in range(L):
        lw = weights.layer(l)
        xs = [decoder_layer(x, lw, cfg, pos) for x in xs]
    return np.stack([rms_norm(x, weights.final_norm, cfg.rms_eps) for x in xs])


def logits_from_hidden(hidden: np.ndarray, lm_head) -> np.ndarray:
    """The last step of the forward: logits = hidden W_lm^T, fp64 (untied
    lm_head, P1 section 2, Methods table)."""
    return linear(np.asarray(hidden, dtype=np.float64), lm_head)


def prefill_logits(cfg, weights, ids: np.ndarray, n_layers: int | None = None) -> np.ndarray:
    """Logits fp64 [B, S, vocab] for ids int [B, S]: final_hidden followed by
    the lm_head product."""
    h = final_hidden(cfg, weights, ids, n_layers)
    out = np.empty(h.shape[:2] + (cfg.vocab,), dtype=np.float64)
    for b in range(h.shape[0]):
        out[b] = logits_from_hidden(h[b], weights.lm_head)
    return out
