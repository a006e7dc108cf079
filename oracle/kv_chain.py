"""fp64 oracle of the K16/V8 cached decode chain: a prefill that fills the
paged cache, then decode steps that append one token per sequence and attend
over the cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows the page "Phi-4: quality transfer and interrupted throughput studies":
the cache keeps keys in FP16 and values in E4M3 FP8 with model-specific
scales (setup paragraph), one new token per sequence is written into the
compressed cache before attention reads it (the candidate kernel
description), and decode attention reads the keys and the decoded values
(oracle/decode.py).  The layer arithmetic is the Phi-3-style decoder of
oracle/prefill.py at any head geometry (the Phi-4 setup: 40 query heads over
10 KV heads at head dimension 128).

Readings where the page is silent:
  - The cache stores the key as the binary16 rounding of its value, and the
    value as the E4M3 code of fp32(binary16(v)) / scale: the f16 engine holds
    activations in binary16 before the cache write (P1 section 2,
    "Precision"), and the division by the per-head scale is taken in fp32 as
    in oracle/decode.kv_append.
  - The prefill's own attention uses the unquantised keys and values; only
    later decode steps read the compressed cache.
  - `exact=True` keeps fp64 keys and values in the cache; then a decode step
    must reproduce the prefill of the longer sequence (a pin of the chain).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import decode
from .prefill import apply_rope, causal_attention, linear, rms_norm, rope_angles, silu, widen


def cache_key(k: np.ndarray, exact: bool = False) -> np.ndarray:
    """Stored form of keys, as fp64 values."""
    return k.astype(np.float64) if exact else k.astype(np.float16).astype(np.float64)


def cache_value_codes(v: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """E4M3 codes of values v [..., kv_heads, d] with per-head scales [kv_heads]."""
    v16 = np.asarray(v, dtype=np.float64).astype(np.float16).astype(np.float32)
    q = (v16 / np.asarray(scale, dtype=np.float32)[:, None]).astype(np.float32)
    return decode.e4m3_encode(q)


@dataclass
class SeqCache:
    """One sequence's cache: per layer a list of (key fp64 [kv_heads, d],
    value fp64 [kv_heads, d] as read back, value codes or None)."""
    layers: list = field(default_factory=list)

    def length(self) -> int:
        return len(self.layers[0]) if self.layers else 0


def _store(cache_layer: list, k, v, scale, exact: bool):
    """Append tokens k, v [T, kv_heads, d] to one layer of a sequence cache."""
    for t in range(k.shape[0]):
        if exact:
            cache_layer.append((k[t].astype(np.float64), v[t].astype(np.float64), None))
        else:
            codes = cache_value_codes(v[t], scale)
            vv = decode.e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[:, None]
            cache_layer.append((cache_key(k[t]), vv, codes))


def _qkv(x, lw, cfg, positions):
    nh, nkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    T = x.shape[0]
    xn = rms_norm(x, lw["ln1"], cfg.rms_eps)
    qkv = linear(xn, lw["qkv"])
    if "qkv_bias" in lw:
        qkv = qkv + widen(lw["qkv_bias"])
    q = qkv[:, : nh * hd].reshape(T, nh, hd)
    k = qkv[:, nh * hd : (nh + nkv) * hd].reshape(T, nkv, hd)
    v = qkv[:, (nh + nkv) * hd :].reshape(T, nkv, hd)
    ang = rope_angles(positions, hd, cfg.rope_theta)
    return apply_rope(q, ang), apply_rope(k, ang), v


def _mlp_tail(x, a, lw, cfg):
    x = x + linear(a, lw["o"])
    xn = rms_norm(x, lw["ln2"], cfg.rms_eps)
    gu = linear(xn, lw["gate_up"])
    I = cfg.intermediate
    return x + linear(silu(gu[:, :I]) * gu[:, I:], lw["down"])


def prefill_fill(cfg, weights, ids: np.ndarray, v_scale: np.ndarray, exact: bool = False, logits: bool = True):
    """Prefill of one sequence (ids int [S]) that fills its cache.

    Returns (logits fp64 [S, vocab] or None when logits=False, SeqCache,
    per-layer raw (k, v) fp64).  v_scale fp32 [n_layers, kv_heads]."""
    ids = np.asarray(ids)
    S = ids.shape[0]
    x = widen(weights.embed[ids])
    pos = np.arange(S)
    cache = SeqCache()
    raw = []
    for l in range(cfg.n_layers):
        lw = weights.layer(l)
        q, k, v = _qkv(x, lw, cfg, pos)
        raw.append((k, v))
        layer_cache: list = []
        _store(layer_cache, k, v, v_scale[l], exact)
        cache.layers.append(layer_cache)
        a = causal_attention(q, k, v, 1.0 / np.sqrt(cfg.head_dim)).reshape(S, -1)
        x = _mlp_tail(x, a, lw, cfg)
    out = linear(rms_norm(x, weights.final_norm, cfg.rms_eps), weights.lm_head) if logits else None
    return out, cache, raw


def decode_step(cfg, weights, token: int, cache: SeqCache, v_scale: np.ndarray, exact: bool = False,
                return_values: bool = False):
    """One decode step of one sequence: the token at position cache.length()
    is appended to every layer's cache, then attends over all cached tokens.
    Returns logits fp64 [vocab]; the cache grows by one token.  With
    return_values, returns (logits, values) where values[l] is the step's
    unquantised value [kv_heads, d] of layer l (what was encoded into the
    cache)."""
    p = cache.length()
    x = widen(weights.embed[np.array([token])])
    nh, nkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    group = nh // nkv
    values = []
    for l in range(cfg.n_layers):
        lw = weights.layer(l)
        q, k, v = _qkv(x, lw, cfg, np.array([p]))  # q [1, heads, d]
        values.append(v[0])
        _store(cache.layers[l], k, v, v_scale[l], exact)
        if exact:
            K = np.stack([e[0] for e in cache.layers[l]])   # [p + 1, kv_heads, d]
            V = np.stack([e[1] for e in cache.layers[l]])
            a = np.empty((nh, hd))
            for h in range(nh):
                g = h // group
                s = (K[:, g, :] @ q[0, h]) / np.sqrt(hd)
                e = np.exp(s - s.max())
                a[h] = (e / e.sum()) @ V[:, g, :]
        else:
            # the compressed cache as pages, read by the decode-attention oracle
            n_pages = -(-(p + 1) // 16)
            table = np.arange(n_pages, dtype=np.int32)[None, :]
            kp, vp = pools_from([cache], table, n_pages, l)
            a = decode.decode_attention(q.astype(np.float64), kp, vp, v_scale[l], table,
                                        np.array([p + 1]), 1.0 / np.sqrt(hd))[0]
        x = _mlp_tail(x, a.reshape(1, -1), lw, cfg)
    out = linear(rms_norm(x, weights.final_norm, cfg.rms_eps), weights.lm_head)[0]
    return (out, values) if return_values else out


def value_scales_from(raw_per_seq: list, n_layers: int) -> np.ndarray:
    """A per-(layer, KV head) scale rule for synthetic models: amax |v| over
    the given prefill values / 448 (the E4M3 maximum), as fp32
    [n_layers, kv_heads].  raw_per_seq: list over sequences of prefill_fill's
    `raw`."""
    out = []
    for l in range(n_layers):
        amax = np.max([np.abs(r[l][1]).max(axis=(0, 2)) for r in raw_per_seq], axis=0)
        out.append(amax / 448.0)
    return np.asarray(out, dtype=np.float32)


def pools_from(caches: list, block_table: np.ndarray, n_pages: int, layer: int, page: int = 16):
    """Pools [n_pages, kv_heads, page, d] (binary16 keys, E4M3 codes) holding
    layer `layer` of every sequence's cache at block_table's pages; slots no
    sequence owns are zero."""
    first = caches[0].layers[layer][0]
    nkv, d = first[0].shape
    kp = np.zeros((n_pages, nkv, page, d), dtype=np.float16)
    vp = np.zeros((n_pages, nkv, page, d), dtype=np.uint8)
    for b, c in enumerate(caches):
        for t, (k, _, codes) in enumerate(c.layers[layer]):
            pg = block_table[b][t // page]
            kp[pg, :, t % page] = k.astype(np.float16)
            vp[pg, :, t % page] = codes
    return kp, vp
