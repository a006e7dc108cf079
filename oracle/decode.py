"""fp64 oracle of K16/V8 paged decode attention, and KV-pool sizing.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows the page "Phi-4: quality transfer and interrupted throughput studies":
keys stored FP16 and values stored E4M3 FP8 with model-specific scales, the
Phi-4 geometry of 40 query heads over 10 KV heads at head dimension 128 (setup
paragraph), a paged persistent KV pool (pool paragraph), and attention plus a
merge kernel on the decode path (matched diagnostic profiles).  The value of
an E4M3 byte is the OCP 8-bit floating point E4M3 ("FN") definition: bias 7,
no infinities, S.1111.111 is NaN, maximum 448.
"""
from __future__ import annotations

import numpy as np


def e4m3_value(code: int) -> float:
    """Exact value of one OCP E4M3FN byte."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * 2.0 ** -6 * (m / 8.0)
    return s * 2.0 ** (e - 7) * (1.0 + m / 8.0)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


_E4M3_FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.int64)


def e4m3_encode(x) -> np.ndarray:
    """OCP E4M3FN code of each value: the nearest finite E4M3 value, ties to
    the code with an even mantissa, magnitudes beyond 448 saturating to +-448.
    (Written as a search over the 254 finite codes, so it is plainly the
    definition; a result of zero keeps the sign of the input, as IEEE rounding
    does.)  NaN encodes as 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    vals = E4M3_TABLE[_E4M3_FINITE]
    out = np.empty(flat.shape, dtype=np.uint8)
    for i, v in enumerate(flat):
        if np.isnan(v):
            out[i] = 0x7F
            continue
        a = min(abs(v), 448.0)
        d = np.abs(vals - np.copysign(a, v))
        best = np.flatnonzero(d == d.min())
        codes = _E4M3_FINITE[best]
        if len(codes) > 1:
            even = codes[(codes & 1) == 0]
            codes = even if len(even) else codes
        c = int(codes[0])
        if E4M3_TABLE[c] == 0.0:
            c = 0x80 if np.signbit(v) else 0x00
        out[i] = c
    return out.reshape(x.shape)


def kv_append(k_pool, v_pool, k_new, v_new, v_scale, block_table, positions):
    """Write token positions[b] of every sequence: K as given (binary16), V as
    the E4M3 code of the fp32 quotient v / v_scale[g] (the same fp32 rounding
    the kernel performs before choosing the code).  A sequence whose position
    or page id falls outside the table or the pool is left unwritten.  Returns
    new pools."""
    k_pool, v_pool = k_pool.copy(), v_pool.copy()
    B, Hkv, D = k_new.shape
    page = k_pool.shape[2]
    for b in range(B):
        p = int(positions[b])
        if not 0 <= p < block_table.shape[1] * page:
            continue
        phys = int(block_table[b][p // page])
        if not 0 <= phys < k_pool.shape[0]:
            continue
        q = (v_new[b].astype(np.float32) / v_scale.astype(np.float32)[:, None]).astype(np.float32)
        k_pool[phys, :, p % page, :] = k_new[b]
        v_pool[phys, :, p % page, :] = e4m3_encode(q)
    return k_pool, v_pool


def gather_sequence(pool: np.ndarray, block_table_row: np.ndarray, ctx_len: int) -> np.ndarray:
    """Logical token t of a sequence lives in physical page block_table[t // page],
    slot t % page.  pool [P, Hkv, page, D] -> [ctx_len, Hkv, D]."""
    page = pool.shape[2]
    n_pages = -(-ctx_len // page)
    pages = pool[np.asarray(block_table_row[:n_pages], dtype=np.int64)]   # [n, Hkv, page, D]
    seq = pages.transpose(0, 2, 1, 3).reshape(n_pages * page, pool.shape[1], pool.shape[3])
    return seq[:ctx_len]


def decode_attention(q, k_pool, v_pool, v_scale, block_table, ctx_lens, sm_scale: float) -> np.ndarray:
    """o[b, h] = v_scale[g] * sum_t softmax_t(sm_scale * q[b, h] . K[b, t, g]) dec(V[b, t, g])
    over the ctx_lens[b] cached tokens, g = h // (Hq / Hkv).  fp64 [B, Hq, D]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    group = Hq // Hkv
    out = np.empty((B, Hq, v_pool.shape[-1]), dtype=np.float64)
    for b in range(B):
        L = int(ctx_lens[b])
        K = gather_sequence(k_pool, block_table[b], L).astype(np.float64)
        V = e4m3_decode(gather_sequence(v_pool, block_table[b], L))
        for h in range(Hq):
            g = h // group
            s = (K[:, g, :] @ q[b, h]) * sm_scale
            e = np.exp(s - s.max())
            out[b, h] = float(v_scale[g]) * ((e / e.sum()) @ V[:, g, :])
    return out


def kv_pool_slots(budget_bytes: int, n_layers: int, n_kv_heads: int, head_dim: int,
                  k_bytes: int, v_bytes: int, page_size: int) -> int:
    """Token slots per layer of a KV pool split evenly over layers, each token
    holding one key and one value per KV head, rounded down to whole pages."""
    per_token = n_kv_heads * head_dim * (k_bytes + v_bytes)
    slots = budget_bytes // n_layers // per_token
    return slots // page_size * page_size
