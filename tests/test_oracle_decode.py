"""Pins of the decode-attention oracle and the KV-pool sizing (CPU only)."""
import json
import os

import numpy as np
import torch

import synth
from oracle import decode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_table_matches_torch_and_ocp_points():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = decode.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    assert np.array_equal(ours[~nan], ref[~nan])
    with open(os.path.join(GOLDEN, "e4m3_ocp_points.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            c, v = line.split()
            got = decode.e4m3_value(int(c, 16))
            if v == "nan":
                assert np.isnan(got)
            else:
                assert got == float(v) and np.signbit(got) == v.startswith("-"), (c, v, got)


def _dense_reference(d):
    """torch fp64 SDPA over the cache gathered into logical order."""
    B, Hq, D = d.q.shape
    Hkv = d.k_pool.shape[1]
    outs = []
    for b in range(B):
        L = int(d.ctx_lens[b])
        K = decode.gather_sequence(d.k_pool, d.block_table[b], L).astype(np.float64)
        V = torch.from_numpy(d.v_pool).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        V = decode.gather_sequence(V, d.block_table[b], L) * d.v_scale.astype(np.float64)[None, :, None]
        tq = torch.from_numpy(d.q[b].astype(np.float64))[:, None, :]              # [Hq, 1, D]
        tk = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)  # [Hq, L, D]
        tv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        outs.append(torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[:, 0].numpy())
    return np.stack(outs)


def test_decode_matches_torch_sdpa_on_gathered_cache():
    wl = synth.DecodeWorkload("t", batch=3, ctx=70, n_q_heads=8, n_kv_heads=2, head_dim=128)
    d = synth.decode_inputs(wl, ctx_lens=[70, 33, 1])
    ours = decode.decode_attention(d.q, d.k_pool, d.v_pool, d.v_scale, d.block_table, d.ctx_lens,
                                   1 / np.sqrt(128))
    ref = _dense_reference(d)
    assert np.abs(ours - ref).max() < 1e-12


def test_decode_one_token_is_the_scaled_value():
    wl = synth.DecodeWorkload("t", batch=2, ctx=16, n_q_heads=4, n_kv_heads=2, head_dim=128)
    d = synth.decode_inputs(wl, ctx_lens=[1, 1])
    out = decode.decode_attention(d.q, d.k_pool, d.v_pool, d.v_scale, d.block_table, d.ctx_lens, 0.1)
    for b in range(2):
        page = d.block_table[b, 0]
        for h in range(4):
            g = h // 2
            want = float(d.v_scale[g]) * decode.e4m3_decode(d.v_pool[page, g, 0])
            assert np.array_equal(out[b, h], want)


def test_decode_all_ones_values_give_ones():
    # every V byte 0x38 (1.0) with scale 1: softmax rows sum to one
    wl = synth.DecodeWorkload("t", batch=2, ctx=50, n_q_heads=4, n_kv_heads=1, head_dim=128)
    d = synth.decode_inputs(wl)
    d.v_pool[:] = 0x38
    out = decode.decode_attention(d.q, d.k_pool, d.v_pool, np.ones(1, np.float32), d.block_table,
                                  d.ctx_lens, 0.5)
    assert np.abs(out - 1).max() < 1e-14


def test_kv_pool_slots_match_the_page():
    with open(os.path.join(GOLDEN, "kv_pool_phi4.json")) as f:
        g = json.load(f)
    args = (g["budget_bytes"], g["n_layers"], g["n_kv_heads"], g["head_dim"])
    assert decode.kv_pool_slots(*args, 2, 1, g["page_size"]) == g["k16v8_slots"]
    assert decode.kv_pool_slots(*args, 2, 2, g["page_size"]) == g["fp16_slots"]
    # only the 16-token page reproduces both printed numbers
    for page in (8, 32, 64):
        assert (decode.kv_pool_slots(*args, 2, 1, page), decode.kv_pool_slots(*args, 2, 2, page)) != \
            (g["k16v8_slots"], g["fp16_slots"])
