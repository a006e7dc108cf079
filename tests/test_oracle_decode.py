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


def test_e4m3_encoder_is_nearest_even_and_matches_torch():
    from synth import to_e4m3
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(3000) * np.exp(rng.uniform(-10, 6, 3000))).astype(np.float32)
    ties = (decode.E4M3_TABLE[[0x38, 0x39, 0x01, 0x02, 0x70, 0x71]] +
            decode.E4M3_TABLE[[0x39, 0x3A, 0x02, 0x03, 0x71, 0x72]]) / 2
    x = np.concatenate([x, ties, -ties, [0.0, -0.0, 448.0, 460.0, 1e6, -1e6, 2.0 ** -10, 3 * 2.0 ** -11]]).astype(np.float32)
    ours = decode.e4m3_encode(x)
    # an independent encoder (the input generator's, written from IEEE bit fields)
    assert np.array_equal(ours, to_e4m3(x.astype(np.float64)))
    # torch rounds in-range values the same way (it maps overflow to NaN, so compare in range)
    inr = np.abs(x) < 448
    ref = torch.from_numpy(x[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours[inr], ref)
    # ties resolved to the even code; saturation, infinities and NaN
    assert decode.e4m3_encode(np.array([1.0625]))[0] == 0x38
    assert list(decode.e4m3_encode(np.array([np.inf, -np.inf, 464.0, -1e30, np.nan]))) == [0x7E, 0xFE, 0x7E, 0xFE, 0x7F]


def test_kv_append_then_decode_reads_the_token():
    wl = synth.DecodeWorkload("t", batch=2, ctx=40, n_q_heads=4, n_kv_heads=2, head_dim=128)
    d = synth.decode_inputs(wl, ctx_lens=[33, 20])
    kn = synth.normal(5, "kn", (2, 2, 128), 1.0, np.float16)
    vn = synth.normal(5, "vn", (2, 2, 128), 1.0, np.float16)
    kp, vp = decode.kv_append(d.k_pool, d.v_pool, kn, vn, d.v_scale, d.block_table, np.array([33, 20]))
    for b, p in ((0, 33), (1, 20)):
        page = d.block_table[b, p // 16]
        assert np.array_equal(kp[page, :, p % 16], kn[b])
        dec = decode.e4m3_decode(vp[page, :, p % 16]) * d.v_scale[:, None]
        assert np.all(np.abs(dec - vn[b].astype(np.float64)) <= 0.07 * np.abs(vn[b].astype(np.float64)) + d.v_scale[:, None] * 2.0 ** -9)
    # nothing else changed
    mask = np.ones(kp.shape[:3], bool)
    mask[d.block_table[0, 2], :, 1] = False
    mask[d.block_table[1, 1], :, 4] = False
    assert np.array_equal(kp[mask], d.k_pool[mask]) and np.array_equal(vp[mask], d.v_pool[mask])


def test_kv_append_skips_out_of_range_slots():
    wl = synth.DecodeWorkload("t", batch=3, ctx=40, n_q_heads=2, n_kv_heads=1, head_dim=128)
    d = synth.decode_inputs(wl, ctx_lens=[10, 10, 10])
    kn = synth.normal(6, "kn", (3, 1, 128), 1.0, np.float16)
    bt = d.block_table.copy()
    bt[1, 0] = wl.n_pages           # page id past the pool
    kp, vp = decode.kv_append(d.k_pool, d.v_pool, kn, kn, d.v_scale, bt, np.array([-1, 3, bt.shape[1] * 16]))
    assert np.array_equal(kp, d.k_pool) and np.array_equal(vp, d.v_pool)
