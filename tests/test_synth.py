"""Seeded input generators and storage encodings (CPU only)."""
import numpy as np
import pytest
import torch

import synth


def test_f16_encoder_matches_ieee_rne():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200_000) * np.exp(rng.uniform(-30, 14, 200_000))
    edge = np.array([65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * (1 + 1e-9),
                     2.0 ** -26, 1.5 * 2.0 ** -24, 2.5 * 2.0 ** -24, 0.0, -0.0, np.inf, -np.inf,
                     1e-300, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2.0 ** -14 * (1 - 2.0 ** -12)])
    x = np.concatenate([x, edge, -edge])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = synth.to_f16(x).view(np.uint16)
    assert np.array_equal(got, want)


def test_e4m3_encoder_rne_and_saturation():
    rng = np.random.default_rng(1)
    y = rng.standard_normal(200_000) * np.exp(rng.uniform(-12, 6, 200_000))
    y = y[np.abs(y) < 448]
    got = synth.to_e4m3(y)
    want = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # y is float64; torch rounds from its float32 image.  Only values whose
    # float32 rounding crosses an E4M3 rounding boundary could differ.
    assert np.mean(got != want) < 1e-4
    # saturation and exact ties
    assert synth.to_e4m3(np.array([448.0, 449.0, 1e9, -500.0])).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    # 1.0625 is halfway between 1.0 (0x38) and 1.125 (0x39): ties go to the even code 0x38
    assert synth.to_e4m3(np.array([1.0625, 1.1875])).tolist() == [0x38, 0x3A]
    # every finite code round-trips through its exact value
    from oracle.decode import E4M3_TABLE
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = synth.to_e4m3(E4M3_TABLE[codes])
    # -0.0 encodes as 0x80
    assert np.array_equal(back, codes)


def test_normals_are_counter_based_and_standard():
    a = synth.normal(7, "t", (1001,))
    b = synth.normal(7, "t", (300_001,))
    assert np.array_equal(a, b[:1001])
    assert abs(b.mean()) < 0.01 and abs(b.std() - 1) < 0.01
    c = synth.normal(8, "t", (1001,))
    assert not np.array_equal(a, c)
    h = synth.normal(7, "t", (300_001,), 0.02, np.float16)
    assert np.array_equal(h, synth.to_f16(0.02 * b))


def test_ids_permutation_and_prefix():
    ids = synth.token_ids(synth.MINI, 1, 4096)
    assert ids.dtype == np.int32 and ids.min() >= 0 and ids.max() < synth.MINI.vocab
    assert np.array_equal(synth.token_ids(synth.MINI, 1, 512)[0], ids[0, :512])
    p = synth.permutation(3, "p", 5000)
    assert np.array_equal(np.sort(p), np.arange(5000))
    assert not np.array_equal(p, np.arange(5000))


def test_int8_row_quantizer():
    rng = np.random.default_rng(2)
    w = synth.to_f16(rng.standard_normal((64, 256)) * 0.02)
    w[5] = 0
    q, s = synth.quantize_rows_i8(w)
    wd = w.astype(np.float64)
    sd = s.astype(np.float64)
    assert q.dtype == np.int8 and np.abs(q.astype(int)).max() <= 127
    assert sd[5] == 1.0 and not q[5].any()
    amax = np.abs(wd).max(axis=1)
    nz = amax > 0
    assert np.array_equal(s[nz], synth.to_f16(amax[nz] / 127.0))
    err = np.abs(q.astype(np.float64) * sd[:, None] - wd)
    assert np.all(err <= sd[:, None] / 2 + 1e-12 + np.maximum(0, amax - 127 * sd)[:, None])
    assert np.all(np.abs(q[nz]).max(axis=1) >= 126)


def test_decode_inputs_shapes():
    wl = synth.DecodeWorkload("t", batch=3, ctx=40, n_q_heads=8, n_kv_heads=2, head_dim=128)
    d = synth.decode_inputs(wl)
    assert d.k_pool.shape == (wl.n_pages, 2, 16, 128) and d.v_pool.dtype == np.uint8
    assert d.block_table.shape == (3, 3)
    assert np.array_equal(np.sort(d.block_table.ravel()), np.arange(wl.n_pages))
    assert d.v_scale.dtype == np.float32 and np.all(d.v_scale > 0)
    # the largest |V| per head lands on the largest code
    assert np.all((d.v_pool & 0x7F).reshape(wl.n_pages, 2, -1).max(axis=(0, 2)) == 0x7E)


def test_weight_digest_is_stable():
    a = synth.WeightSet(synth.TINY).digest()
    b = synth.WeightSet(synth.TINY, cache_layers=False).digest()
    assert a == b
    assert synth.WeightSet(synth.TINY, seed=5).digest() != a
