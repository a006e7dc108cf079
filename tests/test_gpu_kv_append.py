"""K16/V8 cache write vs the oracle (GPU).

Gate: bit-exact pools (integer/byte work), then the decode step that reads the
appended token within the decode gate (relative L2 <= 2e-3 per head).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import decode

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _append_gpu(phi, d, k_new, v_new, positions, v_scale=None, block_table=None):
    kp, vp = _t(d.k_pool), _t(d.v_pool)
    vs = d.v_scale if v_scale is None else v_scale
    bt = d.block_table if block_table is None else block_table
    phi.kv_append_k16v8(_t(k_new), _t(v_new), _t(vs), _t(bt), _t(np.asarray(positions, np.int32)), kp, vp)
    torch.cuda.synchronize()
    return kp.cpu().numpy(), vp.cpu().numpy()


def _wide_values(seed, shape, scales):
    """binary16 values [B, Hkv, D] whose quotients by the per-head scales span
    E4M3's subnormals, normals and the saturating range; a quarter of them are
    a tie between two neighbouring E4M3 values times the head's scale (an
    exact tie of the quotient when the scale is a power of two)."""
    n = int(np.prod(shape))
    mag = synth.normal(seed, "append.mag", (n,), 1.0, np.float64)
    expo = synth.uniform_ints(seed, "append.exp", (n,), 26).astype(np.float64) - 16.0
    v = mag * np.exp2(expo)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    tab = np.sort(decode.E4M3_TABLE[finite])
    mids = (tab[1:] + tab[:-1]) / 2                     # every tie between neighbours
    pick = synth.uniform_ints(seed, "append.tie", (n,), len(mids))
    take = synth.uniform_ints(seed, "append.use", (n,), 4) == 0
    head_scale = np.broadcast_to(np.asarray(scales, np.float64)[None, :, None], shape).reshape(-1)
    v = np.where(take, mids[pick] * head_scale, v)
    return np.clip(v, -60000, 60000).astype(np.float16).reshape(shape)


def _power_of_two_scales(hkv):
    return np.exp2(-(np.arange(hkv) % 4)).astype(np.float32)     # 1, 1/2, 1/4, 1/8: ties stay ties


def test_append_full_shape_bit_exact_then_decode(phi):
    wl = synth.DECODE_WORKLOADS["decode_k16v8_32x1024"]
    lens = (wl.ctx - 1 - (np.arange(wl.batch) % 17)).astype(np.int32)   # slots 15 .. 0 and a page start
    _say("append", wl.name, "positions", int(lens.min()), "..", int(lens.max()))
    d = synth.decode_inputs(wl, ctx_lens=lens)
    k_new = synth.normal(11, "append.k", (wl.batch, wl.n_kv_heads, wl.head_dim), 1.0, np.float16)
    d.v_scale = _power_of_two_scales(wl.n_kv_heads)
    v_new = _wide_values(11, (wl.batch, wl.n_kv_heads, wl.head_dim), d.v_scale)
    kp, vp = _append_gpu(phi, d, k_new, v_new, lens)
    rk, rv = decode.kv_append(d.k_pool, d.v_pool, k_new, v_new, d.v_scale, d.block_table, lens)
    assert np.array_equal(kp.view(np.uint16), rk.view(np.uint16))
    bad = np.flatnonzero(vp.reshape(-1) != rv.reshape(-1))
    assert bad.size == 0, (bad.size, vp.reshape(-1)[bad[:8]], rv.reshape(-1)[bad[:8]])

    # the decode step now reads one more token per sequence
    d.k_pool, d.v_pool, d.ctx_lens = kp, vp, lens + 1
    t = lambda a: _t(a)
    out = phi.attn_decode_k16v8(t(d.q), t(d.k_pool), t(d.v_pool), t(d.v_scale), t(d.block_table),
                                t(d.ctx_lens), int(d.ctx_lens.max()), 1 / np.sqrt(128))
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = decode.decode_attention(d.q, rk, rv, d.v_scale, d.block_table, d.ctx_lens, 1 / np.sqrt(128))
    rel = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    _say(f"  decode after append: max rel L2 = {rel.max():.2e}")
    assert rel.max() <= 2e-3


def test_append_data_scales_and_special_values(phi):
    wl = synth.DecodeWorkload("t", batch=5, ctx=64, n_q_heads=8, n_kv_heads=3)
    d = synth.decode_inputs(wl, ctx_lens=[0, 15, 16, 31, 63])
    k_new = synth.normal(12, "append.k", (5, 3, 128), 1.0, np.float16)
    v_scale = np.array([0.37, 3.1e-3, 11.0], np.float32)            # quotients round in fp32 first
    v_new = _wide_values(12, (5, 3, 128), v_scale)
    v_new[0, 0, :6] = [np.inf, -np.inf, np.nan, 464.0, -0.0, 0.0]
    pos = np.array([0, 15, 16, 31, 63], np.int32)
    kp, vp = _append_gpu(phi, d, k_new, v_new, pos, v_scale=v_scale)
    rk, rv = decode.kv_append(d.k_pool, d.v_pool, k_new, v_new, v_scale, d.block_table, pos)
    assert np.array_equal(kp.view(np.uint16), rk.view(np.uint16))
    assert np.array_equal(vp, rv)
    page = d.block_table[0, 0]
    assert list(vp[page, 0, 0, :6]) == [0x7E, 0xFE, 0x7F, 0x7E, 0x80, 0x00]


def test_append_out_of_range_slots_write_nothing(phi):
    wl = synth.DecodeWorkload("t", batch=4, ctx=32, n_q_heads=2, n_kv_heads=1)
    d = synth.decode_inputs(wl, ctx_lens=[1, 1, 1, 1])
    bt = d.block_table.copy()
    bt[1, 0] = wl.n_pages          # page id past the pool
    bt[2, 1] = -1
    pos = np.array([-1, 3, 20, 32], np.int32)
    k_new = synth.normal(13, "append.k", (4, 1, 128), 1.0, np.float16)
    kp, vp = _append_gpu(phi, d, k_new, k_new, pos, block_table=bt)
    assert np.array_equal(kp.view(np.uint16), d.k_pool.view(np.uint16))
    assert np.array_equal(vp, d.v_pool)


def test_append_empty_batch_is_a_no_op(phi):
    wl = synth.DecodeWorkload("t", batch=1, ctx=16, n_q_heads=2, n_kv_heads=1)
    d = synth.decode_inputs(wl)
    kp, vp = _t(d.k_pool), _t(d.v_pool)
    e = torch.empty((0, 1, 128), dtype=torch.float16, device="cuda")
    phi.kv_append_k16v8(e, e, _t(d.v_scale), _t(d.block_table[:0]), torch.empty(0, dtype=torch.int32,
                        device="cuda"), kp, vp)
    torch.cuda.synchronize()
    assert np.array_equal(kp.cpu().numpy().view(np.uint16), d.k_pool.view(np.uint16))
