"""K16/V8 paged decode attention vs the fp64 oracle (GPU).

Gate: for every (sequence, query head), ||o - o_ref|| / ||o_ref|| <= 2e-3.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import decode

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _gpu(phi, d, max_ctx=None, sm_scale=None):
    D = d.q.shape[-1]
    sm = 1 / np.sqrt(D) if sm_scale is None else sm_scale
    mc = int(d.ctx_lens.max()) if max_ctx is None else max_ctx
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = phi.attn_decode_k16v8(t(d.q), t(d.k_pool), t(d.v_pool), t(d.v_scale), t(d.block_table),
                                t(d.ctx_lens), mc, sm)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _ref(d, sm_scale=None):
    D = d.q.shape[-1]
    sm = 1 / np.sqrt(D) if sm_scale is None else sm_scale
    return decode.decode_attention(d.q, d.k_pool, d.v_pool, d.v_scale, d.block_table, d.ctx_lens, sm)


def _rel(got, ref):
    return np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)


@pytest.mark.parametrize("name", ["decode_k16v8_32x1024", "decode_k16v8_16x8192"])
def test_decode_full_shapes(phi, name):
    wl = synth.DECODE_WORKLOADS[name]
    _say(name)
    d = synth.decode_inputs(wl)
    got = _gpu(phi, d)
    ref = _ref(d)
    rel = _rel(got, ref)
    _say(f"  max rel L2 = {rel.max():.2e}")
    assert rel.max() <= 2e-3


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_ragged_contexts(phi, G):
    wl = synth.DecodeWorkload("t", batch=6, ctx=300, n_q_heads=2 * G, n_kv_heads=2)
    lens = [1, 15, 16, 17, 255, 300]
    _say(f"decode ragged G={G}")
    d = synth.decode_inputs(wl, ctx_lens=lens)
    got = _gpu(phi, d)
    rel = _rel(got, _ref(d))
    assert rel.max() <= 2e-3, rel.max()


# Launches with at least 320 (sequence, KV head, split) workgroups use
# 64-page splits: one split per sequence (normalised in the split kernel, no
# merge) at max_ctx <= 1024, two splits (merged, the second empty for the
# shorter sequences) above.
@pytest.mark.parametrize("max_ctx", [1000, 1500])
def test_decode_long_splits_ragged(phi, max_ctx):
    wl = synth.DecodeWorkload("t", batch=40, ctx=max_ctx, n_q_heads=16, n_kv_heads=8)
    lens = [max_ctx - 37 * i for i in range(40)]
    lens = [max(1, x) for x in lens]
    _say(f"decode long splits max_ctx={max_ctx}")
    d = synth.decode_inputs(wl, ctx_lens=lens)
    got = _gpu(phi, d, max_ctx=max_ctx)
    rel = _rel(got, _ref(d))
    assert rel.max() <= 2e-3, rel.max()


# 16 sequences x 8 KV heads (128 workgroups) at max_ctx 4000 (250 pages)
# would take four 64-page splits and the merge; they run as one split per
# sequence on 8-wave workgroups instead.  Ragged lengths leave some waves
# with no pages at all (a 1-token sequence has one page, for wave 0).
@pytest.mark.parametrize("G", [1, 4, 8])
def test_decode_single_split_eight_waves_ragged(phi, G):
    wl = synth.DecodeWorkload("t", batch=16, ctx=4000, n_q_heads=8 * G, n_kv_heads=8)
    lens = [1, 16, 17, 100, 112, 113, 128, 129, 1000, 2047, 2048, 2049, 3333, 3999, 4000, 4000]
    _say(f"decode one split, 8 waves, G={G}")
    d = synth.decode_inputs(wl, ctx_lens=lens)
    got = _gpu(phi, d, max_ctx=4000)
    rel = _rel(got, _ref(d))
    _say(f"  max rel L2 = {rel.max():.2e}")
    assert rel.max() <= 2e-3, rel.max()


def test_decode_page_permutation_is_invisible(phi):
    wl = synth.DecodeWorkload("t", batch=4, ctx=500, n_q_heads=8, n_kv_heads=2)
    d = synth.decode_inputs(wl)
    a = _gpu(phi, d)
    perm = synth.permutation(99, "repage", wl.n_pages)
    inv = np.argsort(perm)
    d.k_pool, d.v_pool = d.k_pool[perm].copy(), d.v_pool[perm].copy()
    d.block_table = inv[d.block_table].astype(np.int32)
    b = _gpu(phi, d)
    assert np.array_equal(a, b)


def test_decode_unit_values_sum_to_one(phi):
    wl = synth.DecodeWorkload("t", batch=3, ctx=200, n_q_heads=8, n_kv_heads=2)
    d = synth.decode_inputs(wl)
    d.v_pool[:] = 0x38
    d.v_scale[:] = 1.0
    got = _gpu(phi, d)
    assert np.abs(got - 1).max() <= 1e-3


def test_decode_bad_inputs_make_only_that_sequence_nan(phi):
    wl = synth.DecodeWorkload("t", batch=3, ctx=64, n_q_heads=8, n_kv_heads=2)
    d = synth.decode_inputs(wl)
    d.block_table[1, 2] = wl.n_pages + 7
    d.ctx_lens[2] = 0
    got = _gpu(phi, d, max_ctx=64)
    assert np.all(np.isfinite(got[0]))
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2]))
    ref = _ref(d.__class__(d.wl, d.q[:1], d.k_pool, d.v_pool, d.v_scale, d.block_table[:1], d.ctx_lens[:1]))
    assert _rel(got[:1], ref).max() <= 2e-3


def test_decode_deterministic(phi):
    wl = synth.DECODE_WORKLOADS["decode_k16v8_32x1024"]
    d = synth.decode_inputs(wl)
    assert np.array_equal(_gpu(phi, d), _gpu(phi, d))
