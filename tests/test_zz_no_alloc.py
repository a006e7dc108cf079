"""attn_decode_k16v8_noalloc through the C ABI against attn_decode_k16v8 (GPU).

The allocation-free variant keeps its split partials in the library's fixed
scratch array instead of a caller workspace; it runs the same plan and
kernels, so its output must equal the workspace entry point's bit for bit,
and both stay within the decode gate of the fp64 oracle.  Two calls in a row,
the second smaller, check that a call does not depend on what the previous
one left in the shared array.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import decode

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _case(phi, wl, lens, max_ctx):
    d = synth.decode_inputs(wl, ctx_lens=lens)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    q, kp, vp, vs, bt, cl = t(d.q), t(d.k_pool), t(d.v_pool), t(d.v_scale), t(d.block_table), t(d.ctx_lens)
    sm = 1 / np.sqrt(wl.head_dim)
    need = phi.attn_decode_k16v8_workspace_bytes(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, max_ctx)
    _say(f"  {wl.name}: batch {wl.batch}, heads {wl.n_q_heads}/{wl.n_kv_heads}, lens {list(lens)}, "
         f"partials {need} bytes")
    ref_ws = phi.attn_decode_k16v8(q, kp, vp, vs, bt, cl, max_ctx, sm)
    got = phi.attn_decode_k16v8_noalloc(q, kp, vp, vs, bt, cl, max_ctx, sm)
    torch.cuda.synchronize()
    a, b = got.cpu().numpy(), ref_ws.cpu().numpy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    ref = decode.decode_attention(d.q, d.k_pool, d.v_pool, d.v_scale, d.block_table, d.ctx_lens, sm)
    out = a.astype(np.float64)
    rel = np.linalg.norm(out - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    _say(f"    bitwise equal to the workspace call; max rel L2 vs oracle {rel.max():.2e}")
    assert rel.max() <= 2e-3
    return need


def test_noalloc_matches_workspace_entry_point_twice(phi):
    # first call: a 12-split plan (partials in the scratch array), ragged lengths
    wl1 = synth.DecodeWorkload("noalloc_a", batch=3, ctx=3000)
    n1 = _case(phi, wl1, [3000, 1700, 2917], 3000)
    # second call, smaller: another GQA group and fewer partials
    wl2 = synth.DecodeWorkload("noalloc_b", batch=2, ctx=700, n_q_heads=8, n_kv_heads=2)
    n2 = _case(phi, wl2, [700, 333], 700)
    assert n2 < n1 <= (16 << 20)
