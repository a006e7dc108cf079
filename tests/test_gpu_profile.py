"""Per-stage device timing of phi_prefill_logits (GPU).

With profiling on, a stage of one kernel times that kernel's own dispatch
(events attached to it); the QKV stage of a prefill that also fills a KV cache
is timed by an event pair around its two launches.  Checked: launch counts
per stage, positive times, logits unchanged by profiling, a read clears the
record, and the limit of 16 recorded forwards between reads (refused on the
host before anything is enqueued).
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _ids(cfg, batch, seq):
    return torch.from_numpy(np.ascontiguousarray(synth.token_ids(cfg, batch, seq), dtype=np.int32)).cuda()


def _expected_counts(cfg, forwards):
    L = cfg.n_layers
    per = {"embed": 1, "qkv": L, "attn": L, "o_proj": L, "norm": 2 * L, "gate_up": L, "down": L, "lm_head": 1}
    return {k: forwards * v for k, v in per.items()}


def test_profile_counts_times_and_unchanged_results(phi):
    from logits_parity_amd.weights import to_device
    cfg = replace(synth.TINY, wtype="f16")
    m = phi.phi_load_fused(cfg, to_device(synth.WeightSet(cfg), cfg.n_layers))
    ids = _ids(cfg, 2, 40)
    plain = m.prefill_logits(ids).cpu().numpy()
    n = 3
    m.profile_enable(True)
    outs = [m.prefill_logits(ids).cpu().numpy() for _ in range(n)]
    prof = m.profile_read()
    m.profile_enable(False)
    _say("  " + " ".join(f"{k}={v[0]:.4f}ms/{v[1]}" for k, v in prof.items()))
    for o in outs:
        assert np.array_equal(o, plain)
    for k, c in _expected_counts(cfg, n).items():
        ms, cnt = prof[k]
        assert cnt == c, (k, cnt, c)
        assert 0.0 < ms < 1e4, (k, ms)
    assert all(v == (0.0, 0) for v in m.profile_read().values())


def test_profile_record_limit(phi):
    from logits_parity_amd.weights import to_device
    cfg = replace(synth.TINY, wtype="f16")
    m = phi.phi_load_fused(cfg, to_device(synth.WeightSet(cfg), cfg.n_layers))
    ids = _ids(cfg, 1, 8)
    m.profile_enable(True)
    for _ in range(16):
        m.prefill_logits(ids)
    with pytest.raises(phi.PhiError) as e:
        m.prefill_logits(ids)
    assert e.value.status == 4  # PHI_E_RANGE
    prof = m.profile_read()
    assert prof["lm_head"][1] == 16 and prof["qkv"][1] == 16 * cfg.n_layers
    m.prefill_logits(ids)  # the read freed the record
    assert m.profile_read()["embed"][1] == 1
    m.profile_enable(False)


def test_profile_prefill_with_cache_fill(phi):
    from logits_parity_amd.weights import to_device
    cfg = synth.TINY_GQA128
    m = phi.phi_load_fused(cfg, to_device(synth.WeightSet(cfg), cfg.n_layers))
    seq = 20
    ids = _ids(cfg, 1, seq)
    n_pages = 4
    bt = torch.tensor([[2, 0]], dtype=torch.int32, device="cuda")
    v_scale = torch.ones((cfg.n_layers, cfg.n_kv_heads), dtype=torch.float32, device="cuda")
    cache = phi.KVCache.empty(cfg, n_pages, bt, v_scale)
    plain = m.prefill_fill_k16v8(ids, cache).cpu().numpy()
    k0 = [k.clone() for k in cache.k_pools]
    m.profile_enable(True)
    got = m.prefill_fill_k16v8(ids, cache).cpu().numpy()
    prof = m.profile_read()
    m.profile_enable(False)
    _say("  " + " ".join(f"{k}={v[0]:.4f}ms/{v[1]}" for k, v in prof.items()))
    assert np.array_equal(got, plain)
    assert all(torch.equal(a, b) for a, b in zip(k0, cache.k_pools))
    for k, c in _expected_counts(cfg, 1).items():
        ms, cnt = prof[k]
        assert cnt == c, (k, cnt, c)
        assert ms > 0.0, (k, ms)
