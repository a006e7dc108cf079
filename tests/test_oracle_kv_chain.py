"""Pins of the K16/V8 cached decode chain oracle (CPU only).

- With an exact cache (fp64 keys and values), a decode step is the prefill of
  the longer sequence evaluated at its last position: the chain's bookkeeping
  (positions, append-before-attend, GQA grouping, residual stream) is pinned
  against the prefill oracle, itself pinned against transformers' Phi-3.
- The compressed cache holds binary16 keys and the E4M3 codes that the cache
  write (oracle/decode.kv_append, pinned against torch float8_e4m3fn) makes
  of the same values; the quantised decode reads them through the decode
  attention oracle (pinned against torch SDPA).
- Planted mistakes (RoPE at the wrong position, attend before append) fail.
"""
from dataclasses import replace

import numpy as np

import synth
from oracle import decode, kv_chain, prefill


def _model(cfg):
    return synth.WeightSet(cfg)


class _Scaled:
    """A WeightSet with every linear weight multiplied by a factor, so that
    attention is peaked and positions matter (N(0, 0.02) weights give nearly
    uniform attention, which hides position mistakes)."""

    def __init__(self, ws, factor):
        self.ws, self.f = ws, factor
        self.embed, self.final_norm, self.lm_head = ws.embed, ws.final_norm, ws.lm_head

    def layer(self, l):
        w = dict(self.ws.layer(l))
        for k in ("qkv", "o", "gate_up", "down"):
            w[k] = w[k].astype(np.float64) * self.f
        return w


def _scales(cfg, ws, ids_list):
    raws = [kv_chain.prefill_fill(cfg, ws, ids, np.ones((cfg.n_layers, cfg.n_kv_heads), np.float32), exact=True)[2]
            for ids in ids_list]
    return kv_chain.value_scales_from(raws, cfg.n_layers)


def _rel(a, b):
    return np.abs(a - b).max() / np.abs(b).max()


def test_exact_decode_steps_equal_the_longer_prefill():
    for cfg in (synth.TINY_GQA128, replace(synth.TINY, wtype="f16")):
        ws = _Scaled(_model(cfg), 6.0)
        ids = synth.token_ids(cfg, 1, 12)[0]
        scale = np.ones((cfg.n_layers, cfg.n_kv_heads), np.float32)
        logits, cache, _ = kv_chain.prefill_fill(cfg, ws, ids[:9], scale, exact=True)
        full = prefill.prefill_logits(cfg, ws, ids[None])[0]
        assert _rel(logits, full[:9]) < 1e-12
        for p in range(9, 12):
            step = kv_chain.decode_step(cfg, ws, int(ids[p]), cache, scale, exact=True)
            assert _rel(step, full[p]) < 1e-10, (cfg.name, p)
        assert cache.length() == 12


def test_compressed_cache_holds_f16_keys_and_append_codes():
    cfg = synth.TINY_GQA128
    ws = _model(cfg)
    ids = synth.token_ids(cfg, 1, 20)[0]
    scale = _scales(cfg, ws, [ids])
    _, cache, raw = kv_chain.prefill_fill(cfg, ws, ids, scale)
    for l in range(cfg.n_layers):
        k, v = raw[l]
        for t in (0, 7, 19):
            key, _, codes = cache.layers[l][t]
            assert np.array_equal(key, k[t].astype(np.float16).astype(np.float64))
            # the cache write of the same token (its own oracle) gives the same bytes
            kp = np.zeros((1, cfg.n_kv_heads, 16, cfg.head_dim), np.float16)
            vp = np.zeros((1, cfg.n_kv_heads, 16, cfg.head_dim), np.uint8)
            _, vp2 = decode.kv_append(kp, vp, k[t][None].astype(np.float16), v[t][None].astype(np.float16),
                                      scale[l], np.zeros((1, 1), np.int32), np.array([0]))
            assert np.array_equal(codes, vp2[0, :, 0])
    # the scales put each (layer, head)'s largest value at the E4M3 maximum
    for l in range(cfg.n_layers):
        amax = np.abs(raw[l][1]).max(axis=(0, 2))
        assert np.allclose(scale[l], (amax / 448.0).astype(np.float32), rtol=1e-6)
        big = np.abs(cache_codes := np.stack([e[2] for e in cache.layers[l]])) & 0x7F
        assert big.max() == 0x7E   # 448 is reached, never exceeded


def test_quantised_steps_stay_close_to_exact():
    cfg = synth.TINY_GQA128
    ws = _model(cfg)
    ids = synth.token_ids(cfg, 1, 24)[0]
    scale = _scales(cfg, ws, [ids])
    _, cq, _ = kv_chain.prefill_fill(cfg, ws, ids[:20], scale)
    _, ce, _ = kv_chain.prefill_fill(cfg, ws, ids[:20], scale, exact=True)
    for p in range(20, 24):
        a = kv_chain.decode_step(cfg, ws, int(ids[p]), cq, scale)
        b = kv_chain.decode_step(cfg, ws, int(ids[p]), ce, scale, exact=True)
        cos = a @ b / np.linalg.norm(a) / np.linalg.norm(b)
        assert cos > 0.999, cos
        assert 0 < _rel(a, b) < 0.1       # quantisation is visible but small


def test_planted_mistakes_fail_the_prefill_pin():
    cfg = synth.TINY_GQA128
    ws = _Scaled(_model(cfg), 6.0)
    ids = synth.token_ids(cfg, 1, 10)[0]
    scale = np.ones((cfg.n_layers, cfg.n_kv_heads), np.float32)
    full = prefill.prefill_logits(cfg, ws, ids[None])[0]

    orig_qkv = kv_chain._qkv
    try:
        # RoPE at position p - 1 for the new token
        kv_chain._qkv = lambda x, lw, c, pos: orig_qkv(x, lw, c, np.asarray(pos) - (1 if len(pos) == 1 else 0))
        _, cache, _ = kv_chain.prefill_fill(cfg, ws, ids[:9], scale, exact=True)
        bad = kv_chain.decode_step(cfg, ws, int(ids[9]), cache, scale, exact=True)
        assert _rel(bad, full[9]) > 1e-6   # the pin holds to 1e-10
    finally:
        kv_chain._qkv = orig_qkv

    orig_store = kv_chain._store
    try:
        # attend before the new token is in the cache: store it after reading
        calls = []

        def late_store(layer, k, v, sc, exact):
            if k.shape[0] == 1 and not calls:
                calls.append(1)
                return
            orig_store(layer, k, v, sc, exact)
        _, cache, _ = kv_chain.prefill_fill(cfg, ws, ids[:9], scale, exact=True)
        kv_chain._store = late_store
        try:
            bad = kv_chain.decode_step(cfg, ws, int(ids[9]), cache, scale, exact=True)
            assert _rel(bad, full[9]) > 1e-6   # the pin holds to 1e-10
        except ValueError:
            pass   # the stacked caches no longer agree in length: also a failure
    finally:
        kv_chain._store = orig_store
