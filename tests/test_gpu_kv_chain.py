"""K16/V8 cached decoding through the C ABI vs the chain oracle (GPU).

A prefill fills the paged cache of every layer (phi_prefill_fill_k16v8),
then decode steps append one token per sequence and attend over the cache
(phi_decode_step_k16v8).  The oracle is oracle/kv_chain.py.

Gates:
  - pools after the prefill and after the decode steps: keys within the
    binary16 rounding of the oracle's key plus the error that the binary16
    activations feeding the QKV GEMM carry into it (the GPU rounds fp32
    accumulators, the oracle fp64 values, to binary16; the fraction of
    identical keys is printed, not gated, since that activation error is of
    the order of a binary16 step); decoded values within half an E4M3 step of
    the oracle's unquantised value, widened by the same activation error; and
    value codes identical to the oracle's for >= 95 % of elements (a value
    within the activation error of an E4M3 rounding boundary may land on the
    neighbouring code: about 2^-11 / 2^-4 of them, so about 99 % agree);
  - decode-step logits: cosine >= 0.99999 per sequence and argmax agreement
    where the oracle's top-2 gap exceeds 1e-3 (the prefill gate).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import decode, kv_chain, parity, prefill

pytestmark = pytest.mark.gpu
COS_GATE = 0.99999


def _say(*a):
    print(*a, flush=True)


class _Widened:
    """Weights widened to fp64 once (the oracle otherwise widens per call)."""

    def __init__(self, ws, cfg):
        self.embed = ws.embed
        self.final_norm = ws.final_norm
        self.lm_head = prefill.widen(ws.lm_head)
        self._layers = [{k: prefill.widen(v) for k, v in ws.layer(l).items()} for l in range(cfg.n_layers)]

    def layer(self, l):
        return self._layers[l]


def _layout(lens, steps, seed):
    """A shuffled page table: sequence b owns ceil((lens[b] + steps) / 16) pages."""
    need = [-(-(L + steps) // 16) for L in lens]
    n_pages = sum(need) + 3          # a few pages nobody owns
    perm = synth.permutation(seed, "chain.pages", n_pages)
    max_pages = max(need)
    bt = np.full((len(lens), max_pages), perm[-1], dtype=np.int32)   # unused entries: an unowned page
    o = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[o:o + n]
        o += n
    return bt, n_pages


def _check_pools(cache, oracle_caches, raw_vals, bt, n_pages, cfg, v_scale):
    """GPU pools vs the oracle's cache.  Keys: within the binary16 rounding of
    the key plus the error the binary16 activations feeding the QKV GEMM
    carry into it (2^-11 of the row's magnitude).  Values: the decoded code is
    a valid E4M3 rounding of the oracle's unquantised value, within half an
    E4M3 step (2^-4 relative, 2^-10 * scale in the subnormal range) widened
    by the same activation error; codes identical for >= 95 % of elements."""
    for l in range(cfg.n_layers):
        kr, vr = kv_chain.pools_from(oracle_caches, bt, n_pages, l)
        kg = cache.k_pools[l].cpu().numpy()
        vg = cache.v_pools[l].cpu().numpy()
        # unquantised oracle values at the same slots
        vtrue = np.zeros(vr.shape, np.float64)
        for b, c in enumerate(oracle_caches):
            for t in range(c.length()):
                vtrue[bt[b][t // 16], :, t % 16] = raw_vals[b][l][t]
        owned = np.zeros(n_pages, bool)
        for b, c in enumerate(oracle_caches):
            owned[bt[b, : -(-c.length() // 16)]] = True
        ka, kb = kg[owned].astype(np.float64), kr[owned].astype(np.float64)
        krow = np.abs(kb).max(axis=-1, keepdims=True)
        k_err = np.abs(ka - kb) / (2.0 ** -10 * np.abs(kb) + 2.0 ** -11 * krow + 1e-30)
        sc = np.asarray(v_scale[l], np.float64)[None, :, None, None]
        da = decode.e4m3_decode(vg[owned]) * sc
        vt = vtrue[owned]
        vrow = np.abs(vt).max(axis=-1, keepdims=True)
        v_bound = 2.0 ** -4 * np.abs(vt) + 2.0 ** -10 * sc + 2.0 ** -10 * vrow
        v_err = np.abs(da - vt) / v_bound
        same_k, same_v = np.mean(ka == kb), np.mean(vg[owned] == vr[owned])
        _say(f"  layer {l}: keys exact {same_k:.5f} worst {k_err.max():.3f} of bound; "
             f"value codes exact {same_v:.5f} worst {v_err.max():.3f} of bound")
        assert k_err.max() <= 1.0
        assert v_err.max() <= 1.0
        assert same_v >= 0.95


def _chain(phi, cfg, lens, steps, seed):
    from logits_parity_amd.weights import to_device
    ws = synth.WeightSet(cfg)
    wo = _Widened(ws, cfg)
    prompts = [synth.uniform_ints(seed, f"chain.ids{b}", (L + steps,), cfg.vocab) for b, L in enumerate(lens)]
    # per-(layer, head) value scales from the prompts' values (oracle, exact cache)
    raws = [kv_chain.prefill_fill(cfg, wo, p[:L], np.ones((cfg.n_layers, cfg.n_kv_heads), np.float32),
                                  exact=True, logits=False)[2] for p, L in zip(prompts, lens)]
    v_scale = kv_chain.value_scales_from(raws, cfg.n_layers)
    bt, n_pages = _layout(lens, steps, seed)
    m = phi.phi_load_fused(cfg, to_device(ws, cfg.n_layers))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    cache = phi.KVCache.empty(cfg, n_pages, dev(bt), dev(v_scale))
    oc, rv = [], []
    for b, L in enumerate(lens):
        _say(f"  prefill seq {b}: {L} tokens")
        got = m.prefill_fill_k16v8(dev(prompts[b][None, :L].astype(np.int32)), cache.with_table(dev(bt[b:b + 1])))
        ref, c, raw = kv_chain.prefill_fill(cfg, wo, prompts[b][:L], v_scale)
        oc.append(c)
        rv.append([list(r[1]) for r in raw])   # per layer: unquantised values per token
        torch.cuda.synchronize()
        s = parity.summary(got.cpu().numpy()[0], ref)
        assert s["min_cos"] >= COS_GATE and not s["failures"], s
    _check_pools(cache, oc, rv, bt, n_pages, cfg, v_scale)
    max_ctx = max(lens) + steps
    for k in range(steps):
        pos = np.array([L + k for L in lens], np.int32)
        ids = np.array([prompts[b][L + k] for b, L in enumerate(lens)], np.int32)
        got = m.decode_step_k16v8(dev(ids), dev(pos), cache, max_ctx)
        torch.cuda.synchronize()
        got = got.cpu().numpy()
        ref = []
        for b in range(len(lens)):
            logits_b, vals = kv_chain.decode_step(cfg, wo, int(ids[b]), oc[b], v_scale, return_values=True)
            ref.append(logits_b)
            for l in range(cfg.n_layers):   # the step's unquantised value, for the pool check
                rv[b][l].append(vals[l])
        ref = np.stack(ref)
        s = parity.summary(got, ref)
        _say(f"  step {k}: min_cos={s['min_cos']:.9f} gated={s['gated']} agree={s['gated_agree']}")
        assert np.all(np.isfinite(got))
        assert s["min_cos"] >= COS_GATE and not s["failures"], s
    _check_pools(cache, oc, rv, bt, n_pages, cfg, v_scale)
    return m, cache


def test_chain_tiny_gqa128(phi):
    _say("chain tiny gqa128: prompts 20, 33, 16; 3 steps")
    _chain(phi, synth.TINY_GQA128, [20, 33, 16], 3, 51)


def test_chain_phi4_one_layer_full_width(phi):
    _say("chain phi4 1 layer: prompts 37, 64, 20, 50; 2 steps")
    _chain(phi, synth.PHI4_1L, [37, 64, 20, 50], 2, 52)


def test_decode_step_rejects_bad_arguments(phi):
    from logits_parity_amd.weights import to_device
    cfg = synth.TINY_GQA128
    ws = synth.WeightSet(cfg)
    m = phi.phi_load_fused(cfg, to_device(ws, cfg.n_layers))
    bt = torch.arange(4, dtype=torch.int32, device="cuda").reshape(1, 4)
    cache = phi.KVCache.empty(cfg, 4, bt, torch.ones((cfg.n_layers, cfg.n_kv_heads), device="cuda"))
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws_ = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(phi.PhiError) as e:
        m.decode_step_k16v8(ids, ids, cache, 65, workspace=ws_)   # beyond max_pages * 16
    assert e.value.status == 4
    from dataclasses import replace
    cfg96 = replace(synth.TINY, wtype="f16")
    m96 = phi.phi_load_fused(cfg96, to_device(synth.WeightSet(cfg96), cfg96.n_layers))
    c96 = phi.KVCache.empty(cfg96, 4, bt, torch.ones((cfg96.n_layers, cfg96.n_kv_heads), device="cuda"))
    with pytest.raises(phi.PhiError) as e:
        m96.decode_step_k16v8(ids, ids, c96, 8, workspace=ws_)   # head_dim 96: no K16/V8 decode path
    assert e.value.status == 2


def test_decode_step_position_outside_the_table_gives_nan_for_that_sequence_only(phi):
    from logits_parity_amd.weights import to_device
    cfg = synth.TINY_GQA128
    ws = synth.WeightSet(cfg)
    m = phi.phi_load_fused(cfg, to_device(ws, cfg.n_layers))
    bt = torch.arange(8, dtype=torch.int32, device="cuda").reshape(2, 4)
    cache = phi.KVCache.empty(cfg, 8, bt, torch.full((cfg.n_layers, cfg.n_kv_heads), 0.01, device="cuda"))
    ids = torch.tensor([5, 7], dtype=torch.int32, device="cuda")
    pos = torch.tensor([3, 64], dtype=torch.int32, device="cuda")   # 64: past the 4-page table
    got = m.decode_step_k16v8(ids, pos, cache, 64)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert np.all(np.isfinite(got[0])) and np.all(np.isnan(got[1]))
