"""Pins of the prefill oracle on the two other dense families of the parity
harness page (section 3): Qwen2.5-0.5B-style (GQA at head_dim 64, a bias on
the Q/K/V projections, tied embeddings) and SmolLM2-360M-style (GQA at
head_dim 64, tied).  The page's oracle for dense families is HuggingFace
transformers (section 2); here transformers' Qwen2 and Llama models run in
fp64 on the same random weights, split out of the fused tensors.  Layers and
vocabulary are cut down so that the CPU check takes seconds; the head
geometry, norms, RoPE base and ties are the families' own.
"""
from dataclasses import replace

import numpy as np
import torch

import synth
from oracle import parity, prefill


class _Scaled:
    """Linear weights (not the embedding or the norm gains) times a factor,
    so attention is peaked and layer outputs matter next to the embedding."""

    def __init__(self, ws, factor):
        self.ws, self.f = ws, factor
        self.embed, self.final_norm = ws.embed, ws.final_norm
        self.lm_head = ws.lm_head

    def layer(self, l):
        w = dict(self.ws.layer(l))
        for k in ("qkv", "o", "gate_up", "down"):
            w[k] = w[k].astype(np.float64) * self.f
        return w


def _hf(cfg, ws, ids, family):
    from transformers import LlamaConfig, LlamaForCausalLM, Qwen2Config, Qwen2ForCausalLM
    common = dict(vocab_size=cfg.vocab, hidden_size=cfg.hidden, intermediate_size=cfg.intermediate,
                  num_hidden_layers=cfg.n_layers, num_attention_heads=cfg.n_heads,
                  num_key_value_heads=cfg.n_kv_heads, max_position_embeddings=4096, rms_norm_eps=cfg.rms_eps,
                  rope_theta=cfg.rope_theta, tie_word_embeddings=cfg.tie_embeddings, pad_token_id=0,
                  bos_token_id=1, eos_token_id=2)
    if family == "qwen2":
        hc = Qwen2Config(**common, use_sliding_window=False)
        Model = Qwen2ForCausalLM
    else:
        hc = LlamaConfig(**common, attention_bias=False, mlp_bias=False)
        Model = LlamaForCausalLM
    hc._attn_implementation = "eager"
    torch.manual_seed(0)
    m = Model(hc).to(torch.float64).eval()
    t = lambda a: torch.from_numpy(prefill.widen(a))
    nq, nk = cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    sd = {"model.embed_tokens.weight": t(ws.embed), "model.norm.weight": t(ws.final_norm)}
    if not cfg.tie_embeddings:
        sd["lm_head.weight"] = t(ws.lm_head)
    for l in range(cfg.n_layers):
        w, p = ws.layer(l), f"model.layers.{l}."
        qkv, gu = t(w["qkv"]), t(w["gate_up"])
        sd.update({p + "self_attn.q_proj.weight": qkv[:nq], p + "self_attn.k_proj.weight": qkv[nq:nq + nk],
                   p + "self_attn.v_proj.weight": qkv[nq + nk:], p + "self_attn.o_proj.weight": t(w["o"]),
                   p + "mlp.gate_proj.weight": gu[:cfg.intermediate], p + "mlp.up_proj.weight": gu[cfg.intermediate:],
                   p + "mlp.down_proj.weight": t(w["down"]), p + "input_layernorm.weight": t(w["ln1"]),
                   p + "post_attention_layernorm.weight": t(w["ln2"])})
        if cfg.qkv_bias:
            b = t(w["qkv_bias"])
            sd.update({p + "self_attn.q_proj.bias": b[:nq], p + "self_attn.k_proj.bias": b[nq:nq + nk],
                       p + "self_attn.v_proj.bias": b[nq + nk:]})
    missing, unexpected = m.load_state_dict(sd, strict=False)
    missing = [k for k in missing if k != "lm_head.weight"]   # tied: it is the embedding
    assert not missing and not unexpected, (missing, unexpected)
    if cfg.tie_embeddings:
        assert m.lm_head.weight.data_ptr() == m.model.embed_tokens.weight.data_ptr()
    with torch.no_grad():
        return m(torch.from_numpy(np.asarray(ids, dtype=np.int64))).logits.numpy()


def _pin(cfg, family, factor=3.0):
    ws = _Scaled(synth.WeightSet(cfg), factor)
    ids = synth.token_ids(cfg, 2, 20)
    ours = prefill.prefill_logits(cfg, ws, ids)
    ref = _hf(cfg, ws, ids, family)
    err = np.abs(ours - ref).max() / np.sqrt(np.mean(ref ** 2))
    assert err < 1e-4, err
    s = parity.summary(ours.reshape(-1, cfg.vocab), ref.reshape(-1, cfg.vocab))
    assert s["min_cos"] > 1 - 1e-8
    return ours, ref, ws, ids


def test_qwen2_style_matches_transformers():
    cfg = replace(synth.QWEN25_05B, n_layers=2, vocab=2048, norm_gain="ones")
    ours, ref, ws, ids = _pin(cfg, "qwen2")
    # the bias matters: dropping it breaks the pin
    class NoBias(_Scaled):
        def layer(self, l):
            w = dict(super().layer(l))
            w.pop("qkv_bias")
            return w
    nb = NoBias(synth.WeightSet(cfg), 3.0)
    bad = prefill.prefill_logits(cfg, nb, ids)
    assert np.abs(bad - ref).max() / np.sqrt(np.mean(ref ** 2)) > 1e-3


def test_smollm2_style_matches_transformers():
    cfg = replace(synth.SMOLLM2_360M, n_layers=2, vocab=2048, norm_gain="ones")
    _pin(cfg, "llama")


def test_tied_weight_sets_share_the_embedding():
    ws = synth.WeightSet(replace(synth.SMOLLM2_360M, n_layers=1, vocab=256))
    assert ws.lm_head is ws.embed
