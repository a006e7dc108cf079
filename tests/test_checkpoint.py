"""The checkpoint loader on checkpoints written by transformers'
save_pretrained (CPU only: file parsing and the fused-layout mapping).

- Phi-3: config fields, and the fused qkv_proj / gate_up_proj tensors used as
  stored, bit-identical to the synthetic weights.
- Qwen2 (QKV bias, tied embeddings) and Llama: q/k/v and gate/up stacked in
  the row order Q, K, V and gate, up (the layout the Phi-3 page's fused
  tensors use and the oracle's HF pins confirm); the tied lm_head is the
  embedding tensor itself.
- bfloat16 files cast to binary16; rejected configs.
"""
import json
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from hf_checkpoints import save_checkpoint
from logits_parity_amd.checkpoint import load_checkpoint, read_config


def _eq16(t, a):
    return np.array_equal(t.cpu().numpy().view(np.uint16), np.asarray(a, dtype=np.float16).view(np.uint16))


def test_phi3_fused_tensors_load_as_stored(tmp_path):
    cfg = synth.TINY
    ws = synth.WeightSet(cfg)
    path = save_checkpoint(cfg, ws, "phi3", tmp_path / "phi3")
    c = read_config(path)
    assert (c.family, c.n_layers, c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.intermediate, c.vocab) == \
        ("phi3", cfg.n_layers, cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate, cfg.vocab)
    assert c.rms_eps == cfg.rms_eps and c.rope_theta == cfg.rope_theta and c.max_pos == 4096
    assert not c.qkv_bias and not c.tie_embeddings and c.sliding_window is None
    c2, w = load_checkpoint(path, "cpu")
    assert c2 == c
    for l in range(cfg.n_layers):
        lw = ws.layer(l)
        for k in ("ln1", "ln2", "qkv", "o", "gate_up", "down"):
            assert w["layers"][l][k].dtype == torch.float16 and _eq16(w["layers"][l][k], lw[k]), (l, k)
        assert "qkv_bias" not in w["layers"][l]
    assert _eq16(w["embed"], ws.embed) and _eq16(w["lm_head"], ws.lm_head) and _eq16(w["final_norm"], ws.final_norm)


@pytest.mark.parametrize("family", ["qwen2", "llama"])
def test_separate_projections_are_stacked_into_the_fused_layout(tmp_path, family):
    base = synth.QWEN25_05B if family == "qwen2" else synth.SMOLLM2_360M
    cfg = replace(base, n_layers=2, vocab=512)
    ws = synth.WeightSet(cfg)
    path = save_checkpoint(cfg, ws, family, tmp_path / family)
    c, w = load_checkpoint(path, "cpu")
    assert c.family == family and c.qkv_bias == cfg.qkv_bias and c.tie_embeddings == cfg.tie_embeddings
    assert c.head_dim == cfg.head_dim and c.n_kv_heads == cfg.n_kv_heads
    for l in range(cfg.n_layers):
        lw = ws.layer(l)
        assert _eq16(w["layers"][l]["qkv"], lw["qkv"]) and _eq16(w["layers"][l]["gate_up"], lw["gate_up"])
        if cfg.qkv_bias:
            assert _eq16(w["layers"][l]["qkv_bias"], lw["qkv_bias"])
    assert w["lm_head"] is w["embed"]            # tied: one tensor serves both


def test_bfloat16_files_are_cast_to_binary16(tmp_path):
    cfg = replace(synth.TINY, n_layers=1)
    ws = synth.WeightSet(cfg)
    path = save_checkpoint(cfg, ws, "phi3", tmp_path / "bf16", dtype=torch.bfloat16)
    _, w = load_checkpoint(path, "cpu")
    want = torch.from_numpy(np.asarray(ws.layer(0)["qkv"], np.float32)).to(torch.bfloat16).to(torch.float16)
    assert w["layers"][0]["qkv"].dtype == torch.float16 and torch.equal(w["layers"][0]["qkv"], want)
    _, w32 = load_checkpoint(path, "cpu", wtype="f32")
    assert w32["layers"][0]["qkv"].dtype == torch.float32


def test_rejected_configs(tmp_path):
    cfg = replace(synth.TINY, n_layers=1)
    path = save_checkpoint(cfg, synth.WeightSet(cfg), "phi3", tmp_path / "x")
    with open(os.path.join(path, "config.json")) as f:
        c = json.load(f)
    for patch, msg in ((dict(rope_scaling={"type": "longrope"}), "rotary scaling"),
                       (dict(model_type="gpt2"), "model_type"),
                       (dict(partial_rotary_factor=0.5), "partial rotary")):
        with open(os.path.join(path, "config.json"), "w") as f:
            json.dump({**c, **patch}, f)
        with pytest.raises(ValueError, match=msg):
            read_config(path)
    with pytest.raises(ValueError, match="wtype"):
        read_config(path, wtype="i8")


def test_sliding_window_is_reported(tmp_path):
    cfg = replace(synth.TINY, n_layers=1)
    path = save_checkpoint(cfg, synth.WeightSet(cfg), "phi3", tmp_path / "w")
    with open(os.path.join(path, "config.json")) as f:
        c = json.load(f)
    with open(os.path.join(path, "config.json"), "w") as f:
        json.dump({**c, "sliding_window": 2047}, f)
    assert read_config(path).sliding_window == 2047
