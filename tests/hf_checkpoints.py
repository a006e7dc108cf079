"""Test helper: write a synthetic weight set as a HuggingFace checkpoint
directory with transformers' own save_pretrained (config.json +
model.safetensors), so that the loader is checked against files written by an
independent implementation of the format."""
import numpy as np
import torch


def hf_model(cfg, ws, family: str, dtype=torch.float16):
    """transformers model of `family` ("phi3", "qwen2" or "llama") holding the
    weights of `ws`, cast to dtype."""
    from transformers import (LlamaConfig, LlamaForCausalLM, Phi3Config, Phi3ForCausalLM, Qwen2Config,
                              Qwen2ForCausalLM)
    common = dict(vocab_size=cfg.vocab, hidden_size=cfg.hidden, intermediate_size=cfg.intermediate,
                  num_hidden_layers=cfg.n_layers, num_attention_heads=cfg.n_heads,
                  num_key_value_heads=cfg.n_kv_heads, max_position_embeddings=4096, rms_norm_eps=cfg.rms_eps,
                  rope_theta=cfg.rope_theta, tie_word_embeddings=cfg.tie_embeddings, pad_token_id=0,
                  bos_token_id=1, eos_token_id=2)
    if family == "phi3":
        hc, M = Phi3Config(**common, original_max_position_embeddings=4096), Phi3ForCausalLM
    elif family == "qwen2":
        hc, M = Qwen2Config(**common, use_sliding_window=False), Qwen2ForCausalLM
    else:
        hc, M = LlamaConfig(**common, attention_bias=False, mlp_bias=False), LlamaForCausalLM
    torch.manual_seed(0)
    m = M(hc).eval()
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32))
    nq, nk = cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    sd = {"model.embed_tokens.weight": t(ws.embed), "model.norm.weight": t(ws.final_norm)}
    if not cfg.tie_embeddings:
        sd["lm_head.weight"] = t(ws.lm_head)
    for l in range(cfg.n_layers):
        w, p = ws.layer(l), f"model.layers.{l}."
        sd.update({p + "self_attn.o_proj.weight": t(w["o"]), p + "mlp.down_proj.weight": t(w["down"]),
                   p + "input_layernorm.weight": t(w["ln1"]), p + "post_attention_layernorm.weight": t(w["ln2"])})
        qkv, gu = t(w["qkv"]), t(w["gate_up"])
        if family == "phi3":
            sd.update({p + "self_attn.qkv_proj.weight": qkv, p + "mlp.gate_up_proj.weight": gu})
        else:
            sd.update({p + "self_attn.q_proj.weight": qkv[:nq], p + "self_attn.k_proj.weight": qkv[nq:nq + nk],
                       p + "self_attn.v_proj.weight": qkv[nq + nk:],
                       p + "mlp.gate_proj.weight": gu[:cfg.intermediate],
                       p + "mlp.up_proj.weight": gu[cfg.intermediate:]})
            if cfg.qkv_bias:
                b = t(w["qkv_bias"])
                sd.update({p + "self_attn.q_proj.bias": b[:nq], p + "self_attn.k_proj.bias": b[nq:nq + nk],
                           p + "self_attn.v_proj.bias": b[nq + nk:]})
    missing, unexpected = m.load_state_dict(sd, strict=False)
    missing = [k for k in missing if k != "lm_head.weight"]
    assert not missing and not unexpected, (missing, unexpected)
    return m.to(dtype)


def save_checkpoint(cfg, ws, family: str, path, dtype=torch.float16):
    """Write the HuggingFace checkpoint directory of `ws` to `path`."""
    hf_model(cfg, ws, family, dtype).save_pretrained(str(path), safe_serialization=True)
    return str(path)
