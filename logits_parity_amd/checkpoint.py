"""HuggingFace-layout safetensors checkpoints onto this library's fused layout.

The Phi-3-mini page ("Phi-3-mini: fused-tensor direct loading in a sovereign
inference engine", section 1 and section 5, loading path) loads the fused
QKV and gate/up tensors of a Phi-3 checkpoint directly, without splitting
them; the harness page ("The direct HF-logits parity harness", section 1)
dumps per-token logits for externally supplied ids.  This module reads such a
checkpoint directory (config.json plus one model.safetensors file, or shards
listed in model.safetensors.index.json) and returns the config and the device
tensors that `phi_load_fused` borrows:

  - "phi3": self_attn.qkv_proj and mlp.gate_up_proj are used as stored, one
    tensor each (a dtype cast only when the file's dtype differs from the
    compute type, e.g. bfloat16 files for the binary16 path);
  - "llama", "qwen2" (the other dense families of the harness page, section
    3): q/k/v and gate/up are stored separately and are stacked here, in the
    row order Q, K, V and gate, up, into the fused layout; a Qwen2 QKV bias is
    stacked the same way; a tied lm_head is the embedding tensor.

Limits: positions up to 4096 (the engine's RoPE table), rotary scaling is not
wired (a config with rope_scaling is rejected), and a config's sliding window
is reported in `sliding_window` but not applied: logits equal a windowed
reference only for sequences no longer than the window (callers check, as the
dump command does).  Weights are loaded as binary16 or float32; 8-bit weights
are not produced here.
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass

MAX_POSITIONS = 4096

_FAMILIES = {"phi3": "phi3", "llama": "llama", "qwen2": "qwen2"}


@dataclass(frozen=True)
class CheckpointConfig:
    """The model shape fields `phi_load_fused` needs, read from config.json."""
    name: str
    family: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    max_pos: int
    rms_eps: float
    rope_theta: float
    wtype: str                 # "f16" or "f32"
    qkv_bias: bool
    tie_embeddings: bool
    sliding_window: int | None


def read_config(path: str, wtype: str = "f16") -> CheckpointConfig:
    """config.json of a checkpoint directory -> CheckpointConfig.  Raises
    ValueError for families or features this engine does not run."""
    if wtype not in ("f16", "f32"):
        raise ValueError(f"wtype must be 'f16' or 'f32', got {wtype!r}")
    with open(os.path.join(path, "config.json")) as f:
        c = json.load(f)
    family = _FAMILIES.get(c.get("model_type", ""))
    if family is None:
        raise ValueError(f"unsupported model_type {c.get('model_type')!r} (phi3, llama, qwen2)")
    if c.get("rope_scaling"):
        raise ValueError("rotary scaling (rope_scaling) is not wired: positions up to 4096 with plain RoPE only")
    if float(c.get("partial_rotary_factor", 1.0)) != 1.0:
        raise ValueError("partial rotary embeddings are not supported")
    hidden = int(c["hidden_size"])
    heads = int(c["num_attention_heads"])
    kv = int(c.get("num_key_value_heads") or heads)
    head_dim = int(c.get("head_dim") or hidden // heads)
    if family == "llama" and (c.get("attention_bias") or c.get("mlp_bias")):
        raise ValueError("Llama-style biases are not supported")
    window = c.get("sliding_window")
    if family == "qwen2" and not c.get("use_sliding_window", False):
        window = None
    return CheckpointConfig(
        name=os.path.basename(os.path.normpath(path)),
        family=family,
        n_layers=int(c["num_hidden_layers"]),
        hidden=hidden,
        n_heads=heads,
        n_kv_heads=kv,
        head_dim=head_dim,
        intermediate=int(c["intermediate_size"]),
        vocab=int(c["vocab_size"]),
        max_pos=min(int(c.get("max_position_embeddings", MAX_POSITIONS)), MAX_POSITIONS),
        rms_eps=float(c.get("rms_norm_eps", 1e-5)),
        rope_theta=float(c.get("rope_theta", 10000.0)),
        wtype=wtype,
        qkv_bias=family == "qwen2",
        tie_embeddings=bool(c.get("tie_word_embeddings", False)),
        sliding_window=int(window) if window else None,
    )


class _Tensors:
    """Lazy access to the checkpoint's tensors, shard by shard."""

    def __init__(self, path: str, device: str):
        from safetensors import safe_open
        index = os.path.join(path, "model.safetensors.index.json")
        if os.path.exists(index):
            with open(index) as f:
                wmap = json.load(f)["weight_map"]
            files = sorted(set(wmap.values()))
        else:
            files = ["model.safetensors"]
            wmap = None
        self._handles = {fn: safe_open(os.path.join(path, fn), framework="pt", device=device) for fn in files}
        if wmap is None:
            wmap = {k: files[0] for k in self._handles[files[0]].keys()}
        self._map = wmap

    def has(self, name: str) -> bool:
        return name in self._map

    def get(self, name: str):
        if name not in self._map:
            raise KeyError(f"tensor {name!r} not in the checkpoint")
        return self._handles[self._map[name]].get_tensor(name)


def load_checkpoint(path: str, device="cuda", wtype: str = "f16"):
    """Returns (CheckpointConfig, weights dict for phi_load_fused) with every
    tensor on `device`.  Phi-3 fused tensors are used as stored (cast only if
    the stored dtype is not the compute type)."""
    import torch

    cfg = read_config(path, wtype)
    dt = torch.float16 if wtype == "f16" else torch.float32
    ts = _Tensors(path, str(device))

    def get(name, shape):
        t = ts.get(name)
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
        return t if t.dtype == dt else t.to(dt)

    H, I, V, hd = cfg.hidden, cfg.intermediate, cfg.vocab, cfg.head_dim
    q_rows, kv_rows = cfg.n_heads * hd, cfg.n_kv_heads * hd
    layers = []
    for l in range(cfg.n_layers):
        p = f"model.layers.{l}."
        lw = {"ln1": get(p + "input_layernorm.weight", (H,)),
              "ln2": get(p + "post_attention_layernorm.weight", (H,)),
              "o": get(p + "self_attn.o_proj.weight", (H, q_rows)),
              "down": get(p + "mlp.down_proj.weight", (H, I))}
        if cfg.family == "phi3":
            lw["qkv"] = get(p + "self_attn.qkv_proj.weight", (q_rows + 2 * kv_rows, H))
            lw["gate_up"] = get(p + "mlp.gate_up_proj.weight", (2 * I, H))
        else:
            lw["qkv"] = torch.cat([get(p + "self_attn.q_proj.weight", (q_rows, H)),
                                   get(p + "self_attn.k_proj.weight", (kv_rows, H)),
                                   get(p + "self_attn.v_proj.weight", (kv_rows, H))], 0).contiguous()
            lw["gate_up"] = torch.cat([get(p + "mlp.gate_proj.weight", (I, H)),
                                       get(p + "mlp.up_proj.weight", (I, H))], 0).contiguous()
            if cfg.qkv_bias:
                lw["qkv_bias"] = torch.cat([get(p + "self_attn.q_proj.bias", (q_rows,)),
                                            get(p + "self_attn.k_proj.bias", (kv_rows,)),
                                            get(p + "self_attn.v_proj.bias", (kv_rows,))], 0).contiguous()
        layers.append(lw)
    embed = get("model.embed_tokens.weight", (V, H))
    if cfg.tie_embeddings or not ts.has("lm_head.weight"):
        lm_head = embed
    else:
        lm_head = get("lm_head.weight", (V, H))
    weights = {"embed": embed, "layers": layers, "final_norm": get("model.norm.weight", (H,)), "lm_head": lm_head}
    return cfg, weights
