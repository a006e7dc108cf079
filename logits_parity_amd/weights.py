"""Upload host weights (numpy, as stored) into device tensors for the binding."""
from __future__ import annotations

import numpy as np


def _dev(a, device):
    import torch
    if isinstance(a, tuple):
        return tuple(_dev(t, device) for t in a)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_device(source, n_layers: int, device="cuda"):
    """`source` exposes .embed, .layer(l) (dict: ln1, qkv, o, ln2, gate_up,
    down, optional qkv_bias), .final_norm and .lm_head as numpy arrays, or
    (int8 codes, float16 scales) tuples.  Returns the dict phi_load_fused's
    binding expects.  A tied lm_head (the same array as the embedding) is
    uploaded once and shared."""
    layers = []
    for l in range(n_layers):
        lw = source.layer(l)
        layers.append({k: _dev(lw[k], device) for k in ("ln1", "qkv", "o", "ln2", "gate_up", "down", "qkv_bias")
                       if k in lw})
    embed = _dev(source.embed, device)
    lm = embed if source.lm_head is source.embed else _dev(source.lm_head, device)
    return {"embed": embed, "layers": layers, "final_norm": _dev(source.final_norm, device), "lm_head": lm}
