"""The other dense families of the parity harness page (section 3) through
the same C ABI, on random weights at their public shapes (GPU):
Qwen2.5-0.5B-style (24 layers, GQA 14/2 at head_dim 64, QKV bias, tied
embeddings, vocab 151936) and SmolLM2-360M-style (32 layers, GQA 15/5 at
head_dim 64, tied, vocab 49152).  Gates as for Phi-3: per-position cosine
>= 0.99999 against the fp64 oracle (pinned against transformers' Qwen2 and
Llama) and argmax agreement where the oracle's top-2 gap exceeds 1e-3.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from oracle import parity, prefill

pytestmark = pytest.mark.gpu
COS_GATE = 0.99999


def _say(*a):
    print(*a, flush=True)


def _run(phi, cfg, ws, ids):
    from logits_parity_amd.weights import to_device
    dev = to_device(ws, cfg.n_layers)
    if cfg.tie_embeddings and cfg.wtype != "i8":
        assert dev["lm_head"] is dev["embed"]       # one device tensor serves both
    m = phi.phi_load_fused(cfg, dev)
    out = m.prefill_logits(torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda())
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _gate(got, ref):
    s = parity.summary(got.reshape(-1, got.shape[-1]), ref.reshape(-1, ref.shape[-1]))
    _say(f"  min_cos={s['min_cos']:.9f} gated={s['gated']} agree={s['gated_agree']}")
    assert np.all(np.isfinite(got))
    assert s["min_cos"] >= COS_GATE, s
    assert not s["failures"], s


@pytest.mark.parametrize("name,batch,seq", [("qwen25_05b", 1, 64), ("qwen25_05b", 2, 37),
                                            ("smollm2_360m", 1, 64), ("smollm2_360m", 3, 21)])
def test_family_f16_vs_oracle(phi, name, batch, seq):
    cfg = {"qwen25_05b": synth.QWEN25_05B, "smollm2_360m": synth.SMOLLM2_360M}[name]
    _say(f"{name} f16 {batch}x{seq}")
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, batch, seq)
    _gate(_run(phi, cfg, ws, ids), prefill.prefill_logits(cfg, ws, ids))


def test_qwen_style_int8_unit_gains(phi):
    # int8 weights (the tied lm_head is the int8 code of the embedding), unit
    # gains; gated against the oracle run on the same int8 weights
    cfg = replace(synth.QWEN25_05B, n_layers=4, wtype="i8", norm_gain="ones")
    _say("qwen25_05b int8 4 layers 1x48")
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, 1, 48)
    _gate(_run(phi, cfg, ws, ids), prefill.prefill_logits(cfg, ws, ids))


def test_attention_head_dim_64_kernel(phi):
    from test_gpu_kernels import _attn_gpu, _attn_inputs, _attn_ref
    for B, S, nh, nkv in ((1, 1, 2, 1), (1, 77, 14, 2), (2, 130, 15, 5)):
        q, k, v = _attn_inputs(B, S, nh, nkv, np.float16, 61 + S, scale=1.5, D=64)
        got = _attn_gpu(phi, q, k, v)
        ref = _attn_ref(q, k, v)
        assert np.all(np.abs(got - ref) <= 2e-3 + 2e-3 * np.abs(ref)), (S, np.abs(got - ref).max())
