"""Grouped-query prefill at head_dim 128 (the Phi-4 geometry) vs the oracle (GPU).

Gates as for the Phi-3 prefill: per-position logit cosine >= 0.99999 against
the fp64 oracle and argmax agreement wherever the oracle's top-2 gap exceeds
1e-3.  The oracle's head_dim 128 path is pinned against transformers' Phi-3.
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
    m = phi.phi_load_fused(cfg, to_device(ws, cfg.n_layers))
    out = m.prefill_logits(torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda())
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _gate(got, ref):
    s = parity.summary(got.reshape(-1, got.shape[-1]), ref.reshape(-1, ref.shape[-1]))
    _say(f"  min_cos={s['min_cos']:.9f} gated={s['gated']} agree={s['gated_agree']}")
    assert np.all(np.isfinite(got))
    assert s["min_cos"] >= COS_GATE, s
    assert not s["failures"], s


@pytest.mark.parametrize("batch,seq", [(2, 64), (1, 70), (3, 5)])
def test_tiny_gqa128_f16(phi, batch, seq):
    cfg = synth.TINY_GQA128
    _say(f"tiny gqa128 f16 {batch}x{seq}")
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, batch, seq)
    _gate(_run(phi, cfg, ws, ids), prefill.prefill_logits(cfg, ws, ids))


def test_tiny_gqa128_unit_gains_int8(phi):
    cfg = replace(synth.TINY_GQA128, norm_gain="ones", wtype="i8")
    _say("tiny gqa128 int8 unit gains")
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, 2, 40)
    _gate(_run(phi, cfg, ws, ids), prefill.prefill_logits(cfg, ws, ids))


def test_phi4_one_layer_full_width(phi):
    # hidden 5120, 40 query heads over 10 KV heads at 128, intermediate 17920,
    # vocab 100352: one decoder layer at full Phi-4 width
    cfg = synth.PHI4_1L
    _say("phi4 1 layer 1x100")
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, 1, 100)
    _gate(_run(phi, cfg, ws, ids), prefill.prefill_logits(cfg, ws, ids))
