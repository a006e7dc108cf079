"""Checkpoint directories written by transformers' save_pretrained, loaded
and run end to end by the logit-dump path (GPU).

Gates as for every prefill: per-position cosine >= 0.99999 against the fp64
oracle on the same weights and argmax agreement where the oracle's top-2 gap
exceeds 1e-3.  The dump command's file output equals the in-process result.
"""
from dataclasses import replace

import numpy as np
import pytest

import synth
from hf_checkpoints import save_checkpoint
from oracle import parity, prefill

pytestmark = pytest.mark.gpu
COS_GATE = 0.99999


def _say(*a):
    print(*a, flush=True)


def _gate(got, ref):
    s = parity.summary(got.reshape(-1, got.shape[-1]), ref.reshape(-1, ref.shape[-1]))
    _say(f"  min_cos={s['min_cos']:.9f} gated={s['gated']} agree={s['gated_agree']}")
    assert np.all(np.isfinite(got))
    assert s["min_cos"] >= COS_GATE, s
    assert not s["failures"], s


@pytest.mark.parametrize("family,wtype", [("phi3", "f16"), ("phi3", "f32"), ("qwen2", "f16"), ("llama", "f16")])
def test_checkpoint_dump_vs_oracle(phi, tmp_path, family, wtype):
    from logits_parity_amd.dump import dump
    base = {"phi3": synth.TINY, "qwen2": synth.QWEN25_05B, "llama": synth.SMOLLM2_360M}[family]
    cfg = replace(base, wtype=wtype) if family == "phi3" else replace(base, n_layers=2, vocab=2048)
    _say(f"checkpoint {family} {wtype}")
    ws = synth.WeightSet(cfg)
    import torch
    path = save_checkpoint(cfg, ws, family, tmp_path / family, dtype=torch.float32 if wtype == "f32" else torch.float16)
    ids = synth.token_ids(cfg, 2, 23)
    got = dump(path, ids, wtype)
    _gate(got, prefill.prefill_logits(cfg, ws, ids))


def test_dump_command_writes_the_logits(phi, tmp_path):
    from logits_parity_amd.dump import dump, main
    cfg = synth.TINY
    ws = synth.WeightSet(cfg)
    path = save_checkpoint(cfg, ws, "phi3", tmp_path / "m")
    ids = synth.token_ids(cfg, 1, 17)
    np.save(tmp_path / "ids.npy", ids)
    assert main(["--model", path, "--ids", str(tmp_path / "ids.npy"), "--out", str(tmp_path / "out.npy")]) == 0
    out = np.load(tmp_path / "out.npy")
    assert out.dtype == np.float32 and out.shape == (1, 17, cfg.vocab)
    assert np.array_equal(out, dump(path, ids))      # deterministic: the same logits twice
    with open(tmp_path / "ids.json", "w") as f:
        f.write(str(ids[0].tolist()))
    assert main(["--model", path, "--ids", str(tmp_path / "ids.json"), "--out", str(tmp_path / "o2.npy")]) == 0
    assert np.array_equal(np.load(tmp_path / "o2.npy"), out)


def test_dump_refuses_what_it_cannot_compute(phi, tmp_path):
    import json
    import os
    from logits_parity_amd.dump import dump
    cfg = replace(synth.TINY, n_layers=1)
    path = save_checkpoint(cfg, synth.WeightSet(cfg), "phi3", tmp_path / "m")
    with pytest.raises(ValueError, match=r"ids must lie"):
        dump(path, np.array([[0, cfg.vocab]], np.int32))
    with open(os.path.join(path, "config.json")) as f:
        c = json.load(f)
    with open(os.path.join(path, "config.json"), "w") as f:
        json.dump({**c, "sliding_window": 8}, f)
    with pytest.raises(ValueError, match="sliding window"):
        dump(path, np.zeros((1, 9), np.int32))
