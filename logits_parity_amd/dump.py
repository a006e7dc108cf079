"""Per-token logit dump of a checkpoint for externally supplied ids.

The harness page ("The direct HF-logits parity harness", section 1) compares
an engine with a reference by dumping the logits of every position for the
same token ids and comparing them offline.  This command is the engine side:

    python -m logits_parity_amd.dump --model DIR --ids IDS --out LOGITS.npy

IDS is a .npy int array [B, S] (or [S]) or a JSON list of lists; the output is
float32 [B, S, vocab] in .npy format.  The prefill runs on the GPU through the
C ABI; there is no CPU path.
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np


def read_ids(path: str) -> np.ndarray:
    if path.endswith(".npy"):
        ids = np.load(path, allow_pickle=False)
    else:
        with open(path) as f:
            ids = np.asarray(json.load(f))
    ids = np.asarray(ids)
    if ids.ndim == 1:
        ids = ids[None, :]
    if ids.ndim != 2 or not np.issubdtype(ids.dtype, np.integer):
        raise ValueError("ids must be integers of shape [B, S] or [S]")
    return ids.astype(np.int32)


def dump(model_dir: str, ids: np.ndarray, wtype: str = "f16", device: str = "cuda:0") -> np.ndarray:
    """Logits float32 [B, S, V] of the checkpoint in `model_dir` for ids [B, S]."""
    import torch

    import logits_parity_amd as phi
    from logits_parity_amd.checkpoint import load_checkpoint

    if not torch.cuda.is_available():
        raise RuntimeError("the logit dump runs on the GPU; no device is visible")
    cfg, weights = load_checkpoint(model_dir, device, wtype)
    B, S = ids.shape
    if S > cfg.max_pos:
        raise ValueError(f"sequence length {S} exceeds the supported {cfg.max_pos} positions")
    if cfg.sliding_window is not None and S > cfg.sliding_window:
        raise ValueError(f"sequence length {S} exceeds the checkpoint's sliding window {cfg.sliding_window}, "
                         "which this engine does not apply")
    model = phi.phi_load_fused(cfg, weights)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    logits = torch.empty((B, S, cfg.vocab), dtype=torch.float32, device=device)
    try:
        # host ids: the library range-checks them before anything is enqueued
        phi.phi_prefill_logits_host_ids(model, ids, logits)
    except phi.PhiError as e:
        if e.status == 4:  # PHI_E_RANGE
            raise ValueError(f"ids must lie in [0, {cfg.vocab})") from e
        raise
    torch.cuda.synchronize()
    return logits.cpu().numpy()


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--model", required=True, help="checkpoint directory (config.json + safetensors)")
    ap.add_argument("--ids", required=True, help=".npy or .json token ids, [B, S] or [S]")
    ap.add_argument("--out", required=True, help="output .npy, float32 [B, S, vocab]")
    ap.add_argument("--wtype", default="f16", choices=["f16", "f32"])
    a = ap.parse_args(argv)
    logits = dump(a.model, read_ids(a.ids), a.wtype)
    np.save(a.out, logits)
    print(f"wrote {a.out}: {logits.shape[0]} x {logits.shape[1]} x {logits.shape[2]} float32", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
