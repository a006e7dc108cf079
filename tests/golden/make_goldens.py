"""Write the stored fp64-oracle results used by the full-size GPU parity tests.

Calls only ``oracle`` and ``synth``: every stored value is the oracle's.
For each prefill workload it saves ``<workload>.npz`` holding
  weights_sha256, ids_sha256  digests of the exact input bytes (the GPU test
                              refuses to compare if its inputs differ)
  argmax, gap                 oracle argmax and top-2 gap at every position
  pos, rows                   full oracle logit rows (float32) at sampled
                              positions, flat index b * seq + s
  hidden                      the oracle's normalised final hidden state
                              rmsnorm(x) * g_final at every position, float32
                              [batch * seq, hidden]: a test forms any logit
                              row from it with the oracle's own lm_head step
                              (oracle.prefill.logits_from_hidden).  Rounding
                              it to float32 moves a row's cosine by about
                              1e-14, far below the 1e-5 gate.
and, for the int8 workload, argmax, gap, pos and rows for the float16 oracle
on the float16 weights the int8 ones were quantized from (prefix ``f16_``).

Usage:  python tests/golden/make_goldens.py [workload ...]
"""
from __future__ import annotations

import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import synth  # noqa: E402
from oracle import parity, prefill  # noqa: E402

SAMPLES = {
    "mini_f16_1x512": [0, 1, 2, 5, 17, 64, 127, 128, 255, 256, 383, 400, 480, 509, 510, 511],
    "mini_f16_1x4096": [0, 1, 3, 100, 511, 512, 1000, 1023, 1024, 2047, 2048, 3000, 3500, 4000, 4094, 4095],
    "mini_w8_4x1024": [0, 511, 1022, 1023, 1024, 1500, 2046, 2047, 2048, 2600, 3070, 3071, 3072, 3600, 4094, 4095],
}


def ids_digest(ids: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(ids, dtype=np.int32).tobytes()).hexdigest()


def run(cfg, ids, pos, keep_hidden=True):
    ws = synth.WeightSet(cfg, cache_layers=False)
    t = time.time()
    hidden = prefill.final_hidden(cfg, ws, ids).reshape(-1, cfg.hidden)
    flat = prefill.logits_from_hidden(hidden, ws.lm_head)
    print(f"  oracle {cfg.name} {ids.shape}: {time.time() - t:.0f} s", flush=True)
    out = {"argmax": np.argmax(flat, axis=1).astype(np.int32), "gap": parity.top2_gap(flat),
           "rows": flat[pos].astype(np.float32)}
    if keep_hidden:
        out["hidden"] = hidden.astype(np.float32)
        # the stored (float32) hidden state reproduces the fp64 rows
        again = prefill.logits_from_hidden(out["hidden"][pos], ws.lm_head)
        print(f"  float32 hidden: min row cosine {parity.row_cosines(again, flat[pos]).min():.15f}", flush=True)
    del hidden, flat
    out["weights_sha256"] = np.array(synth.WeightSet(cfg, cache_layers=False).digest())
    return out


def make(name: str):
    wl = synth.PREFILL_WORKLOADS[name]
    ids = synth.token_ids(wl.cfg, wl.batch, wl.seq)
    pos = np.array(SAMPLES[name], dtype=np.int64)
    res = {"pos": pos, "ids_sha256": np.array(ids_digest(ids))}
    res.update(run(wl.cfg, ids, pos))
    if wl.cfg.wtype == "i8":
        f16 = run(synth.as_f16_config(wl.cfg), ids, pos, keep_hidden=False)
        res.update({"f16_" + k: v for k, v in f16.items()})
    path = os.path.join(HERE, name + ".npz")
    np.savez_compressed(path, **res)
    print(f"wrote {path}", flush=True)


if __name__ == "__main__":
    names = sys.argv[1:] or list(SAMPLES)
    for n in names:
        make(n)
