"""Parity metrics of the logits harness — TEST INFRASTRUCTURE ONLY.

The page "The direct HF-logits parity harness" (section 1 and the Methods
table) compares an engine's per-token logits with an oracle's row by row:
cosine similarity per token row is the gate, argmax agreement is reported.
The Phi-3-mini page (section 2, Methods: "Metric + gate") uses the same
per-position cosine and top-1 count.
"""
from __future__ import annotations

import numpy as np


def row_cosines(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Cosine of each last-axis row of a against the same row of b, in fp64."""
    a = np.asarray(a, dtype=np.float64).reshape(-1, a.shape[-1])
    b = np.asarray(b, dtype=np.float64).reshape(-1, b.shape[-1])
    num = np.einsum("ij,ij->i", a, b)
    den = np.linalg.norm(a, axis=1) * np.linalg.norm(b, axis=1)
    return num / den


def top2_gap(oracle: np.ndarray) -> np.ndarray:
    """Per row: largest minus second-largest logit."""
    o = np.asarray(oracle, dtype=np.float64).reshape(-1, oracle.shape[-1])
    part = np.partition(o, -2, axis=1)
    return part[:, -1] - part[:, -2]


def argmax_report(test: np.ndarray, oracle: np.ndarray, gap_min: float = 1e-3) -> dict:
    """Argmax agreement; a row is gated when the oracle's top-2 gap exceeds
    gap_min (near-ties may resolve either way)."""
    t = np.asarray(test).reshape(-1, test.shape[-1])
    o = np.asarray(oracle, dtype=np.float64).reshape(-1, oracle.shape[-1])
    gap = top2_gap(o)
    agree = np.argmax(t, axis=1) == np.argmax(o, axis=1)
    gated = gap > gap_min
    return {"rows": int(len(gap)), "gated": int(gated.sum()), "gated_agree": int((agree & gated).sum()),
            "agree_all": int(agree.sum()), "failures": np.nonzero(gated & ~agree)[0].tolist()}


def summary(test: np.ndarray, oracle: np.ndarray, gap_min: float = 1e-3) -> dict:
    cos = row_cosines(test, oracle)
    rep = argmax_report(test, oracle, gap_min)
    rep.update({"min_cos": float(cos.min()), "mean_cos": float(cos.mean()),
                "worst_row": int(np.argmin(cos))})
    return rep
