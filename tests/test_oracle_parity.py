"""Pins of the parity metrics (oracle/parity.py) against closed cases.

Every gate in the repository goes through row_cosines, top2_gap and
argmax_report: the per-position cosine and the top-1 agreement that the HF
logits parity harness page defines (section 2, Methods, "Metric + gate"), with
argmax gated where the oracle's top-2 gap exceeds 1e-3.  The checks below use
values fixed by geometry and by construction, not by the functions
themselves, and each planted mistake (a flipped gate comparison, the gap taken
as max - min, an unnormalised cosine, argmax read on the wrong operand, the
gap read from the test operand) must make one of them fail.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import parity


def _basis(n: int, seed: int = 7) -> np.ndarray:
    """A seeded orthonormal basis of R^n (columns)."""
    q, _ = np.linalg.qr(np.random.default_rng(seed).standard_normal((n, n)))
    return q


# ---------------------------------------------------------------- checks
def check_row_cosines(fn) -> None:
    """Rows at known angles, with unequal and non-unit norms, in a rotated
    basis: cosine = cos(theta), for acute, right, obtuse and opposite angles."""
    n = 48
    Q = _basis(n)
    thetas = np.array([0.0, 1e-3, 0.3, np.pi / 3, np.pi / 2, 2.0, np.pi])
    a = np.stack([Q @ np.r_[np.cos(t), np.sin(t), np.zeros(n - 2)] for t in thetas]) * 3.7
    b = np.stack([Q[:, 0] * (0.2 + i) for i in range(len(thetas))])
    got = np.asarray(fn(a, b))
    assert got.shape == (len(thetas),)
    np.testing.assert_allclose(got, np.cos(thetas), rtol=0, atol=1e-13)
    # symmetric, scale-free, and computed per row over the last axis of any shape
    np.testing.assert_allclose(fn(b, a), got, rtol=0, atol=1e-13)
    np.testing.assert_allclose(fn(a.reshape(7, 1, n) * 1e-3, b.reshape(7, 1, n)), got, rtol=0, atol=1e-13)
    # float32 inputs: identical rows give exactly 1
    x = np.ones((1, 4096), dtype=np.float32)
    assert float(fn(x, x)[0]) == 1.0


def check_top2_gap(fn) -> None:
    """Largest minus second-largest, per row: rows built with a known gap, one
    with a tied maximum (gap 0), negative values, and a far minimum (so that
    max - min differs from the gap)."""
    rows = np.array([
        [0.1, 0.5, 0.87, -3.0, 0.2],     # 0.87 - 0.5
        [-1.0, -2.5, -1.25, -9.0, -1.1],  # -1.0 - (-1.1)
        [4.0, 1.0, 4.0, -100.0, 0.0],    # tied maximum
        [0.0, 0.0, 1e-4, 0.0, 0.0],      # gap 1e-4
    ])
    want = np.array([0.37, 0.1, 0.0, 1e-4])
    np.testing.assert_allclose(fn(rows), want, rtol=0, atol=1e-12)
    # order of the row does not matter
    perm = np.random.default_rng(3).permutation(5)
    np.testing.assert_allclose(fn(rows[:, perm]), want, rtol=0, atol=1e-12)


def check_argmax_report(fn) -> None:
    """Planted flips on either side of the 1e-3 gate, with the gap read from
    the oracle operand only."""
    V = 16
    rng = np.random.default_rng(11)
    base = rng.uniform(-1.0, -0.1, size=(6, V))
    oracle = base.copy()
    # row: oracle top index, oracle top-2 gap (top = gap, runner-up = 0, so
    # the gap is exact: row 2 sits exactly at the threshold)
    plan = [(3, 2e-3), (7, 5e-4), (1, 1e-3), (9, 0.5), (12, 2e-3), (5, 0.4)]
    for r, (i, g) in enumerate(plan):
        j = (i + 1) % V
        oracle[r, i], oracle[r, j] = g, 0.0
    test = oracle.copy()
    # rows 0, 1, 2: the test prefers the oracle's runner-up (a flip)
    for r in (0, 1, 2):
        i = plan[r][0]
        j = (i + 1) % V
        test[r, i], test[r, j] = 0.0, plan[r][1]
    # row 4: the test has a huge top-2 gap of its own but agrees; row 5: the
    # test's own gap is tiny and it disagrees, while the oracle's gap is large
    test[4, 12] = 50.0
    test[5, 5], test[5, 6] = 0.0, 1e-6
    rep = fn(test, oracle)
    assert rep["rows"] == 6
    # gated: gap > 1e-3 strictly -> rows 0, 3, 4, 5 (row 2 sits exactly at 1e-3)
    assert rep["gated"] == 4, rep
    # agreement: rows 3, 4 agree among the gated ones; 0 and 5 are failures
    assert rep["gated_agree"] == 2, rep
    assert rep["failures"] == [0, 5], rep
    # all rows: 3 and 4 agree; 0, 1, 2, 5 do not
    assert rep["agree_all"] == 2, rep
    # a near-tie flip alone is accepted
    rep = fn(test[1:2], oracle[1:2])
    assert rep["gated"] == 0 and rep["failures"] == []
    # the threshold is a parameter: at 1e-4 the row with gap 5e-4 is gated and fails
    rep = fn(test[1:2], oracle[1:2], gap_min=1e-4)
    assert rep["gated"] == 1 and rep["failures"] == [0]


def check_summary(fn) -> None:
    """min/mean cosine and the worst row of a known set of angles."""
    n = 32
    Q = _basis(n, 5)
    thetas = np.array([0.01, 0.002, 0.03, 0.0])
    test = np.stack([Q @ np.r_[np.cos(t), np.sin(t), np.zeros(n - 2)] for t in thetas])
    oracle = np.stack([Q[:, 0] * 2.0 for _ in thetas])
    s = fn(test, oracle)
    assert s["worst_row"] == 2
    assert abs(s["min_cos"] - np.cos(0.03)) < 1e-13
    assert abs(s["mean_cos"] - np.cos(thetas).mean()) < 1e-13


# ---------------------------------------------------------------- the real functions pass
def test_row_cosines_known_angles():
    check_row_cosines(parity.row_cosines)


def test_top2_gap_known_gaps():
    check_top2_gap(parity.top2_gap)


def test_argmax_report_planted_flips():
    check_argmax_report(parity.argmax_report)


def test_summary_known_angles():
    check_summary(parity.summary)


# ---------------------------------------------------------------- planted mistakes fail
def _cos_unnormalised(a, b):
    a = np.asarray(a, dtype=np.float64).reshape(-1, np.shape(a)[-1])
    b = np.asarray(b, dtype=np.float64).reshape(-1, np.shape(b)[-1])
    return np.einsum("ij,ij->i", a, b)


def _cos_float32(a, b):
    a = np.asarray(a, dtype=np.float32).reshape(-1, np.shape(a)[-1])
    b = np.asarray(b, dtype=np.float32).reshape(-1, np.shape(b)[-1])
    num = np.sum(a * b, axis=1, dtype=np.float32)
    return num / (np.linalg.norm(a, axis=1) * np.linalg.norm(b, axis=1))


def _gap_max_minus_min(o):
    o = np.asarray(o, dtype=np.float64).reshape(-1, np.shape(o)[-1])
    return o.max(axis=1) - o.min(axis=1)


def _gap_unique_values(o):
    # a tied maximum would count the next distinct value
    o = np.asarray(o, dtype=np.float64).reshape(-1, np.shape(o)[-1])
    out = []
    for r in o:
        u = np.unique(r)
        out.append(u[-1] - u[-2])
    return np.array(out)


def _report_variant(flip_gate=False, wrong_operand=False, gap_from_test=False):
    def fn(test, oracle, gap_min=1e-3):
        t = np.asarray(test).reshape(-1, np.shape(test)[-1])
        o = np.asarray(oracle, dtype=np.float64).reshape(-1, np.shape(oracle)[-1])
        gap = parity.top2_gap(t if gap_from_test else o)
        agree = np.argmax(o if wrong_operand else t, axis=1) == np.argmax(o, axis=1)
        gated = gap < gap_min if flip_gate else gap > gap_min
        return {"rows": int(len(gap)), "gated": int(gated.sum()), "gated_agree": int((agree & gated).sum()),
                "agree_all": int(agree.sum()), "failures": np.nonzero(gated & ~agree)[0].tolist()}
    return fn


def _report_gate_inclusive(test, oracle, gap_min=1e-3):
    t = np.asarray(test).reshape(-1, np.shape(test)[-1])
    o = np.asarray(oracle, dtype=np.float64).reshape(-1, np.shape(oracle)[-1])
    gap = parity.top2_gap(o)
    agree = np.argmax(t, axis=1) == np.argmax(o, axis=1)
    gated = gap >= gap_min
    return {"rows": int(len(gap)), "gated": int(gated.sum()), "gated_agree": int((agree & gated).sum()),
            "agree_all": int(agree.sum()), "failures": np.nonzero(gated & ~agree)[0].tolist()}


@pytest.mark.parametrize("mutant", [_cos_unnormalised, _cos_float32], ids=["unnormalised", "float32-sums"])
def test_cosine_mutants_fail(mutant):
    with pytest.raises(AssertionError):
        check_row_cosines(mutant)


@pytest.mark.parametrize("mutant", [_gap_max_minus_min, _gap_unique_values], ids=["max-minus-min", "unique"])
def test_gap_mutants_fail(mutant):
    with pytest.raises(AssertionError):
        check_top2_gap(mutant)


@pytest.mark.parametrize("kw", [{"flip_gate": True}, {"wrong_operand": True}, {"gap_from_test": True}],
                         ids=["flipped-gate", "argmax-on-oracle-only", "gap-from-test"])
def test_report_mutants_fail(kw):
    with pytest.raises(AssertionError):
        check_argmax_report(_report_variant(**kw))


def test_report_inclusive_gate_fails():
    with pytest.raises(AssertionError):
        check_argmax_report(_report_gate_inclusive)


def test_report_with_max_minus_min_gap_fails(monkeypatch):
    # the report reads the gap through top2_gap: a wrong gap there breaks it too
    monkeypatch.setattr(parity, "top2_gap", _gap_max_minus_min)
    with pytest.raises(AssertionError):
        check_argmax_report(parity.argmax_report)
