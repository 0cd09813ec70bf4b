"""Central finite differences of the oracle's gradients, and planted mistakes
that the pins must catch.

Finite differences follow the by-hand page, section four (double precision, two
step sizes, a threshold fixed in advance: 1e-7 absolute) and chapter 31, sec. 6
(scalar loss L = sum(O * G_O), every element of Q, K and V perturbed by +-eps).
Inputs are N(0,1) so no softmax row saturates (by-hand page, section four).
"""

import numpy as np
import pytest

import oracle
from oracle import attention as oa

from test_oracle_pins import MASK_CASES, random_problem, run_example, load

EPS = (1e-5, 1e-6)
THRESHOLD = 1e-7


def loss(Q, K, V, GO, kw):
    return float((oracle.attention_forward(Q, K, V, **kw)["O"] * GO).sum())


def fd_max_error(Q, K, V, GO, kw):
    out = oracle.attention_backward(Q, K, V, GO, **kw)
    analytic = {"Q": out["GQ"], "K": out["GK"], "V": out["GV"]}
    worst = 0.0
    for eps in EPS:
        for name in ("Q", "K", "V"):
            arrs = {"Q": Q, "K": K, "V": V}
            X = arrs[name]
            for idx in np.ndindex(X.shape):
                orig = X[idx]
                X[idx] = orig + eps
                lp = loss(arrs["Q"], arrs["K"], arrs["V"], GO, kw)
                X[idx] = orig - eps
                lm = loss(arrs["Q"], arrs["K"], arrs["V"], GO, kw)
                X[idx] = orig
                worst = max(worst, abs((lp - lm) / (2 * eps) - analytic[name][idx]))
    return worst


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: c["name"])
def test_finite_differences_every_coordinate(case):
    Q, K, V, GO, kw = random_problem(case, seed=21)
    assert fd_max_error(Q, K, V, GO, kw) < THRESHOLD


def test_finite_differences_worked_example():
    """The by-hand page's own check: every coordinate of Q, K, V of worked
    example 1 with the probe G."""
    import math
    Q = (math.sqrt(2) * math.log(3) * np.eye(2))[None, None].copy()
    K = np.eye(2)[None, None].copy()
    V = np.diag([2.0, 4.0])[None, None].copy()
    G = np.array([[1.0, 0.0], [0.0, 2.0]])[None, None]
    assert fd_max_error(Q, K, V, G, {}) < THRESHOLD


# ---------------------------------------------------------------------------
# planted mistakes (chapter 31, sec. 8 negative controls): each must make a
# pin fail.  The mistakes are planted in the oracle, on the CPU, via monkeypatch.
# ---------------------------------------------------------------------------

def _drop_c(A, GA, M):
    GS = np.where(M, A * GA, 0.0)
    return GS, np.zeros(A.shape[0])


def _no_mask_softmax(S, M):
    # ignores the visible set (only inactive rows kept zero)
    active = M.any(axis=1)
    full = np.where(active[:, None], True, False) & np.ones_like(M)
    return _orig_softmax(S, full)


def _column_softmax(S, M):
    A, m, ell = _orig_softmax(S.T, M.T)
    return A.T, m, ell


def _no_transpose_scores(q, k):
    return (q @ k) / np.sqrt(q.shape[1])


_orig_softmax = oa.masked_softmax


def test_mutation_drop_row_term_fails_fd_and_rowsum(monkeypatch):
    monkeypatch.setattr(oa, "score_grad", _drop_c)
    case = MASK_CASES[0]
    Q, K, V, GO, kw = random_problem(case, seed=21)
    assert fd_max_error(Q, K, V, GO, kw) > 1e-3
    _, _, _, out = run_example(np.eye(2))
    assert not np.allclose(out["GS"][0], load("worked_example_1.json")["printed"]["dS"])


def test_mutation_drop_mask_fails_causal_gradient_test(monkeypatch):
    monkeypatch.setattr(oa, "masked_softmax", _no_mask_softmax)
    rng = np.random.default_rng(11)
    Q = rng.normal(size=(1, 1, 5, 4))
    K = rng.normal(size=(1, 1, 8, 4))
    V = rng.normal(size=(1, 1, 8, 3))
    GO = np.zeros((1, 1, 5, 3))
    GO[:, :, 0] = 1.0
    out = oracle.attention_backward(Q, K, V, GO, causal=True)
    assert np.abs(out["GV"][0, 0, 1:]).max() > 1e-3


def test_mutation_column_normalisation_fails_row_sums(monkeypatch):
    monkeypatch.setattr(oa, "masked_softmax", _column_softmax)
    rng = np.random.default_rng(1)
    Q = rng.normal(size=(1, 1, 4, 4))
    K = rng.normal(size=(1, 1, 4, 4))
    V = rng.normal(size=(1, 1, 4, 3))
    out = oracle.attention_forward(Q, K, V, keep=True)
    assert not np.allclose(out["A"][0].sum(axis=1), 1.0)


def test_mutation_missing_transpose_fails_transpose_check(monkeypatch):
    monkeypatch.setattr(oa, "scores", _no_transpose_scores)
    gold = load("transpose_check.json")
    Q = np.array(gold["inputs"]["Q"])[None, None]
    K = np.array(gold["inputs"]["K"])[None, None]
    out = oracle.attention_forward(Q, K, np.eye(2)[None, None], keep=True)
    assert not np.allclose(out["S"][0] * np.sqrt(2), gold["printed"]["QKt"])
