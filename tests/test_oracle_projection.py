"""Pins of the oracle's projections (oracle/projection.py).

* The by-hand page's worked example 1 is stated with projections (X = I,
  W_Q = sqrt(2) ln3 I, W_K = I, W_V = diag(2, 4)): through them the oracle
  must reproduce the printed O, J = 15/2 and, by eq. A.10.11 of the A.10 page,
  G_X = dQ W_Q^T + dK W_K^T + dV W_V^T from the printed dS and A.
* Central finite differences (by-hand page, section four: float64, two step
  sizes, threshold 1e-7; its own check perturbs the shared input X) on every
  coordinate of X and of W, for self-attention (padded and packed) and for
  cross-attention (X_q and X_kv separately).
* Planted mistakes the differences must catch: a branch that overwrites the
  others instead of adding (the by-hand page warns against exactly this), and
  a branch counted twice in the key/value input of cross-attention (the A.10
  page: each branch that shares an input is summed once).
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import projection as op
from oracle import attention as oa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS = (1e-5, 1e-6)
THRESHOLD = 1e-7


def test_worked_example_through_projections():
    g = json.load(open(os.path.join(GOLDEN, "worked_example_1.json")))
    a = math.sqrt(2) * math.log(3)
    X = np.eye(2)[None]                       # B = 1, n = 2, d_model = 2
    W_Q, W_K, W_V = a * np.eye(2), np.eye(2), np.diag([2.0, 4.0])
    W = np.concatenate([W_Q, W_K, W_V], axis=1)
    G = np.array(g["inputs"]["G"])[None, None]  # [B, H, n, d_v]
    out = op.self_attention_backward(X, W, G, H_q=1, H_kv=1, d_h=2, d_v=2)
    assert np.allclose(out["O"][0, 0], g["printed"]["O"], atol=1e-14)
    assert abs((out["O"][0, 0] * G[0, 0]).sum() - g["printed"]["J"]) < 1e-13
    dS = np.array(g["printed"]["dS"])
    A = np.array(g["printed"]["A"])
    dQ = dS / math.sqrt(2)                    # page: K = I
    dK = math.log(3) * dS.T                   # page: Q = sqrt(2) ln3 I
    dV = A.T @ G[0, 0]
    want_GX = dQ @ W_Q.T + dK @ W_K.T + dV @ W_V.T
    assert np.allclose(out["G_X"][0], want_GX, atol=1e-13)
    # X = I: each weight gradient is its branch's gradient (G_W = X^T G)
    assert np.allclose(out["G_W"], np.concatenate([dQ, dK, dV], axis=1), atol=1e-13)


def _loss_self(X, W, GO, kw):
    o = op.self_attention_backward(X, W, GO, **kw)["O"]
    return float((o * GO).sum())


def _fd(f, arr, analytic):
    worst = 0.0
    for eps in EPS:
        for idx in np.ndindex(arr.shape):
            orig = arr[idx]
            arr[idx] = orig + eps
            lp = f()
            arr[idx] = orig - eps
            lm = f()
            arr[idx] = orig
            worst = max(worst, abs((lp - lm) / (2 * eps) - analytic[idx]))
    return worst


SELF_CASES = [
    dict(name="mha_full", B=1, n=4, d_model=5, H_q=2, H_kv=2, d_h=3, d_v=3, causal=False),
    dict(name="gqa_causal_lens", B=2, n=4, d_model=5, H_q=2, H_kv=1, d_h=3, d_v=2, causal=True,
         seqlens=[4, 3]),
    dict(name="mqa_causal_offset", B=1, n=3, d_model=4, H_q=3, H_kv=1, d_h=2, d_v=3, causal=True, offset=1),
]


def _self_problem(c, seed):
    rng = np.random.default_rng(seed)
    C = c["H_q"] * c["d_h"] + c["H_kv"] * c["d_h"] + c["H_kv"] * c["d_v"]
    X = rng.normal(size=(c["B"], c["n"], c["d_model"]))
    W = rng.normal(size=(c["d_model"], C)) / math.sqrt(c["d_model"])
    GO = rng.normal(size=(c["B"], c["H_q"], c["n"], c["d_v"]))
    kw = dict(H_q=c["H_q"], H_kv=c["H_kv"], d_h=c["d_h"], d_v=c["d_v"], causal=c["causal"],
              offset=c.get("offset", 0), seqlens_q=c.get("seqlens"), seqlens_k=c.get("seqlens"))
    return X, W, GO, kw


@pytest.mark.parametrize("case", SELF_CASES, ids=lambda c: c["name"])
def test_self_attention_finite_differences(case):
    X, W, GO, kw = _self_problem(case, seed=3)
    out = op.self_attention_backward(X, W, GO, **kw)
    f = lambda: _loss_self(X, W, GO, kw)  # noqa: E731
    assert _fd(f, X, out["G_X"]) < THRESHOLD
    assert _fd(f, W, out["G_W"]) < THRESHOLD


def test_self_attention_packed_finite_differences():
    rng = np.random.default_rng(8)
    H_q, H_kv, d_h, d_v, d_model = 2, 1, 3, 2, 4
    cu = [0, 3, 4, 7]
    C = H_q * d_h + H_kv * (d_h + d_v)
    X = rng.normal(size=(7, d_model))
    W = rng.normal(size=(d_model, C)) / 2
    GO = rng.normal(size=(7, H_q, d_v))
    kw = dict(H_q=H_q, H_kv=H_kv, d_h=d_h, d_v=d_v, causal=True, cu_seqlens=cu)
    out = op.self_attention_backward(X, W, GO, **kw)
    f = lambda: float((op.self_attention_backward(X, W, GO, **kw)["O"] * GO).sum())  # noqa: E731
    assert _fd(f, X, out["G_X"]) < THRESHOLD
    assert _fd(f, W, out["G_W"]) < THRESHOLD
    # each packed sequence equals its own padded problem
    for b in range(3):
        rows = slice(cu[b], cu[b + 1])
        ob = op.self_attention_backward(X[rows][None], W, GO[rows].transpose(1, 0, 2)[None], H_q=H_q, H_kv=H_kv,
                                        d_h=d_h, d_v=d_v, causal=True)
        assert np.allclose(ob["O"][0].transpose(1, 0, 2), out["O"][rows], atol=1e-14)
        assert np.allclose(ob["G_X"][0], out["G_X"][rows], atol=1e-14)


def _cross_problem(seed, causal=False):
    rng = np.random.default_rng(seed)
    B, n_q, n_k, d_q, d_kv, H_q, H_kv, d_h, d_v = 2, 3, 5, 4, 3, 2, 1, 3, 2
    Xq = rng.normal(size=(B, n_q, d_q))
    Xkv = rng.normal(size=(B, n_k, d_kv))
    Wq = rng.normal(size=(d_q, H_q * d_h)) / 2
    Wkv = rng.normal(size=(d_kv, H_kv * (d_h + d_v))) / 2
    GO = rng.normal(size=(B, H_q, n_q, d_v))
    kw = dict(H_q=H_q, H_kv=H_kv, d_h=d_h, d_v=d_v, causal=causal, offset=2 if causal else 0,
              seqlens_k=[5, 4])
    return Xq, Xkv, Wq, Wkv, GO, kw


@pytest.mark.parametrize("causal", [False, True])
def test_cross_attention_finite_differences(causal):
    Xq, Xkv, Wq, Wkv, GO, kw = _cross_problem(5, causal)
    out = op.cross_attention_backward(Xq, Xkv, Wq, Wkv, GO, **kw)
    f = lambda: float((op.cross_attention_backward(Xq, Xkv, Wq, Wkv, GO, **kw)["O"] * GO).sum())  # noqa: E731
    for arr, g in ((Xq, "G_Xq"), (Xkv, "G_Xkv"), (Wq, "G_Wq"), (Wkv, "G_Wkv")):
        assert _fd(f, arr, out[g]) < THRESHOLD, g


def test_projection_equals_plain_attention_on_projected_inputs():
    """Projections only feed the core: O and the head gradients equal the
    core's on Q = X W_Q, K = X W_K, V = X W_V (eq. A.10.10)."""
    X, W, GO, kw = _self_problem(SELF_CASES[1], seed=11)
    out = op.self_attention_backward(X, W, GO, **kw)
    W_Q, W_K, W_V = op.split_qkv_weight(W, kw["H_q"], kw["H_kv"], kw["d_h"], kw["d_v"])
    Q = op.to_heads(X @ W_Q, kw["H_q"], kw["d_h"])
    K = op.to_heads(X @ W_K, kw["H_kv"], kw["d_h"])
    V = op.to_heads(X @ W_V, kw["H_kv"], kw["d_v"])
    ref = oa.attention_backward(Q, K, V, GO, causal=kw["causal"], seqlens_q=kw["seqlens_q"],
                                seqlens_k=kw["seqlens_k"])
    for name in ("O", "lse", "GQ", "GK", "GV"):
        assert np.array_equal(out[name], ref[name])
    assert np.array_equal(op.from_heads(op.to_heads(X @ W_Q, kw["H_q"], kw["d_h"])), X @ W_Q)


# ---------------------------------------------------------------- planted mistakes

def test_branch_overwrite_is_caught():
    """G_X from the last branch only (overwriting the first two) fails the
    finite differences."""
    X, W, GO, kw = _self_problem(SELF_CASES[0], seed=4)
    out = op.self_attention_backward(X, W, GO, **kw)
    W_Q, W_K, W_V = op.split_qkv_weight(W, kw["H_q"], kw["H_kv"], kw["d_h"], kw["d_v"])
    GPV = op.from_heads(out["GV"]).reshape(-1, W_V.shape[1])
    wrong = (GPV @ W_V.T).reshape(X.shape)
    f = lambda: _loss_self(X, W, GO, kw)  # noqa: E731
    assert _fd(f, X, wrong) > 1e-3


def test_cross_branch_counted_twice_is_caught():
    """G_Xkv with its key branch added a second time fails the differences."""
    Xq, Xkv, Wq, Wkv, GO, kw = _cross_problem(6)
    out = op.cross_attention_backward(Xq, Xkv, Wq, Wkv, GO, **kw)
    W_K = Wkv[:, :kw["H_kv"] * kw["d_h"]]
    GPK = op.from_heads(out["GK"]).reshape(-1, W_K.shape[1])
    wrong = out["G_Xkv"] + (GPK @ W_K.T).reshape(Xkv.shape)
    f = lambda: float((op.cross_attention_backward(Xq, Xkv, Wq, Wkv, GO, **kw)["O"] * GO).sum())  # noqa: E731
    assert _fd(f, Xkv, wrong) > 1e-3


def test_cross_query_branch_alone_in_query_input():
    """For cross-attention the query input receives only the query branch:
    changing the key/value input's weights leaves the formula G_Q W_Q^T
    (its value changes only through G_Q)."""
    Xq, Xkv, Wq, Wkv, GO, kw = _cross_problem(9)
    out = op.cross_attention_backward(Xq, Xkv, Wq, Wkv, GO, **kw)
    GPQ = op.from_heads(out["GQ"]).reshape(-1, Wq.shape[1])
    assert np.array_equal(out["G_Xq"], (GPQ @ Wq.T).reshape(Xq.shape))
