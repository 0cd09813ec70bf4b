"""Pins of the float64 oracle to what the pages and the mathematics fix.

Each test names the passage it follows.  None of them compares the oracle with
a retyped copy of its own formulas: they use printed values of the worked
examples (tests/golden/), closed forms, invariants, a second independent
implementation, torch's float64 autograd of a library attention routine, and
the structural zeros the definitions imply.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as oa
from oracle.tiny import attention_tiny

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
A_WE = math.sqrt(2.0) * math.log(3.0)


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bhnd(x):
    """2-D matrix -> [1, 1, n, d] float64."""
    return np.asarray(x, dtype=np.float64)[None, None]


def run_example(K):
    Q = A_WE * np.eye(2)
    V = np.diag([2.0, 4.0])
    G = np.array([[1.0, 0.0], [0.0, 2.0]])
    out = oracle.attention_backward(bhnd(Q), bhnd(K), bhnd(V), bhnd(G), keep=True)
    return Q, V, G, out


# ---------------------------------------------------------------------------
# worked examples printed on the by-hand page
# ---------------------------------------------------------------------------

def test_worked_example_1_forward():
    """by-hand page, worked example 1: A, O and the probe J as printed."""
    gold = load("worked_example_1.json")["printed"]
    K = np.eye(2)
    _, _, G, out = run_example(K)
    A = out["A"][0]
    O = out["O"][0, 0]
    np.testing.assert_allclose(out["S"][0], math.log(3.0) * np.eye(2), atol=1e-15)
    np.testing.assert_allclose(A, gold["A"], atol=1e-14)
    np.testing.assert_allclose(O, gold["O"], atol=1e-14)
    J = float((O * G).sum())
    assert abs(J - gold["J"]) < 1e-12
    # lse closed form: row softmax denominators exp(ln3)+exp(0) = 4
    np.testing.assert_allclose(out["lse"][0, 0], [math.log(4.0)] * 2, atol=1e-15)


def test_worked_example_1_backward():
    """by-hand page, section three: dA, the row weighted means, dS, and the
    stated relations dQ = dS/sqrt(2), dK = ln3 dS^T, dV = A^T G."""
    gold = load("worked_example_1.json")["printed"]
    K = np.eye(2)
    _, _, G, out = run_example(K)
    GS = out["GS"][0]
    np.testing.assert_allclose(GS, gold["dS"], atol=1e-14)
    np.testing.assert_allclose(out["c"][0, 0], gold["row_weighted_means_c"], atol=1e-14)
    dS = np.array(gold["dS"])
    np.testing.assert_allclose(out["GQ"][0, 0], dS / math.sqrt(2.0), atol=1e-14)
    np.testing.assert_allclose(out["GK"][0, 0], math.log(3.0) * dS.T, atol=1e-14)
    A = np.array(gold["A"])
    np.testing.assert_allclose(out["GV"][0, 0], A.T @ G, atol=1e-14)
    # dA = G V^T as printed
    V = np.diag([2.0, 4.0])
    np.testing.assert_allclose(G @ V.T, gold["dA"], atol=0)


def test_worked_example_2_identical_keys():
    """by-hand page, worked example 2: identical keys give A = 1/2, O = [1,2] in
    both rows exactly, J = 5, dS as printed, dQ = 0 and dK != 0."""
    gold = load("worked_example_2_identical_keys.json")["printed"]
    K = np.ones((2, 2))
    _, _, G, out = run_example(K)
    np.testing.assert_allclose(out["A"][0], gold["A"], atol=1e-15)
    assert np.array_equal(out["O"][0, 0], np.array(gold["O"]))  # exact, as the page asserts
    assert abs(float((out["O"][0, 0] * G).sum()) - gold["J"]) < 1e-12
    np.testing.assert_allclose(out["c"][0, 0], gold["row_weighted_means_c"], atol=1e-14)
    np.testing.assert_allclose(out["GS"][0], gold["dS"], atol=1e-14)
    assert np.abs(out["GQ"][0, 0]).max() < 1e-12
    assert np.abs(out["GK"][0, 0]).max() > 0.1
    np.testing.assert_allclose(out["lse"][0, 0], [math.log(6.0)] * 2, atol=1e-15)


def test_transpose_check():
    """by-hand page, section one: for the non-symmetric pair the score matrix is
    Q K^T = [[1,4],[0,1]] (times 1/sqrt(2)), not Q K = [[5,2],[2,1]]."""
    gold = load("transpose_check.json")
    Q = np.array(gold["inputs"]["Q"])
    K = np.array(gold["inputs"]["K"])
    V = np.eye(2)
    out = oracle.attention_forward(bhnd(Q), bhnd(K), bhnd(V), keep=True)
    S = out["S"][0] * math.sqrt(2.0)
    np.testing.assert_allclose(S, gold["printed"]["QKt"], atol=1e-14)
    assert not np.allclose(S, gold["printed"]["QK_wrong"])


def test_two_position_jacobian():
    """by-hand page, worked example 2 discussion: for row weights [a, 1-a] and
    upstream weight gradient [u, v], dS = a(1-a)(u-v) * [1, -1]; zero when u = v."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        s = rng.normal(size=2)
        vrow = rng.normal(size=(2, 3))
        go = rng.normal(size=3)
        # one query row, keys chosen so that S = s exactly: q = s*sqrt(d), K = I
        d = 2
        q = (s * math.sqrt(d))[None, :]
        k = np.eye(2)
        out = oracle.attention_backward(q[None, None], k[None, None], vrow[None, None],
                                        go[None, None, None], keep=True)
        a = out["A"][0][0, 0]
        u, v = vrow @ go
        expect = a * (1 - a) * (u - v)
        np.testing.assert_allclose(out["GS"][0][0], [expect, -expect], atol=1e-14)
    # u == v: both derivatives vanish
    vrow = np.array([[1.0, 2.0], [1.0, 2.0]])
    out = oracle.attention_backward(np.array([[[[0.3, -1.2]]]]), np.eye(2)[None, None],
                                    vrow[None, None], np.array([[[[0.7, 0.1]]]]), keep=True)
    assert np.abs(out["GS"][0]).max() < 1e-15


# ---------------------------------------------------------------------------
# invariants of the definition
# ---------------------------------------------------------------------------

MASK_CASES = [
    dict(name="full", n_q=5, n_k=7, causal=False, offset=0, lq=None, lk=None),
    dict(name="causal", n_q=6, n_k=6, causal=True, offset=0, lq=None, lk=None),
    dict(name="causal_off2", n_q=4, n_k=7, causal=True, offset=2, lq=None, lk=None),
    dict(name="keypad", n_q=5, n_k=7, causal=False, offset=0, lq=None, lk=[7, 3]),
    dict(name="rowpad_causal", n_q=6, n_k=6, causal=True, offset=0, lq=[6, 4], lk=[6, 4]),
    dict(name="nonsquare_offset_pad", n_q=3, n_k=9, causal=True, offset=5, lq=[3, 2], lk=[9, 6]),
    # one causal offset per sequence (each sequence's own cached history)
    dict(name="per_sequence_offsets", n_q=4, n_k=8, causal=True, offset=[1, 4], lq=None, lk=[8, 6]),
]


def random_problem(case, H_q=4, H_kv=2, d_h=4, d_v=3, seed=0, B=2):
    rng = np.random.default_rng(seed)
    Q = rng.normal(size=(B, H_q, case["n_q"], d_h))
    K = rng.normal(size=(B, H_kv, case["n_k"], d_h))
    V = rng.normal(size=(B, H_kv, case["n_k"], d_v))
    GO = rng.normal(size=(B, H_q, case["n_q"], d_v))
    kw = dict(causal=case["causal"], offset=case["offset"],
              seqlens_q=case["lq"], seqlens_k=case["lk"])
    return Q, K, V, GO, kw


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: c["name"])
def test_invariants(case):
    """A rows non-negative and summing to 1 on active rows, zero off the visible
    set ([A.10, sec. A.10.1]); O inside the convex hull of visible V rows
    (by-hand page, worked example 1 discussion); G_S rows sum to 0 and vanish
    off the visible set ([A.10, eq. A.10.7] and the shift invariance after it);
    c_i equals rowsum(G_O * O)."""
    Q, K, V, GO, kw = random_problem(case)
    out = oracle.attention_backward(Q, K, V, GO, keep=True, **kw)
    B, H_q = Q.shape[:2]
    H_kv = K.shape[1]
    for idx, (A, GS, M) in enumerate(zip(out["A"], out["GS"], out["M"])):
        b, r = divmod(idx, H_q)
        g = oracle.kv_group(r, H_q, H_kv)
        active = M.any(axis=1)
        assert (A >= 0).all()
        np.testing.assert_allclose(A[active].sum(axis=1), 1.0, atol=1e-13)
        assert (A[~M] == 0).all()
        assert (GS[~M] == 0).all()
        np.testing.assert_allclose(GS.sum(axis=1), 0.0, atol=1e-13)
        O = out["O"][b, r]
        for i in np.nonzero(active)[0]:
            vis = V[b, g][M[i]]
            assert (O[i] <= vis.max(axis=0) + 1e-12).all()
            assert (O[i] >= vis.min(axis=0) - 1e-12).all()
        # inactive rows: exact zeros
        assert (O[~active] == 0).all() and (out["lse"][b, r][~active] == 0).all()
        assert (out["GQ"][b, r][~active] == 0).all()
    np.testing.assert_allclose(out["c"], out["D"], atol=1e-12)


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: c["name"])
def test_matches_pure_python_oracle(case):
    """The numpy oracle and the independent pure-Python one agree to 1e-13."""
    Q, K, V, GO, kw = random_problem(case, seed=3)
    a = oracle.attention_backward(Q, K, V, GO, **kw)
    t = attention_tiny(Q.tolist(), K.tolist(), V.tolist(), GO.tolist(), kw["causal"],
                       kw["offset"], kw["seqlens_q"], kw["seqlens_k"])
    for key in ("O", "lse", "GQ", "GK", "GV"):
        np.testing.assert_allclose(a[key], np.array(t[key]), atol=1e-13, rtol=0, err_msg=key)


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: c["name"])
def test_matches_torch_autograd(case):
    """Library-routine pin: torch's float64 scaled_dot_product_attention with a
    boolean mask (K/V repeated per query-head group) and its autograd gradients.
    Only problems whose rows are all active are compared (torch has no notion
    of an inactive padding row)."""
    torch = pytest.importorskip("torch")
    if case["lq"] is not None:
        pytest.skip("torch SDPA defines no inactive rows")
    Q, K, V, GO, kw = random_problem(case, seed=4)
    out = oracle.attention_backward(Q, K, V, GO, **kw)
    B, H_q, n_q, _ = Q.shape
    H_kv, n_k = K.shape[1], K.shape[2]
    grp = H_q // H_kv
    q = torch.tensor(Q, requires_grad=True)
    k = torch.tensor(K, requires_grad=True)
    v = torch.tensor(V, requires_grad=True)
    mask = torch.zeros(B, 1, n_q, n_k, dtype=torch.bool)
    lk = kw["seqlens_k"] or [n_k] * B
    offs = kw["offset"] if isinstance(kw["offset"], list) else [kw["offset"]] * B
    for b in range(B):
        i = torch.arange(n_q)[:, None]
        j = torch.arange(n_k)[None, :]
        m = j < lk[b]
        if kw["causal"]:
            m = m & (j <= i + offs[b])
        mask[b, 0] = m
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(grp, dim=1), v.repeat_interleave(grp, dim=1), attn_mask=mask)
    o.backward(torch.tensor(GO))
    np.testing.assert_allclose(out["O"], o.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(out["GQ"], q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(out["GK"], k.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(out["GV"], v.grad.numpy(), atol=1e-12)


def test_causal_first_row_loss_zero_future_gradients():
    """Chapter 31, sec. 6: with only the first output row in the loss of a causal
    problem, keys/values after the visible prefix receive exactly zero gradient."""
    rng = np.random.default_rng(11)
    for off in (0, 2):
        Q = rng.normal(size=(1, 2, 5, 4))
        K = rng.normal(size=(1, 1, 8, 4))
        V = rng.normal(size=(1, 1, 8, 3))
        GO = np.zeros((1, 2, 5, 3))
        GO[:, :, 0] = rng.normal(size=(1, 2, 3))
        out = oracle.attention_backward(Q, K, V, GO, causal=True, offset=off)
        assert (out["GK"][0, 0, off + 1:] == 0).all()
        assert (out["GV"][0, 0, off + 1:] == 0).all()
        assert np.abs(out["GV"][0, 0, : off + 1]).max() > 0
        # and G_Q of rows outside the loss is zero too
        assert (out["GQ"][0, :, 1:] == 0).all()


def test_special_cases_closed_forms():
    """Closed forms of the definition ([A.10, eqs. A.10.1-A.10.3]):
    Q = 0 gives uniform weights on each visible set, O = mean of visible V rows
    (causal: prefix means) and lse = ln|V_i|; a ones column in V gives an O
    column of ones; a row with one visible key copies that key's value."""
    rng = np.random.default_rng(2)
    n, d = 6, 4
    V = rng.normal(size=(1, 1, n, 3))
    V[..., 2] = 1.0
    K = rng.normal(size=(1, 1, n, d))
    out = oracle.attention_forward(np.zeros((1, 1, n, d)), K, V, causal=True)
    for i in range(n):
        np.testing.assert_allclose(out["O"][0, 0, i], V[0, 0, : i + 1].mean(axis=0), atol=1e-14)
        assert abs(out["lse"][0, 0, i] - math.log(i + 1)) < 1e-14
    Q = rng.normal(size=(1, 1, n, d))
    out = oracle.attention_forward(Q, K, V, causal=True)
    np.testing.assert_allclose(out["O"][0, 0, :, 2], 1.0, atol=1e-14)
    np.testing.assert_allclose(out["O"][0, 0, 0], V[0, 0, 0], atol=1e-15)
    GO = rng.normal(size=(1, 1, n, 3))
    bw = oracle.attention_backward(Q, K, V, GO, causal=True, keep=True)
    assert (bw["GS"][0][0] == 0).all()


def test_gqa_equals_repeated_mha():
    """[A.10, sec. A.10.5]: grouped heads are MHA with K/V repeated per group, and
    the grouped G_K/G_V are the sums of the repeated heads' gradients."""
    rng = np.random.default_rng(8)
    B, H_q, H_kv, n, d = 2, 6, 2, 5, 4
    Q = rng.normal(size=(B, H_q, n, d))
    K = rng.normal(size=(B, H_kv, n, d))
    V = rng.normal(size=(B, H_kv, n, 3))
    GO = rng.normal(size=(B, H_q, n, 3))
    grp = H_q // H_kv
    g = oracle.attention_backward(Q, K, V, GO, causal=True)
    m = oracle.attention_backward(Q, np.repeat(K, grp, axis=1), np.repeat(V, grp, axis=1), GO,
                                  causal=True)
    np.testing.assert_allclose(g["O"], m["O"], atol=1e-14)
    np.testing.assert_allclose(g["GQ"], m["GQ"], atol=1e-14)
    np.testing.assert_allclose(g["GK"], m["GK"].reshape(B, H_kv, grp, n, d).sum(2), atol=1e-13)
    np.testing.assert_allclose(g["GV"], m["GV"].reshape(B, H_kv, grp, n, 3).sum(2), atol=1e-13)
    # MQA is the H_kv = 1 case of the same map
    assert [oracle.kv_group(r, 6, 1) for r in range(6)] == [0] * 6
    assert [oracle.kv_group(r, 8, 2) for r in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]


def test_permutation_equivariance_unmasked():
    """Chapter 15, sec. 15.6: without a mask, permuting query rows permutes output
    rows, and permuting key/value rows jointly leaves the output unchanged.
    The causal mask breaks the second property."""
    rng = np.random.default_rng(9)
    Q = rng.normal(size=(1, 1, 5, 4))
    K = rng.normal(size=(1, 1, 6, 4))
    V = rng.normal(size=(1, 1, 6, 3))
    pq = rng.permutation(5)
    pk = rng.permutation(6)
    base = oracle.attention_forward(Q, K, V)["O"]
    np.testing.assert_allclose(oracle.attention_forward(Q[:, :, pq], K, V)["O"], base[:, :, pq],
                               atol=1e-14)
    np.testing.assert_allclose(oracle.attention_forward(Q, K[:, :, pk], V[:, :, pk])["O"], base,
                               atol=1e-14)
    c1 = oracle.attention_forward(Q, K[:, :, :5], V[:, :, :5], causal=True)["O"]
    c2 = oracle.attention_forward(Q, K[:, :, pk[pk < 5]], V[:, :, pk[pk < 5]], causal=True)["O"]
    assert not np.allclose(c1, c2)


def test_extreme_scores_stay_finite():
    """by-hand page, section four: a separate extreme-score check.  Scores around
    +-1e3 (Q scaled by 100) must give finite O and lse, with near one-hot rows;
    max subtraction ([ch.15, sec. 15.1]) is what makes this work."""
    rng = np.random.default_rng(12)
    Q = 100.0 * rng.normal(size=(1, 2, 8, 16))
    K = rng.normal(size=(1, 2, 8, 16))
    V = rng.normal(size=(1, 2, 8, 5))
    GO = rng.normal(size=(1, 2, 8, 5))
    out = oracle.attention_backward(Q, K, V, GO, causal=True, keep=True)
    for key in ("O", "lse", "GQ", "GK", "GV"):
        assert np.isfinite(out[key]).all(), key
    assert np.mean([A.max(axis=1)[1:].mean() for A in out["A"]]) > 0.9
    np.testing.assert_allclose(out["lse"][0, 0, 0], out["S"][0][0, 0], atol=1e-12)


# ---------------------------------------------------------------------------
# validation: the rejected problems
# ---------------------------------------------------------------------------

def test_validation_errors():
    """Fully masked active rows are rejected ([A.10, sec. A.10.1]; [ch.31, sec. 3]);
    inactive padding rows are not errors."""
    z = np.zeros
    with pytest.raises(oracle.EmptyRow):  # negative causal offset empties row 0
        oracle.attention_forward(z((1, 1, 3, 4)), z((1, 1, 3, 4)), z((1, 1, 3, 4)), causal=True,
                                 offset=-1)
    with pytest.raises(oracle.EmptyRow):  # a sequence with no keys but active rows
        oracle.attention_forward(z((2, 1, 3, 4)), z((2, 1, 3, 4)), z((2, 1, 3, 4)),
                                 seqlens_k=[3, 0])
    with pytest.raises(oracle.EmptyRow):  # no keys at all
        oracle.attention_forward(z((1, 1, 3, 4)), z((1, 1, 0, 4)), z((1, 1, 0, 4)))
    with pytest.raises(oracle.InvalidArgument):
        oracle.attention_forward(z((1, 3, 3, 4)), z((1, 2, 3, 4)), z((1, 2, 3, 4)))
    with pytest.raises(oracle.InvalidArgument):
        oracle.attention_forward(z((1, 1, 3, 4)), z((1, 1, 3, 4)), z((1, 1, 3, 4)),
                                 seqlens_k=[4])
    # a sequence whose rows are all inactive is fine even without keys
    out = oracle.attention_forward(z((2, 1, 3, 4)), z((2, 1, 3, 4)), z((2, 1, 3, 4)),
                                   seqlens_q=[3, 0], seqlens_k=[3, 0])
    assert (out["O"][1] == 0).all()
    # negative offset is fine when rows that would be empty are inactive? no:
    # row 0 is active whenever L_q >= 1, so the offset must be >= 0 then.
    with pytest.raises(oracle.EmptyRow):
        oracle.attention_forward(z((1, 1, 3, 4)), z((1, 1, 5, 4)), z((1, 1, 5, 4)), causal=True,
                                 offset=-2, seqlens_q=[1])
