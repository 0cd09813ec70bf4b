"""Pins of the oracle's packed ("varlen") layout and per-sequence causal
offsets.

The packed layout stores the sequences' rows one after another with no
padding; sequence b is the padded definition restricted to its own rows
("Appendix A.10", sec. A.10.6: padding positions are simply not in the
visible sets).  Pins: the identity with the padded layout plus per-sequence
lengths, an independent pure-Python implementation that indexes the packed
rows directly, the absence of any coupling between sequences, and central
finite differences on every coordinate (by-hand page, section four;
chapter 31, sec. 6).
"""

import numpy as np
import pytest

import oracle
from oracle import attention as oa
from oracle.tiny import attention_tiny_packed

EPS = (1e-5, 1e-6)
THRESHOLD = 1e-7

# (L_q per sequence, L_k per sequence, causal, offset) -- includes an empty
# sequence, a sequence with more queries than keys (offset makes it valid)
# and per-sequence offsets
CASES = [
    dict(name="full", lq=[3, 5, 2], lk=[4, 6, 3], causal=False, offset=0),
    dict(name="causal", lq=[3, 5, 4], lk=[3, 5, 4], causal=True, offset=0),
    dict(name="causal_per_seq_offsets", lq=[2, 4, 3], lk=[5, 4, 7], causal=True, offset=[3, 0, 4]),
    dict(name="empty_sequence", lq=[3, 0, 2], lk=[3, 0, 4], causal=True, offset=[0, 0, 2]),
]


def packed_problem(case, H_q=4, H_kv=2, d_h=4, d_v=3, seed=0):
    rng = np.random.default_rng(seed)
    cu_q = np.concatenate([[0], np.cumsum(case["lq"])]).astype(int).tolist()
    cu_k = np.concatenate([[0], np.cumsum(case["lk"])]).astype(int).tolist()
    Q = rng.normal(size=(cu_q[-1], H_q, d_h))
    K = rng.normal(size=(cu_k[-1], H_kv, d_h))
    V = rng.normal(size=(cu_k[-1], H_kv, d_v))
    GO = rng.normal(size=(cu_q[-1], H_q, d_v))
    return Q, K, V, GO, cu_q, cu_k


def to_padded(X, cu, n):
    """[rows, H, d] packed -> [B, H, n, d] zero-padded."""
    B = len(cu) - 1
    out = np.zeros((B, X.shape[1], n, X.shape[2]))
    for b in range(B):
        L = cu[b + 1] - cu[b]
        out[b, :, :L] = X[cu[b]:cu[b + 1]].transpose(1, 0, 2)
    return out


@pytest.mark.parametrize("case", CASES, ids=lambda c: c["name"])
def test_packed_equals_padded_with_lengths(case):
    Q, K, V, GO, cu_q, cu_k = packed_problem(case, seed=1)
    kw = dict(causal=case["causal"], offset=case["offset"])
    pk = oracle.attention_backward_packed(Q, K, V, GO, cu_q, cu_k, **kw)
    n_q, n_k = max(case["lq"]), max(case["lk"])
    pad = oracle.attention_backward(to_padded(Q, cu_q, n_q), to_padded(K, cu_k, n_k),
                                    to_padded(V, cu_k, n_k), to_padded(GO, cu_q, n_q),
                                    seqlens_q=case["lq"], seqlens_k=case["lk"], **kw)
    np.testing.assert_array_equal(to_padded(pk["O"], cu_q, n_q), pad["O"])
    np.testing.assert_array_equal(to_padded(pk["GQ"], cu_q, n_q), pad["GQ"])
    np.testing.assert_array_equal(to_padded(pk["GK"], cu_k, n_k), pad["GK"])
    np.testing.assert_array_equal(to_padded(pk["GV"], cu_k, n_k), pad["GV"])
    for b in range(len(case["lq"])):
        L = case["lq"][b]
        np.testing.assert_array_equal(pk["lse"][:, cu_q[b]:cu_q[b] + L], pad["lse"][b, :, :L])
        np.testing.assert_array_equal(pk["D"][:, cu_q[b]:cu_q[b] + L], pad["D"][b, :, :L])


@pytest.mark.parametrize("case", CASES, ids=lambda c: c["name"])
def test_packed_matches_pure_python(case):
    Q, K, V, GO, cu_q, cu_k = packed_problem(case, seed=2)
    kw = dict(causal=case["causal"], offset=case["offset"])
    a = oracle.attention_backward_packed(Q, K, V, GO, cu_q, cu_k, **kw)
    t = attention_tiny_packed(Q.tolist(), K.tolist(), V.tolist(), GO.tolist(), cu_q, cu_k, **kw)
    for key in ("O", "lse", "GQ", "GK", "GV"):
        np.testing.assert_allclose(a[key], np.array(t[key]), atol=1e-13, rtol=0, err_msg=key)


def test_sequences_do_not_interact():
    """Changing every input row of one sequence leaves every output row of the
    others bit-identical."""
    case = CASES[2]
    Q, K, V, GO, cu_q, cu_k = packed_problem(case, seed=3)
    kw = dict(causal=case["causal"], offset=case["offset"])
    a = oracle.attention_backward_packed(Q, K, V, GO, cu_q, cu_k, **kw)
    rng = np.random.default_rng(9)
    Q2, K2, V2, GO2 = Q.copy(), K.copy(), V.copy(), GO.copy()
    sq, sk = slice(cu_q[1], cu_q[2]), slice(cu_k[1], cu_k[2])
    Q2[sq] = rng.normal(size=Q2[sq].shape)
    K2[sk] = rng.normal(size=K2[sk].shape)
    V2[sk] = rng.normal(size=V2[sk].shape)
    GO2[sq] = rng.normal(size=GO2[sq].shape)
    b = oracle.attention_backward_packed(Q2, K2, V2, GO2, cu_q, cu_k, **kw)
    keep_q = np.r_[cu_q[0]:cu_q[1], cu_q[2]:cu_q[3]]
    keep_k = np.r_[cu_k[0]:cu_k[1], cu_k[2]:cu_k[3]]
    for key in ("O", "GQ"):
        np.testing.assert_array_equal(a[key][keep_q], b[key][keep_q])
    for key in ("GK", "GV"):
        np.testing.assert_array_equal(a[key][keep_k], b[key][keep_k])
    np.testing.assert_array_equal(a["lse"][:, keep_q], b["lse"][:, keep_q])
    assert not np.array_equal(a["O"][sq], b["O"][sq])


def test_per_sequence_offsets_equal_separate_problems():
    """A batch with one offset per sequence equals each sequence run alone with
    its own scalar offset."""
    case = CASES[2]
    Q, K, V, GO, cu_q, cu_k = packed_problem(case, seed=4)
    a = oracle.attention_backward_packed(Q, K, V, GO, cu_q, cu_k, causal=True, offset=case["offset"])
    for b, off in enumerate(case["offset"]):
        sq, sk = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        one = oracle.attention_backward_packed(Q[sq], K[sk], V[sk], GO[sq], [0, sq.stop - sq.start],
                                               [0, sk.stop - sk.start], causal=True, offset=off)
        np.testing.assert_array_equal(a["O"][sq], one["O"])
        np.testing.assert_array_equal(a["GK"][sk], one["GK"])


@pytest.mark.parametrize("case", CASES[2:3], ids=lambda c: c["name"])
def test_packed_finite_differences(case):
    Q, K, V, GO, cu_q, cu_k = packed_problem(case, H_q=2, H_kv=1, d_h=3, d_v=2, seed=5)
    kw = dict(causal=case["causal"], offset=case["offset"])
    out = oracle.attention_backward_packed(Q, K, V, GO, cu_q, cu_k, **kw)

    def loss(Qx, Kx, Vx):
        return float((oracle.attention_backward_packed(Qx, Kx, Vx, None, cu_q, cu_k, **kw)["O"] * GO).sum())

    worst = 0.0
    for eps in EPS:
        for name, X, G in (("Q", Q, out["GQ"]), ("K", K, out["GK"]), ("V", V, out["GV"])):
            for idx in np.ndindex(X.shape):
                orig = X[idx]
                X[idx] = orig + eps
                lp = loss(Q, K, V)
                X[idx] = orig - eps
                lm = loss(Q, K, V)
                X[idx] = orig
                worst = max(worst, abs((lp - lm) / (2 * eps) - G[idx]))
    assert worst < THRESHOLD


def test_packed_validation():
    Q, K, V, GO, cu_q, cu_k = packed_problem(CASES[0])
    with pytest.raises(oracle.InvalidArgument):
        oracle.attention_backward_packed(Q, K, V, GO, [1, 3, 8, 10], cu_k)
    with pytest.raises(oracle.InvalidArgument):
        oracle.attention_backward_packed(Q, K, V, GO, [0, 3, 2, 10], cu_k)
    with pytest.raises(oracle.EmptyRow):  # active rows of the second sequence, no keys
        oracle.attention_backward_packed(Q, K, V, GO, cu_q, [0, 4, 4, 7])
    with pytest.raises(oracle.EmptyRow):  # negative per-sequence offset
        oracle.attention_backward_packed(Q, K, V, GO, cu_q, cu_k, causal=True, offset=[0, -1, 0])
