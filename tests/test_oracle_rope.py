"""Pins of the oracle's rotary position encoding and of attention with it.

"Chapter 15" sec. 15.6 defines RoPE as a 2-D rotation of every column pair of
q_i and k_j by the position times a fixed frequency, so that
R_i^T R_j = R((j - i) omega): scores depend on the position difference only.
"Chapter 31" sec. 5: the rotation is orthogonal and its backward is the
transposed rotation of the upstream gradient.  Pins: that relative-position
identity, orthogonality, explicit 2x2 matrices, a quarter turn, the zero-angle
table (reduces to plain attention), and central finite differences on every
coordinate (by-hand page, section four).
"""

import math

import numpy as np
import pytest

import oracle

EPS = (1e-5, 1e-6)
THRESHOLD = 1e-7


def test_scores_depend_on_position_difference_only():
    rng = np.random.default_rng(0)
    d = 8
    table = oracle.rope_table(64, d).astype(np.float64)
    q = rng.normal(size=(1, d))
    k = rng.normal(size=(1, d))
    for (i, j, c) in [(3, 7, 11), (10, 2, 25), (0, 0, 40)]:
        s0 = (oracle.rope_rotate(q, table, [i]) @ oracle.rope_rotate(k, table, [j]).T).item()
        s1 = (oracle.rope_rotate(q, table, [i + c]) @ oracle.rope_rotate(k, table, [j + c]).T).item()
        # the float32-rounded table is not exactly cos/sin of integer multiples,
        # so the identity holds to the table's rounding
        assert abs(s0 - s1) < 1e-5 * (1 + abs(s0))


def test_exact_relative_identity_with_exact_angles():
    """With angles computed in float64 the identity holds to rounding."""
    d, n = 6, 50
    omega = np.array([1.0, 0.1, 0.01])
    theta = np.arange(n)[:, None] * omega[None, :]
    table = np.stack([np.cos(theta), np.sin(theta)], axis=-1)
    rng = np.random.default_rng(1)
    q, k = rng.normal(size=(1, d)), rng.normal(size=(1, d))
    s0 = (oracle.rope_rotate(q, table, [4]) @ oracle.rope_rotate(k, table, [9]).T).item()
    s1 = (oracle.rope_rotate(q, table, [30]) @ oracle.rope_rotate(k, table, [35]).T).item()
    assert abs(s0 - s1) < 1e-12


def test_rotation_is_orthogonal_and_matches_explicit_matrices():
    rng = np.random.default_rng(2)
    d, n = 8, 5
    table = oracle.rope_table(n, d).astype(np.float64)
    X = rng.normal(size=(3, n, d))
    pos = np.arange(n)
    Y = oracle.rope_rotate(X, table, pos)
    np.testing.assert_allclose(oracle.rope_rotate(Y, table, pos, inverse=True), X, atol=1e-14)
    # explicit 2x2 rotation matrices acting on column vectors (x_2k, x_2k+1)
    for h in range(3):
        for i in range(n):
            for kk in range(d // 2):
                c, s = table[i, kk]
                R = np.array([[c, -s], [s, c]])
                np.testing.assert_allclose(Y[h, i, 2 * kk:2 * kk + 2], R @ X[h, i, 2 * kk:2 * kk + 2], atol=1e-14)
    # each pair keeps its length
    np.testing.assert_allclose(np.hypot(Y[..., 0::2], Y[..., 1::2]), np.hypot(X[..., 0::2], X[..., 1::2]),
                               atol=1e-14)


def test_quarter_turn():
    table = np.zeros((2, 1, 2))
    table[0] = (1.0, 0.0)
    table[1] = (0.0, 1.0)   # theta = pi/2 at position 1
    X = np.array([[3.0, 5.0], [3.0, 5.0]])
    Y = oracle.rope_rotate(X, table, [0, 1])
    np.testing.assert_array_equal(Y, [[3.0, 5.0], [-5.0, 3.0]])


def test_zero_angles_reduce_to_plain_attention():
    rng = np.random.default_rng(3)
    B, Hq, Hk, nq, nk, d = 2, 4, 2, 5, 7, 4
    Q = rng.normal(size=(B, Hq, nq, d))
    K = rng.normal(size=(B, Hk, nk, d))
    V = rng.normal(size=(B, Hk, nk, 3))
    GO = rng.normal(size=(B, Hq, nq, 3))
    table = np.zeros((20, d // 2, 2))
    table[..., 0] = 1.0
    kw = dict(causal=True, offset=[2, 1], seqlens_k=[7, 4])
    a = oracle.attention_backward_rope(Q, K, V, GO, table, **kw)
    b = oracle.attention_backward(Q, K, V, GO, **kw)
    for key in ("O", "lse", "GQ", "GK", "GV"):
        np.testing.assert_array_equal(a[key], b[key])


@pytest.mark.parametrize("kw", [dict(causal=False, offset=0), dict(causal=True, offset=[1, 3], seqlens_k=[6, 5])],
                         ids=["full", "causal_per_seq_offsets"])
def test_rope_attention_finite_differences(kw):
    rng = np.random.default_rng(4)
    B, Hq, Hk, nq, nk, d, dv = 2, 2, 1, 3, 6, 4, 2
    Q = rng.normal(size=(B, Hq, nq, d))
    K = rng.normal(size=(B, Hk, nk, d))
    V = rng.normal(size=(B, Hk, nk, dv))
    GO = rng.normal(size=(B, Hq, nq, dv))
    table = oracle.rope_table(16, d, base=3.0).astype(np.float64)
    out = oracle.attention_backward_rope(Q, K, V, GO, table, **kw)

    def loss():
        return float((oracle.attention_backward_rope(Q, K, V, None, table, **kw)["O"] * GO).sum())

    worst = 0.0
    for eps in EPS:
        for X, G in ((Q, out["GQ"]), (K, out["GK"]), (V, out["GV"])):
            for idx in np.ndindex(X.shape):
                orig = X[idx]
                X[idx] = orig + eps
                lp = loss()
                X[idx] = orig - eps
                lm = loss()
                X[idx] = orig
                worst = max(worst, abs((lp - lm) / (2 * eps) - G[idx]))
    assert worst < THRESHOLD


def test_table_is_the_geometric_one():
    t = oracle.rope_table(3, 4, base=100.0).astype(np.float64)
    # omega = (1, 100^-0.5 = 0.1); position 2
    np.testing.assert_allclose(t[2, 0], [math.cos(2.0), math.sin(2.0)], rtol=1e-7)
    np.testing.assert_allclose(t[2, 1], [math.cos(0.2), math.sin(0.2)], rtol=1e-7)
