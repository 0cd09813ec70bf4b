"""Pin of oracle.attention_group, the per-(sequence, KV head) restriction of the
oracle through which the full-size GPU checks run.

"Appendix A.10 - Attention matrices and backpropagation" (glenzli.com),
sec. A.10.5: the query heads that share a KV head each run the ordinary
single-head computation on that KV head's K and V, and the KV head's G_K and
G_V are the sums of their contributions.  attention_group must therefore be
exactly the slice of the whole-batch oracle (attention_backward, itself pinned
by the worked examples, finite differences and torch autograd) that belongs
to sequence b and KV head g: O, lse, G_Q and D of the group's query heads and
G_K, G_V of the KV head.  The shapes use grouped heads, per-sequence lengths
and per-sequence causal offsets, so a wrong head selection, a wrong
sequence's offset or length, or a D taken from the wrong head fails.

Planted mistakes (in the oracle, on the CPU) check that the pin has teeth:
an interleaved head map instead of contiguous groups, and every sequence
reading the next sequence's offset.  The whole-batch reference is computed
before the mistake is planted, so only attention_group sees it.
"""

import numpy as np
import pytest

import oracle
from oracle import attention as oa

B, H_Q, H_KV, N_Q, N_K, D_H, D_V = 3, 8, 2, 23, 31, 8, 6
LENS_Q = [23, 17, 9]
LENS_K = [31, 20, 28]
OFFSETS = [8, 3, 19]  # per sequence: each row sees keys j <= i + offset_b


def _inputs(seed=11):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, H_Q, N_Q, D_H))
    K = rng.standard_normal((B, H_KV, N_K, D_H))
    V = rng.standard_normal((B, H_KV, N_K, D_V))
    GO = rng.standard_normal((B, H_Q, N_Q, D_V))
    return Q, K, V, GO


CASES = {
    "causal_per_sequence_offsets": dict(causal=True, offset=OFFSETS, seqlens_q=LENS_Q, seqlens_k=LENS_K),
    "padding_only": dict(causal=False, offset=0, seqlens_q=LENS_Q, seqlens_k=LENS_K),
    "causal_one_offset": dict(causal=True, offset=4, seqlens_q=None, seqlens_k=LENS_K),
}


def _group_errors(Q, K, V, GO, full, kw):
    """Largest absolute difference of every group's outputs from the slices of
    the whole-batch result."""
    worst = 0.0
    group = H_Q // H_KV
    for b in range(B):
        for g in range(H_KV):
            o = oracle.attention_group(Q, K, V, GO, b, g, **kw)
            heads = list(range(g * group, (g + 1) * group))
            pairs = [(o["O"], full["O"][b, heads]), (o["lse"], full["lse"][b, heads]),
                     (o["GQ"], full["GQ"][b, heads]), (o["D"], full["D"][b, heads]),
                     (o["GK"], full["GK"][b, g]), (o["GV"], full["GV"][b, g])]
            for got, ref in pairs:
                if got.shape != ref.shape:
                    return np.inf
                worst = max(worst, float(np.max(np.abs(got - ref))))
    return worst


@pytest.mark.parametrize("case", sorted(CASES))
def test_group_equals_slices_of_whole_batch(case):
    kw = CASES[case]
    Q, K, V, GO = _inputs()
    full = oracle.attention_backward(Q, K, V, GO, **kw)
    # the group's heads are the contiguous block r // (H_q / H_kv) == g
    o = oracle.attention_group(Q, K, V, GO, 1, 1, **kw)
    assert o["heads"] == [4, 5, 6, 7]
    assert _group_errors(Q, K, V, GO, full, kw) < 1e-12


def test_group_sums_gradients_over_its_heads():
    """sec. A.10.5: G_K / G_V of the group are the sums of the single-head
    gradients of its query heads (each head run alone as an MHA problem on
    the shared K, V)."""
    kw = CASES["causal_per_sequence_offsets"]
    Q, K, V, GO = _inputs(5)
    b, g = 2, 0
    o = oracle.attention_group(Q, K, V, GO, b, g, **kw)
    GK = np.zeros((N_K, D_H))
    GV = np.zeros((N_K, D_V))
    for r in o["heads"]:
        one = oracle.attention_backward(Q[b:b + 1, r:r + 1], K[b:b + 1, g:g + 1], V[b:b + 1, g:g + 1],
                                        GO[b:b + 1, r:r + 1], causal=True, offset=OFFSETS[b],
                                        seqlens_q=[LENS_Q[b]], seqlens_k=[LENS_K[b]])
        GK += one["GK"][0, 0]
        GV += one["GV"][0, 0]
    np.testing.assert_allclose(o["GK"], GK, atol=1e-12)
    np.testing.assert_allclose(o["GV"], GV, atol=1e-12)


def test_planted_interleaved_head_map_fails(monkeypatch):
    kw = CASES["causal_per_sequence_offsets"]
    Q, K, V, GO = _inputs()
    full = oracle.attention_backward(Q, K, V, GO, **kw)
    monkeypatch.setattr(oa, "kv_group", lambda r, H_q, H_kv: r % H_kv)
    assert _group_errors(Q, K, V, GO, full, kw) > 1e-3


def test_planted_wrong_sequence_offset_fails(monkeypatch):
    kw = CASES["causal_per_sequence_offsets"]
    Q, K, V, GO = _inputs()
    full = oracle.attention_backward(Q, K, V, GO, **kw)
    real = oa.offsets_per_sequence
    monkeypatch.setattr(oa, "offsets_per_sequence", lambda off, n: (lambda v: v[1:] + v[:1])(real(off, n)))
    assert _group_errors(Q, K, V, GO, full, kw) > 1e-3
