"""Host-side checks of the seeded input generator and the work accounting."""

import numpy as np

import oracle
from exact_masked_scaled_amd import workloads as W


def test_bf16_rounding_is_single_step_rne():
    # exact bf16 values stay put; halfway cases go to the even neighbour
    one = 1.0
    ulp = 2.0 ** -7  # spacing of bf16 values in [1, 2)
    x = np.array([one, one + ulp, one + ulp / 2, one + 3 * ulp / 2, -(one + ulp / 2), 3.0e-3])
    r = W.round_to_bf16(x)
    assert r[0] == 1.0 and r[1] == 1.0 + ulp
    assert r[2] == 1.0                      # tie -> even (1.0)
    assert r[3] == 1.0 + 2 * ulp            # tie -> even (1 + 2 ulp)
    assert r[4] == -1.0
    # a float64 value just above a tie must round up (no double rounding via fp32)
    y = np.array([one + ulp / 2 + 2.0 ** -40])
    assert W.round_to_bf16(y)[0] == one + ulp
    # bit patterns round-trip
    rng = np.random.default_rng(0)
    z = W.round_to_bf16(rng.standard_normal(10000))
    assert np.array_equal(W.bf16_bits_to_f64(W.bf16_bits(z)), z)
    assert np.abs(z / W.round_to_bf16(z) - 1).max() == 0


def test_chunked_draw_matches_single_draw():
    a = W._draw_rounded(np.random.default_rng(5), (3, 1000), W.F32, chunk=7)
    b = np.random.default_rng(5).standard_normal(3000).astype(np.float32).reshape(3, 1000)
    assert np.array_equal(a, b)


def test_seeded_inputs_are_reproducible():
    x = W.make_inputs(1)
    y = W.make_inputs(1)
    assert np.array_equal(x.Q, y.Q) and np.array_equal(x.GO, y.GO)
    assert x.Q.dtype == np.float32 and x.Q.shape == (1, 1, 128, 64)


def test_pair_count_matches_oracle_mask():
    for wl in W.WORKLOADS.values():
        lq = [wl.n_q // 2 + 3] * wl.B if wl.pad_rows_like_keys else None
        lk = [wl.n_k // 2 + 5] * wl.B if wl.len_k_range else None
        if lq is not None:
            lq = lk
        # shrink to keep the mask small but keep the structure
        counts = W.visible_pairs_per_sequence(wl.n_q, wl.n_k, wl.causal, wl.offset, lq, lk, wl.B)
        for b in range(min(wl.B, 2)):
            M = oracle.visible_mask(wl.n_q, wl.n_k, (lq or [wl.n_q] * wl.B)[b],
                                    (lk or [wl.n_k] * wl.B)[b], wl.causal, wl.offset)
            assert counts[b] == int(M.sum())


def test_literal_flop_formula_close_for_square_causal():
    wl = W.WORKLOADS[2]
    w = W.work(wl)
    assert abs(w["fwd_flop"] / w["literal_fwd_flop"] - 1) < 1e-3
    assert w["bwd_flop"] == 5 * w["fwd_flop"] // 2
