"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on the
same seeded inputs, element by element, within the stated tolerance
(max|gpu - ref| / max|ref| <= 1e-5 for float32 I/O, <= 2e-2 for bf16 I/O).

Outputs and the workspace are NaN-poisoned before every call, so an element
the kernels never write fails the comparison."""

import math
import zlib

import numpy as np
import pytest

from exact_masked_scaled_amd import attn as A
from exact_masked_scaled_amd import workloads as W

import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    A.lib()  # fail loudly if the library is missing


# --------------------------------------------------------------------- small, full comparison
SMALL = [
    # (name, dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, offset, lens_q, lens_k)
    ("f32_d64_full", W.F32, 1, 2, 1, 70, 90, 64, 64, False, 0, None, None),
    ("f32_d128_causal", W.F32, 2, 2, 2, 97, 97, 128, 128, True, 0, None, None),
    ("f32_dh128_dv64_pad", W.F32, 2, 4, 2, 45, 150, 128, 64, False, 0, None, [150, 33]),
    ("f32_dh64_dv128_off", W.F32, 1, 3, 1, 40, 200, 64, 128, True, 160, None, None),
    ("bf16_d128_full_ragged", W.BF16, 2, 2, 1, 200, 333, 128, 128, False, 0, None, None),
    ("bf16_d128_causal_ragged", W.BF16, 2, 4, 2, 300, 300, 128, 128, True, 0, None, None),
    ("bf16_gqa_causal_rowpad", W.BF16, 3, 8, 2, 260, 260, 128, 128, True, 0, [260, 129, 1],
     [260, 129, 1]),
    ("bf16_cross_dv64_keypad", W.BF16, 2, 4, 4, 130, 700, 128, 64, False, 0, None, [700, 65]),
    ("bf16_mqa_offset", W.BF16, 2, 8, 1, 70, 520, 128, 128, True, 450, None, None),
    ("bf16_d64", W.BF16, 2, 2, 2, 190, 190, 64, 64, True, 0, None, None),
    ("bf16_dh64_dv128", W.BF16, 1, 2, 1, 64, 256, 64, 128, False, 0, None, None),
    ("bf16_offset_beyond_nk", W.BF16, 1, 2, 2, 33, 77, 128, 128, True, 1000, None, None),
    ("bf16_one_row_one_key", W.BF16, 1, 1, 1, 1, 1, 128, 128, True, 0, None, None),
    ("bf16_all_rows_inactive_seq", W.BF16, 2, 2, 1, 100, 100, 128, 128, False, 0, [0, 100],
     [0, 100]),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_small_full_parity(case):
    name, dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, off, lq, lk = case
    P.say(f"[parity] {name}")
    wl = W.custom_workload(dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, off, name)
    inp = W.make_custom_inputs(wl, seed=zlib.crc32(name.encode()) % 10000, seqlens_q=lq, seqlens_k=lk)
    gpu = P.run_gpu(inp)
    errs, ref = P.compare_full(inp, gpu)
    P.assert_within(errs, dtype, name)
    # structural zeros: inactive rows and padded keys
    if lq is not None:
        for b, L in enumerate(lq):
            assert (P.to_f64(gpu["O"][b, :, L:]) == 0).all()
            assert (P.to_f64(gpu["lse"][b, :, L:]) == 0).all()
            assert (P.to_f64(gpu["GQ"][b, :, L:]) == 0).all()
    if lk is not None:
        for b, L in enumerate(lk):
            assert (P.to_f64(gpu["GK"][b, :, L:]) == 0).all()
            assert (P.to_f64(gpu["GV"][b, :, L:]) == 0).all()


# --------------------------------------------------------------------- the five workloads
def test_workload1_full():
    """fp32 B=1, H=1, n=128, d=64, unmasked: every element."""
    inp = W.make_inputs(1)
    P.say(f"[parity] {inp.wl.describe()}")
    gpu = P.run_gpu(inp)
    errs, _ = P.compare_full(inp, gpu)
    P.assert_within(errs, W.F32, "workload 1")


FULL_SIZE = [(1, "bench"), (2, "bench"), (3, "bench"), (4, "bench"), (5, "bench"),
             (1, "unsplit"), (4, "unsplit"), (5, "unsplit"), (2, "two-pass"), (3, "two-pass")]


@pytest.mark.parametrize("wid,forward", FULL_SIZE, ids=lambda x: str(x))
@pytest.mark.timeout(900)
def test_full_size_every_group(wid, forward):
    """The five workloads at full size, with the forward and backward the
    benchmark runs ("bench": split over the keys with the automatic part
    count where that divides the problem, else unsplit; the backward keeping
    G_S where the library supports it, else the two passes), the unsplit
    forward, or the benchmark's forward with the two-pass backward
    ("two-pass"): every element of O, lse, G_Q, G_K and G_V against the
    float64 oracle, one (sequence, KV head) group at a time, plus the
    structural zeros of padded keys and inactive rows."""
    inp = W.make_inputs(wid)
    wl = inp.wl
    prob = A.make_problem(wl.B, wl.H_q, wl.H_kv, wl.n_q, wl.n_k, wl.d_h, wl.d_v,
                          A.BF16 if wl.dtype == W.BF16 else A.F32)
    ns = P.bench_forward_splits(prob) if forward != "unsplit" else 1
    gs = forward == "bench" and A.gs_workspace_size(prob) > A.workspace_size(prob)
    label = (f"workload {wid} ({'split forward, automatic parts' if ns == 0 else 'unsplit forward'}, "
             f"{'G_S kept' if gs else 'two-pass'} backward)")
    P.say(f"[parity] {label}: {wl.describe()} lens_k={inp.seqlens_k}")
    gpu = P.run_gpu(inp, num_splits=ns, keep_gs=gs)
    errs = P.compare_groups(inp, gpu, progress=8)
    P.record(f"workload {wid}", errs, forward="split" if ns == 0 else "unsplit", dtype=wl.dtype,
             backward="G_S kept" if gs else "two-pass", elements={n: int(t.numel()) for n, t in gpu.items()})
    P.assert_within(errs, wl.dtype, label)
    if inp.seqlens_k:
        for b, L in enumerate(inp.seqlens_k):
            assert not bool(gpu["GK"][b, :, L:].any()) and not bool(gpu["GV"][b, :, L:].any())
    if inp.seqlens_q:
        for b, L in enumerate(inp.seqlens_q):
            for n in ("O", "lse", "GQ"):
                assert not bool(gpu[n][b, :, L:].any()), n


# --------------------------------------------------------------------- pinned examples on the GPU
def _embed_example(K2, dtype):
    """The by-hand page's 2-position examples embedded at d = 128: zero-padded,
    with Q multiplied by exactly 8 = sqrt(128 / 2) so the scores are unchanged."""
    import torch
    d = 128
    tdt = torch.float32 if dtype == W.F32 else torch.bfloat16
    a = math.sqrt(2) * math.log(3)
    Q = torch.zeros(1, 1, 2, d, dtype=torch.float64)
    Q[0, 0, 0, 0] = 8 * a
    Q[0, 0, 1, 1] = 8 * a
    K = torch.zeros(1, 1, 2, d, dtype=torch.float64)
    K[0, 0, :, :2] = torch.tensor(K2, dtype=torch.float64)
    V = torch.zeros(1, 1, 2, d, dtype=torch.float64)
    V[0, 0, 0, 0] = 2.0
    V[0, 0, 1, 1] = 4.0
    G = torch.zeros(1, 1, 2, d, dtype=torch.float64)
    G[0, 0, 0, 0] = 1.0
    G[0, 0, 1, 1] = 2.0
    return [t.to(tdt).cuda() for t in (Q, K, V, G)]


def test_worked_examples_on_gpu_fp32():
    """Worked examples 1 and 2 of the by-hand page, through the fp32 kernels:
    O, lse, G_S-derived G_Q (chain rule for the x8 pre-scale), G_K and G_V."""
    gold1 = {"O": [[1.5, 1.0], [0.5, 3.0]], "dS": [[0.375, -0.375], [-1.5, 1.5]]}
    q, k, v, g = _embed_example([[1.0, 0.0], [0.0, 1.0]], W.F32)
    o, lse = A.fwd(q, k, v)
    dq, dk, dv = A.bwd(q, k, v, o, lse, g)
    O = P.to_f64(o)[0, 0, :, :2]
    np.testing.assert_allclose(O, gold1["O"], atol=2e-6)
    np.testing.assert_allclose(P.to_f64(lse)[0, 0], [math.log(4)] * 2, atol=2e-6)
    dS = np.array(gold1["dS"])
    np.testing.assert_allclose(8 * P.to_f64(dq)[0, 0, :, :2], dS / math.sqrt(2), atol=2e-6)
    np.testing.assert_allclose(P.to_f64(dk)[0, 0, :, :2], math.log(3) * dS.T, atol=2e-6)
    A1 = np.array([[0.75, 0.25], [0.25, 0.75]])
    np.testing.assert_allclose(P.to_f64(dv)[0, 0, :, :2], A1.T @ np.diag([1.0, 2.0]), atol=2e-6)
    assert np.abs(P.to_f64(o)[0, 0, :, 2:]).max() == 0
    # identical keys: O = [1, 2] in both rows, G_Q = 0, G_K != 0
    q, k, v, g = _embed_example([[1.0, 1.0], [1.0, 1.0]], W.F32)
    o, lse = A.fwd(q, k, v)
    dq, dk, dv = A.bwd(q, k, v, o, lse, g)
    np.testing.assert_allclose(P.to_f64(o)[0, 0, :, :2], [[1.0, 2.0], [1.0, 2.0]], atol=2e-6)
    assert np.abs(P.to_f64(dq)).max() < 1e-5
    assert np.abs(P.to_f64(dk)).max() > 0.1


def test_causal_first_row_loss_zero_future_gradients_gpu():
    """Chapter 31, sec. 6 on the GPU: G_O nonzero only in row 0 of a causal
    problem gives exactly zero G_K / G_V for every key after key 0."""
    import torch
    torch.manual_seed(0)
    q = torch.randn(1, 4, 200, 128).bfloat16().cuda()
    k = torch.randn(1, 2, 200, 128).bfloat16().cuda()
    v = torch.randn(1, 2, 200, 128).bfloat16().cuda()
    o, lse = A.fwd(q, k, v, causal=True)
    g = torch.zeros_like(o)
    g[:, :, 0] = torch.randn(1, 4, 128).bfloat16().cuda()
    dq, dk, dv = A.bwd(q, k, v, o, lse, g, causal=True)
    assert not bool(dk[:, :, 1:].any()) and not bool(dv[:, :, 1:].any())
    assert bool(dv[:, :, 0].any())
    assert not bool(dq[:, :, 1:].any())


def test_empty_row_is_an_error_on_gpu_call():
    import torch
    q = torch.randn(1, 1, 8, 128).bfloat16().cuda()
    with pytest.raises(A.AttnError) as ei:
        A.fwd(q, q, q, causal=True, offset=-1)
    assert ei.value.status == A.EMPTY_ROW
    with pytest.raises(A.AttnError) as ei:
        A.fwd(q, q, q, seqlens_k=[0])
    assert ei.value.status == A.EMPTY_ROW


def test_repeat_calls_are_stable():
    """Every output is bitwise reproducible (each element is written once, in a
    fixed order of additions)."""
    inp = W.make_custom_inputs(W.custom_workload(W.BF16, 1, 4, 1, 256, 256, 128, 128, True), seed=3)
    a = P.run_gpu(inp)
    b = P.run_gpu(inp)
    for n in ("O", "lse", "GQ", "GK", "GV"):
        assert bool((a[n] == b[n]).all()), n


def test_staged_backward_equals_bwd():
    """attn_bwd_dq followed by attn_bwd_dkdv gives what attn_bwd gives."""
    import torch
    inp = W.make_custom_inputs(W.custom_workload(W.BF16, 2, 4, 2, 200, 260, 128, 128, True, 60),
                               seed=5, seqlens_q=[200, 111], seqlens_k=[260, 170])
    ref = P.run_gpu(inp)
    q, k, v, do = (P.to_device(x) for x in (inp.Q, inp.K, inp.V, inp.GO))
    o, lse = ref["O"], ref["lse"]
    dq, dk, dv = (P.poison(torch.empty_like(x)) for x in (q, k, v))
    prob = A._problem_from(q, k, v, A._strides(o))
    ws = torch.full((A.workspace_size(prob),), 0xFF, dtype=torch.uint8, device=q.device)
    st = A.StagedBackward(q, k, v, o, lse, do, dq, dk, dv, ws, **inp.mask_kwargs())
    st.dq(); st.dkdv()
    torch.cuda.synchronize()
    assert bool((dk == ref["GK"]).all()) and bool((dv == ref["GV"]).all())
    assert bool((dq == ref["GQ"]).all())


DIVIDED_CASES = [
    # (name, dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, offset, lens_q, lens_k)
    ("bf16_chunked_gqa_divided", W.BF16, 1, 8, 2, 96, 1024, 128, 128, True, 928, None, None),
    ("bf16_cross_mqa_divided_ragged", W.BF16, 2, 8, 1, 70, 700, 128, 64, False, 0, [70, 33], [700, 517]),
    ("f32_chunked_divided", W.F32, 1, 2, 1, 64, 640, 64, 64, True, 576, None, None),
]


@pytest.mark.parametrize("case", DIVIDED_CASES, ids=lambda c: c[0])
def test_divided_backward_parity(case):
    """Grids too small for the GPU divide the backward passes (dQ over key
    parts, bf16 dK/dV over parts of each group's heads, float32 partials
    summed by combine kernels): the whole result against the oracle."""
    name, dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, off, lq, lk = case
    P.say(f"[parity] {name}")
    prob = A.make_problem(B, H_q, H_kv, n_q, n_k, d_h, d_v, A.BF16 if dtype == W.BF16 else A.F32)
    d_only = (B * H_q * n_q * 4 + 255) // 256 * 256
    assert A.workspace_size(prob) > d_only  # partials present: the passes are divided
    wl = W.custom_workload(dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, off, name)
    inp = W.make_custom_inputs(wl, seed=zlib.crc32(name.encode()) % 10000, seqlens_q=lq, seqlens_k=lk)
    gpu = P.run_gpu(inp)
    errs, ref = P.compare_full(inp, gpu)
    P.assert_within(errs, dtype, name)
