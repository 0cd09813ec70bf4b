"""GPU parity of attn_bwd_gs (the backward that keeps G_S from the dK/dV pass
and forms G_Q as one product over it) against the float64 oracle, element by
element (max|gpu - ref| / max|ref| <= 2e-2 bf16), with exact zeros required
for inactive rows and padded keys.  The workspace starts as NaN bit patterns,
so a G_S block the product read without the dK/dV pass having written it
would show.  Cases: grouped (group sizes that do and do not divide the
product's eight waves, and more than eight), MQA and MHA heads, both head
widths, the causal
rule with one offset and one per sequence, ragged and empty sequences, and
the random sweep's bf16 problems (those whose grids would be divided run the
two-pass backward, which attn_bwd_gs falls back to)."""

import zlib

import pytest

from exact_masked_scaled_amd import workloads as W

import parity as P
from test_gpu_random_sweep import CASES as SWEEP

pytestmark = pytest.mark.gpu

CASES = [
    # (name, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, offset, lens_q, lens_k)
    ("gqa_causal_ragged", 3, 8, 2, 300, 300, 128, 128, True, 0, [300, 129, 77], [300, 129, 77]),
    ("mqa_chunk_offsets", 2, 4, 1, 96, 400, 128, 128, True, [304, 17], [96, 40], [400, 57]),
    ("mha_d64_empty_seq", 3, 2, 2, 200, 200, 64, 64, True, 0, [200, 0, 65], [200, 31, 65]),
    ("cross_dv64", 2, 4, 4, 130, 700, 128, 64, False, 0, None, [700, 333]),
    ("gqa_dh64_dv128", 2, 4, 2, 256, 256, 64, 128, True, 0, None, None),
    ("group3", 2, 6, 2, 150, 150, 128, 128, True, 0, [150, 97], [150, 97]),
    ("group12_mqa", 1, 12, 1, 90, 260, 128, 128, True, 170, None, None),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check(name, dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, off, lq, lk):
    label = (f"[bwd_gs] {name} B={B} H_q={H_q} H_kv={H_kv} n_q={n_q} n_k={n_k} d_h={d_h} d_v={d_v} "
             f"causal={causal} off={off} lq={lq} lk={lk}")
    P.say(label)
    wl = W.custom_workload(dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, 0, name)
    inp = W.make_custom_inputs(wl, seed=zlib.crc32(name.encode()) % 10000, seqlens_q=lq, seqlens_k=lk)
    kw = dict(causal=causal, offset=off, seqlens_q=lq, seqlens_k=lk)
    inp.mask_kwargs = lambda: kw
    gpu = P.run_gpu(inp, keep_gs=True)
    errs, _ = P.compare_full(inp, gpu)
    P.assert_within(errs, dtype, label)
    for b in range(B):
        L_q = n_q if lq is None else lq[b]
        L_k = n_k if lk is None else lk[b]
        assert (P.to_f64(gpu["GQ"][b, :, L_q:]) == 0).all(), "G_Q of inactive rows"
        for t in ("GK", "GV"):
            assert (P.to_f64(gpu[t][b, :, L_k:]) == 0).all(), f"{t} of padded keys"


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_bwd_gs(case):
    _check(case[0], W.BF16, *case[1:])


@pytest.mark.parametrize("case", [c for c in SWEEP if c[1] == W.BF16], ids=lambda c: c[0])
def test_bwd_gs_sweep(case):
    _check(case[0], *case[1:13])


def test_bwd_gs_stages_equal_one_call():
    """attn_bwd_gs_stage 0, 1, 2 in order give attn_bwd_gs's results bit for
    bit (the benchmark times the stages separately), and its G_K and G_V are
    attn_bwd's."""
    import torch
    from exact_masked_scaled_amd import attn as A

    name, B, H_q, H_kv, n, d = "stages", 2, 8, 2, 384, 128
    P.say(f"[bwd_gs] {name} B={B} H_q={H_q} H_kv={H_kv} n={n} d={d} causal")
    g = torch.Generator().manual_seed(7)
    q, k, v, do = (torch.randn(B, H, n, d, generator=g).to(torch.bfloat16).cuda()
                   for H in (H_q, H_kv, H_kv, H_q))
    o, lse = A.fwd(q, k, v, causal=True)
    ref = A.bwd(q, k, v, o, lse, do, causal=True, keep_gs=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    prob = A._problem_from(q, k, v, A._strides(o), None, None, None, None)
    ws = torch.empty(A.gs_workspace_size(prob), dtype=torch.uint8, device=q.device)
    st = A.StagedBackward(q, k, v, o, lse, do, dq, dk, dv, ws, causal=True)
    for s_ in (0, 1, 2):
        st.gs_stage(s_)
    torch.cuda.synchronize()
    for a, b in zip(ref, (dq, dk, dv)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # G_K and G_V are the two-pass backward's, bit for bit (same dK/dV arithmetic and D)
    two = A.bwd(q, k, v, o, lse, do, causal=True)
    for a, b in zip(two[1:], (dk, dv)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_bwd_gs_repeatable_full_size():
    """The headline workload at full size (long key ranges: many rounds of
    the product pass's tile ring and every remainder length): three G_S
    backwards give bit-identical results, and G_K, G_V equal the two-pass
    backward's, so no stage of either pass is read before it has landed."""
    import torch
    from exact_masked_scaled_amd import attn as A

    inp = W.make_inputs(3)
    wl = inp.wl
    P.say(f"[bwd_gs] repeatable full size: {wl.describe()}")
    kw = inp.mask_kwargs()
    q, k, v, do = (P.to_device(x) for x in (inp.Q, inp.K, inp.V, inp.GO))
    o, lse = A.fwd(q, k, v, **kw)
    prob = A._problem_from(q, k, v, A._strides(o))
    assert A.gs_workspace_size(prob) > A.workspace_size(prob)
    ws = torch.empty(A.gs_workspace_size(prob), dtype=torch.uint8, device=q.device)
    first = [t.clone() for t in A.bwd(q, k, v, o, lse, do, workspace=ws, keep_gs=True, **kw)]
    for _ in range(2):
        again = A.bwd(q, k, v, o, lse, do, workspace=ws, keep_gs=True, **kw)
        for n, a, b in zip(("G_Q", "G_K", "G_V"), first, again):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), n
    two = A.bwd(q, k, v, o, lse, do, **kw)
    for n, a, b in zip(("G_K", "G_V"), first[1:], two[1:]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), n
