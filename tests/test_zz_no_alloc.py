"""attn_bwd_noalloc, the backward whose workspace is the library's fixed
device array, against attn_bwd with a caller workspace: bitwise equal results
on two calls in a row, the second with a smaller problem (the array keeps the
first call's contents, which the second must not depend on)."""

import zlib

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
    A.lib()


CASES = [
    # (name, dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, offset, lens_q, lens_k)
    ("bf16_gqa_causal_rowpad", W.BF16, 3, 8, 2, 700, 700, 128, 128, True, 0, [700, 333, 41], [700, 333, 41]),
    ("bf16_chunked_mqa_divided", W.BF16, 1, 8, 1, 96, 1500, 128, 128, True, 1404, None, None),
    ("f32_cross_small", W.F32, 2, 2, 1, 50, 90, 64, 64, False, 0, None, [90, 17]),
]


def _run(case):
    import torch
    name, dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, off, lq, lk = case
    wl = W.custom_workload(dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, off, name)
    inp = W.make_custom_inputs(wl, seed=zlib.crc32(name.encode()) % 10000, seqlens_q=lq, seqlens_k=lk)
    ref = P.run_gpu(inp)  # attn_fwd, then attn_bwd with a caller workspace
    q, k, v, do = (P.to_device(x) for x in (inp.Q, inp.K, inp.V, inp.GO))
    dq, dk, dv = (P.poison(torch.empty_like(x)) for x in (q, k, v))
    A.bwd_noalloc(q, k, v, ref["O"], ref["lse"], do, dq=dq, dk=dk, dv=dv, **inp.mask_kwargs())
    torch.cuda.synchronize()
    for n, t in (("GQ", dq), ("GK", dk), ("GV", dv)):
        assert torch.equal(t, ref[n]), f"{name}: {n} differs from attn_bwd"
    return ref


def test_noalloc_equals_bwd_two_calls_second_smaller():
    """Largest problem first, then smaller ones reusing the same array."""
    for case in CASES:
        P.say(f"[noalloc] {case[0]}")
        _run(case)
    # and the first again after the smaller ones
    P.say(f"[noalloc] {CASES[0][0]} again")
    _run(CASES[0])
