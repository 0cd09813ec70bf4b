"""GPU parity of the forward split over the keys (attn_fwd_splitkv): against
the float64 oracle on the same seeded, rounded inputs (max|gpu - ref| /
max|ref| <= 1e-5 float32, <= 2e-2 bf16), and against the unsplit forward.

Shapes follow the chunked and decoding uses the split is for: few query rows
per KV head against a long key range, with causal offsets, padding, grouped
heads, the packed layout, more parts than key tiles and a single part."""

import zlib

import numpy as np
import pytest

import oracle
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
    # (name, dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, offset, lens_q, lens_k, splits)
    ("bf16_chunked_mqa", W.BF16, 2, 8, 1, 256, 2100, 128, 128, True, 1844, None, None, 0),
    ("bf16_decode_gqa", W.BF16, 3, 8, 2, 1, 3000, 128, 128, True, 2999, None, [3000, 1700, 1], 0),
    ("bf16_cross_pad_dv64", W.BF16, 2, 4, 4, 70, 1500, 128, 64, False, 0, [70, 33], [1500, 700], 5),
    ("bf16_more_parts_than_tiles", W.BF16, 1, 2, 1, 40, 100, 128, 128, False, 0, None, None, 64),
    ("bf16_single_part", W.BF16, 1, 4, 2, 130, 600, 128, 128, True, 470, None, None, 1),
    ("bf16_d64_per_seq_offsets", W.BF16, 2, 4, 2, 50, 900, 64, 64, True, [850, 100], None, [900, 500], 7),
    ("f32_d128", W.F32, 1, 2, 1, 30, 700, 128, 128, True, 670, None, None, 3),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_splitkv_forward(case):
    torch = pytest.importorskip("torch")
    name, dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, off, lq, lk, splits = case
    P.say(f"[splitkv] {name}")
    wl = W.custom_workload(dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, 0, name)
    inp = W.make_custom_inputs(wl, seed=zlib.crc32(name.encode()) % 10000, seqlens_q=lq, seqlens_k=lk,
                               with_grad=False)
    kw = dict(causal=causal, offset=off, seqlens_q=lq, seqlens_k=lk)
    q, k, v = P.to_device(inp.Q), P.to_device(inp.K), P.to_device(inp.V)
    o = P.poison(torch.empty(B, H_q, n_q, d_v, dtype=q.dtype, device=q.device))
    lse = P.poison(torch.empty(B, H_q, n_q, dtype=torch.float32, device=q.device))
    prob = A._problem_from(q, k, v, A._strides(o))
    ws = torch.full((max(A.splitkv_workspace_size(prob, splits), 1),), 0xFF, dtype=torch.uint8, device="cuda")
    A.fwd_splitkv(q, k, v, num_splits=splits, out=o, lse=lse, workspace=ws, **kw)
    o1, lse1 = A.fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    f64 = W.payload_to_f64
    ref = oracle.attention_forward(f64(inp.Q), f64(inp.K), f64(inp.V), **kw)
    errs = {"O": P.rel_err(P.to_f64(o), ref["O"]), "lse": P.rel_err(P.to_f64(lse), ref["lse"])}
    P.assert_within(errs, dtype, name)
    # the split and the unsplit forward agree to rounding
    tol = 1e-5 if dtype == W.F32 else 1e-2
    assert P.rel_err(P.to_f64(o), P.to_f64(o1)) < tol
    assert P.rel_err(P.to_f64(lse), P.to_f64(lse1)) < 1e-5
    if lq is not None:  # inactive rows: exact zeros
        for b, L in enumerate(lq):
            assert (P.to_f64(o[b, :, L:]) == 0).all() and (P.to_f64(lse[b, :, L:]) == 0).all()


def test_splitkv_packed_layout():
    torch = pytest.importorskip("torch")
    lq, lk = [64, 1, 130], [1400, 333, 2000]
    H_q, H_kv, d = 4, 1, 128
    offs = [1336, 332, 1870]
    B = len(lq)
    wl = W.custom_workload(W.BF16, B, H_q, H_kv, max(lq), max(lk), d, d, True, 0, "split_packed")
    inp = W.make_custom_inputs(wl, seed=77, with_grad=False)

    def pack(X, lens):
        return np.ascontiguousarray(np.concatenate([X[b, :, :L].transpose(1, 0, 2) for b, L in enumerate(lens)]))
    cu_q = [0] + np.cumsum(lq).astype(int).tolist()
    cu_k = [0] + np.cumsum(lk).astype(int).tolist()
    Qp, Kp, Vp = pack(inp.Q, lq), pack(inp.K, lk), pack(inp.V, lk)
    P.say("[splitkv] packed")
    q, k, v = P.to_device(Qp), P.to_device(Kp), P.to_device(Vp)
    pk = dict(causal=True, offset=offs, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)
    o, lse = A.fwd_splitkv(q, k, v, num_splits=0, **pk)
    torch.cuda.synchronize()
    f64 = W.payload_to_f64
    ref = oracle.attention_backward_packed(f64(Qp), f64(Kp), f64(Vp), None, cu_q, cu_k, causal=True, offset=offs)
    errs = {"O": P.rel_err(P.to_f64(o), ref["O"]), "lse": P.rel_err(P.to_f64(lse), ref["lse"])}
    P.assert_within(errs, W.BF16, "splitkv packed")
