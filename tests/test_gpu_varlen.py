"""GPU parity of per-sequence causal offsets and the packed ("varlen") layout:
the HIP path through the C ABI against the float64 oracle on the same seeded,
rounded inputs (max|gpu - ref| / max|ref| <= 1e-5 float32, <= 2e-2 bf16).

Packed tensors are views into larger NaN/sentinel-filled buffers: every row
the kernels must write is poisoned first, and the rows after the last
sequence must come back untouched (no write past a sequence's own rows)."""

import zlib

import numpy as np
import pytest

import oracle
from exact_masked_scaled_amd import attn as A
from exact_masked_scaled_amd import workloads as W

import parity as P

pytestmark = pytest.mark.gpu

SLACK = 40  # extra rows after the packed rows of every buffer


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    A.lib()


# --------------------------------------------------------------------- per-sequence offsets
OFFSET_CASES = [
    # (name, dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, offsets, lens_q, lens_k)
    ("bf16_gqa_offsets", W.BF16, 3, 8, 2, 200, 450, 128, 128, [250, 0, 120], None, [450, 200, 333]),
    ("bf16_chunked_offsets_rowpad", W.BF16, 3, 4, 1, 130, 700, 128, 128, [570, 3, 640],
     [130, 64, 1], [700, 67, 641]),
    ("bf16_dv64_offsets", W.BF16, 2, 4, 4, 96, 300, 128, 64, [204, 0], None, None),
    ("f32_d64_offsets", W.F32, 2, 2, 1, 70, 160, 64, 64, [90, 10], None, [160, 80]),
]


@pytest.mark.parametrize("case", OFFSET_CASES, ids=lambda c: c[0])
def test_per_sequence_offsets(case):
    name, dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, offs, lq, lk = case
    P.say(f"[varlen] {name}")
    wl = W.custom_workload(dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, True, 0, name)
    inp = W.make_custom_inputs(wl, seed=zlib.crc32(name.encode()) % 10000, seqlens_q=lq, seqlens_k=lk)
    # the inputs carry one offset; this problem uses one per sequence
    kw = dict(causal=True, offset=offs, seqlens_q=lq, seqlens_k=lk)
    inp.mask_kwargs = lambda: kw
    gpu = P.run_gpu(inp)
    errs, ref = P.compare_full(inp, gpu)
    P.assert_within(errs, dtype, name)
    # a sequence's keys past its offset window get exactly zero gradient from
    # its rows: the last visible key of sequence b is min(L_k, L_q - 1 + off + 1)
    for b in range(B):
        L_q = n_q if lq is None else lq[b]
        L_k = n_k if lk is None else lk[b]
        last = min(L_k, L_q + offs[b]) if L_q > 0 else 0
        assert (P.to_f64(gpu["GK"][b, :, last:]) == 0).all()
        assert (P.to_f64(gpu["GV"][b, :, last:]) == 0).all()


# --------------------------------------------------------------------- packed layout
PACKED_CASES = [
    # (name, dtype, H_q, H_kv, d_h, d_v, lens_q, lens_k, causal, offset)
    ("bf16_gqa_causal", W.BF16, 8, 2, 128, 128, [37, 300, 129, 1, 256], [37, 300, 129, 1, 256], True, 0),
    ("bf16_gqa_causal_empty_seqs", W.BF16, 4, 2, 128, 128, [0, 190, 0, 65], [0, 190, 7, 65], True, 0),
    ("bf16_chunked_per_seq_offsets", W.BF16, 4, 1, 128, 128, [64, 1, 130], [400, 33, 530], True,
     [336, 32, 400]),
    ("bf16_cross_dv64", W.BF16, 4, 4, 128, 64, [70, 128, 33], [500, 65, 257], False, 0),
    ("bf16_d64", W.BF16, 2, 2, 64, 64, [100, 31], [100, 31], True, 0),
    ("f32_d128_causal", W.F32, 2, 1, 128, 128, [45, 97], [45, 97], True, 0),
]


def _pack(X: np.ndarray, lens) -> np.ndarray:
    """[B, H, n, d] (payload dtype) -> [sum(lens), H, d]."""
    parts = [X[b, :, :L].transpose(1, 0, 2) for b, L in enumerate(lens)]
    return np.ascontiguousarray(np.concatenate(parts, axis=0)) if parts else X[:0, :, 0]


def _device_rows(a: np.ndarray, fill):
    """Packed payload -> device tensor view of its rows inside a buffer with
    SLACK more rows, all of them set to ``fill`` first."""
    torch = pytest.importorskip("torch")
    rows = a.shape[0]
    t = P.to_device(a)
    buf = torch.empty((rows + SLACK,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
    buf.fill_(fill)
    buf[:rows].copy_(t)
    return buf[:rows], buf


def _empty_rows(rows, shape_tail, dtype, fill):
    torch = pytest.importorskip("torch")
    buf = torch.empty((rows + SLACK,) + tuple(shape_tail), dtype=dtype, device="cuda")
    buf.fill_(fill)
    return buf[:rows], buf


@pytest.mark.parametrize("case", PACKED_CASES, ids=lambda c: c[0])
def test_packed_layout(case):
    torch = pytest.importorskip("torch")
    name, dtype, H_q, H_kv, d_h, d_v, lq, lk, causal, off = case
    P.say(f"[varlen] {name}")
    B, n_q, n_k = len(lq), max(lq), max(lk)
    wl = W.custom_workload(dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, 0, name)
    inp = W.make_custom_inputs(wl, seed=zlib.crc32(name.encode()) % 10000)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(int).tolist()
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(int).tolist()
    Qp, Kp, Vp, GOp = (_pack(inp.Q, lq), _pack(inp.K, lk), _pack(inp.V, lk), _pack(inp.GO, lq))
    tq, tk = cu_q[-1], cu_k[-1]
    sentinel = 7.0
    q, _ = _device_rows(Qp, sentinel)
    k, _ = _device_rows(Kp, sentinel)
    v, _ = _device_rows(Vp, sentinel)
    do, _ = _device_rows(GOp, sentinel)
    tdt = q.dtype
    o, o_buf = _empty_rows(tq, (H_q, d_v), tdt, sentinel)
    o.fill_(float("nan"))
    lse_buf = torch.full((H_q, tq + SLACK), sentinel, dtype=torch.float32, device="cuda")
    lse = lse_buf[:, :tq].contiguous()  # lse must be contiguous [H_q, total]
    lse.fill_(float("nan"))
    pk = dict(causal=causal, offset=off, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)
    A.fwd(q, k, v, out=o, lse=lse, **pk)
    dq, dq_buf = _empty_rows(tq, (H_q, d_h), tdt, sentinel)
    dk, dk_buf = _empty_rows(tk, (H_kv, d_h), tdt, sentinel)
    dv, dv_buf = _empty_rows(tk, (H_kv, d_v), tdt, sentinel)
    for t in (dq, dk, dv):
        t.fill_(float("nan"))
    prob = A._problem_from(q, k, v, A._strides(o), cu_q, cu_k)
    ws = torch.full((max(A.workspace_size(prob), 1),), 0xFF, dtype=torch.uint8, device="cuda")
    A.bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, **pk)
    torch.cuda.synchronize()
    f64 = W.payload_to_f64
    ref = oracle.attention_backward_packed(f64(Qp), f64(Kp), f64(Vp), f64(GOp), cu_q, cu_k,
                                           causal=causal, offset=off)
    errs = {"O": P.rel_err(P.to_f64(o), ref["O"]), "lse": P.rel_err(P.to_f64(lse), ref["lse"]),
            "GQ": P.rel_err(P.to_f64(dq), ref["GQ"]), "GK": P.rel_err(P.to_f64(dk), ref["GK"]),
            "GV": P.rel_err(P.to_f64(dv), ref["GV"])}
    P.assert_within(errs, dtype, name)
    # nothing written past the packed rows
    for nm, buf, rows in (("O", o_buf, tq), ("GQ", dq_buf, tq), ("GK", dk_buf, tk), ("GV", dv_buf, tk)):
        assert (P.to_f64(buf[rows:]) == sentinel).all(), f"{name}: {nm} written past its rows"


def test_packed_equals_padded_on_gpu():
    """The packed call and the padded call with the same lengths give the same
    numbers (the kernels see the same rows in the same order)."""
    torch = pytest.importorskip("torch")
    lq = [37, 300, 129, 1]
    B, H_q, H_kv, d = len(lq), 8, 2, 128
    n = max(lq)
    wl = W.custom_workload(W.BF16, B, H_q, H_kv, n, n, d, d, True, 0, "pk_vs_pad")
    inp = W.make_custom_inputs(wl, seed=123, seqlens_q=lq, seqlens_k=lq)
    P.say("[varlen] packed vs padded")
    pad = P.run_gpu(inp)
    cu = np.concatenate([[0], np.cumsum(lq)]).astype(int).tolist()
    q, k, v, do = (P.to_device(_pack(inp.Q, lq)), P.to_device(_pack(inp.K, lq)),
                   P.to_device(_pack(inp.V, lq)), P.to_device(_pack(inp.GO, lq)))
    pk = dict(causal=True, offset=0, cu_seqlens_q=cu, cu_seqlens_k=cu)
    o, lse = A.fwd(q, k, v, **pk)
    dq, dk, dv = A.bwd(q, k, v, o, lse, do, **pk)
    torch.cuda.synchronize()
    for b, L in enumerate(lq):
        rows = slice(cu[b], cu[b + 1])
        for got, ref in ((o[rows], pad["O"][b, :, :L]), (dq[rows], pad["GQ"][b, :, :L]),
                         (dk[rows], pad["GK"][b, :, :L]), (dv[rows], pad["GV"][b, :, :L])):
            assert torch.equal(got.transpose(0, 1), ref)
        assert torch.equal(lse[:, rows], pad["lse"][b, :, :L])


# --------------------------------------------------------------------- padding content
NAN_PAD_CASES = [
    # (name, dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, offset, lens_q, lens_k)
    ("bf16_gqa_causal_nanpad", W.BF16, 3, 8, 2, 200, 200, 128, 128, True, 0, [200, 77, 130], [200, 77, 130]),
    ("bf16_cross_nanpad", W.BF16, 2, 4, 4, 150, 300, 128, 64, False, 0, [33, 150], [290, 65]),
    ("f32_d64_nanpad", W.F32, 2, 2, 1, 96, 96, 64, 64, True, 0, [50, 96], [50, 96]),
]


@pytest.mark.parametrize("case", NAN_PAD_CASES, ids=lambda c: c[0])
def test_padding_rows_never_read(case):
    """Rows past L_q and keys past L_k in the padded layout may hold anything,
    NaN included: every output, and every inactive row or padded key of the
    outputs (zeros), is the same as with finite padding."""
    torch = pytest.importorskip("torch")
    name, dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, off, lq, lk = case
    P.say(f"[varlen] {name}")
    wl = W.custom_workload(dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, off, name)
    inp = W.make_custom_inputs(wl, seed=zlib.crc32(name.encode()) % 10000, seqlens_q=lq, seqlens_k=lk)
    kw = inp.mask_kwargs()
    q, k, v, do = (P.to_device(inp.Q), P.to_device(inp.K), P.to_device(inp.V), P.to_device(inp.GO))
    for b in range(B):
        q[b, :, lq[b]:] = float("nan")
        do[b, :, lq[b]:] = float("nan")
        k[b, :, lk[b]:] = float("nan")
        v[b, :, lk[b]:] = float("nan")
    o, lse = A.fwd(q, k, v, **kw)
    # the split forward takes the same copies
    o_s, lse_s = A.fwd_splitkv(q, k, v, num_splits=3, **kw)
    dq, dk, dv = A.bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    gpu = {"O": o, "lse": lse, "GQ": dq, "GK": dk, "GV": dv}
    for nm, t in list(gpu.items()) + [("O_split", o_s), ("lse_split", lse_s)]:
        assert torch.isfinite(t.float()).all(), f"{name}: {nm} not finite"
    errs, ref = P.compare_full(inp, gpu)
    P.assert_within(errs, dtype, name)
    for b in range(B):
        assert (P.to_f64(o[b, :, lq[b]:]) == 0).all() and (P.to_f64(dq[b, :, lq[b]:]) == 0).all()
        assert (P.to_f64(o_s[b, :, lq[b]:]) == 0).all()
        assert (P.to_f64(dk[b, :, lk[b]:]) == 0).all() and (P.to_f64(dv[b, :, lk[b]:]) == 0).all()


# --------------------------------------------------------------------- more sequences than one launch takes
def test_many_sequences_chunked_launches():
    """300 sequences with their own lengths and offsets (more than one
    launch's 128): the padded forward, the split forward, the backward (its
    dK/dV pass divided over heads for this small grid), and the packed
    layout, against the oracle."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(2024)
    B, H_q, H_kv, n_q, n_k, d = 300, 2, 1, 48, 80, 128
    lq = rng.integers(0, n_q + 1, size=B).tolist()
    lk = [int(x) for x in rng.integers(1, n_k + 1, size=B)]
    offs = [int(rng.integers(0, k_ + 1)) for k_ in lk]  # row 0 sees keys 0..off
    wl = W.custom_workload(W.BF16, B, H_q, H_kv, n_q, n_k, d, d, True, 0, "many_seqs")
    inp = W.make_custom_inputs(wl, seed=77, seqlens_q=lq, seqlens_k=lk)
    kw = dict(causal=True, offset=offs, seqlens_q=lq, seqlens_k=lk)
    inp.mask_kwargs = lambda: kw
    P.say("[varlen] 300 sequences, padded")
    gpu = P.run_gpu(inp)
    errs, ref = P.compare_full(inp, gpu)
    P.assert_within(errs, W.BF16, "many sequences padded")
    q, k, v = P.to_device(inp.Q), P.to_device(inp.K), P.to_device(inp.V)
    o_s, lse_s = A.fwd_splitkv(q, k, v, num_splits=2, **kw)
    torch.cuda.synchronize()
    es = {"O": P.rel_err(P.to_f64(o_s), ref["O"]), "lse": P.rel_err(P.to_f64(lse_s), ref["lse"])}
    P.assert_within(es, W.BF16, "many sequences split forward")
    # packed: the same sequences without padding rows
    P.say("[varlen] 300 sequences, packed")
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(int).tolist()
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(int).tolist()
    qp, kp, vp, dop = (P.to_device(_pack(inp.Q, lq)), P.to_device(_pack(inp.K, lk)), P.to_device(_pack(inp.V, lk)),
                       P.to_device(_pack(inp.GO, lq)))
    pk = dict(causal=True, offset=offs, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, max_seqlen_q=n_q, max_seqlen_k=n_k)
    op, lsep = A.fwd(qp, kp, vp, **pk)
    dqp, dkp, dvp = A.bwd(qp, kp, vp, op, lsep, dop, **pk)
    torch.cuda.synchronize()
    for b in range(B):
        rq, rk = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        for got, want in ((op[rq].transpose(0, 1), gpu["O"][b, :, :lq[b]]), (dqp[rq].transpose(0, 1), gpu["GQ"][b, :, :lq[b]]),
                          (dkp[rk].transpose(0, 1), gpu["GK"][b, :, :lk[b]]), (dvp[rk].transpose(0, 1), gpu["GV"][b, :, :lk[b]])):
            assert torch.equal(got, want), b
