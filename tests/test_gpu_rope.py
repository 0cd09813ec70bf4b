"""GPU parity of the rotary-position path (attn_rope_apply, attn_fwd_rope,
attn_bwd_rope) through the C ABI against the float64 oracle
(oracle.attention_backward_rope, oracle.rope_rotate) on the same seeded,
rounded inputs and the same float32 cos/sin table.

Tolerance: max|gpu - ref| / max|ref| <= 1e-5 (float32 I/O) or 2e-2 (bf16 I/O)
per tensor, as for the unrotated path.  Besides the oracle, the fused forms
are checked against the unfused ones: the forward turns Q in registers through
the same rotation as the standalone kernel, so attn_fwd_rope equals attn_fwd
on explicitly rotated inputs bit for bit; in the backward G_Q / G_K differ
from turning back a rounded G_Q~ / G_K~ only by that rounding, and G_V from
attn_bwd on rotated inputs only by float32 summation order."""

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


def _table(n_pos, d_h):
    cs = oracle.rope_table(n_pos, d_h)  # float32 [n_pos, d_h/2, 2]
    return cs, P.to_device(cs)


CASES = [
    # (name, dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, offset, lens_q, lens_k, n_pos)
    ("bf16_gqa_causal", W.BF16, 2, 8, 2, 256, 256, 128, 128, True, 0, None, None, 256),
    ("bf16_gqa_causal_lens", W.BF16, 3, 4, 2, 200, 200, 128, 128, True, 0, [200, 77, 130], [200, 77, 130], 300),
    ("bf16_chunked", W.BF16, 2, 4, 1, 96, 400, 128, 128, True, 304, None, None, 400),
    ("bf16_chunked_per_seq", W.BF16, 3, 4, 2, 70, 333, 128, 128, True, [263, 5, 100],
     [70, 64, 1], [333, 69, 101], 333),
    ("bf16_cross_shifted", W.BF16, 2, 4, 4, 130, 260, 128, 64, False, 50, None, [260, 129], 260),
    ("bf16_d64", W.BF16, 2, 2, 1, 160, 160, 64, 64, True, 0, None, None, 160),
    ("f32_d128", W.F32, 2, 2, 1, 100, 100, 128, 128, True, 0, None, [100, 57], 128),
    ("f32_d64_chunked", W.F32, 1, 2, 2, 40, 150, 64, 64, True, 110, None, None, 150),
]


def _inputs(case):
    name, dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, off, lq, lk, n_pos = case
    wl = W.custom_workload(dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, 0, name)
    inp = W.make_custom_inputs(wl, seed=zlib.crc32(name.encode()) % 10000, seqlens_q=lq, seqlens_k=lk)
    kw = dict(causal=causal, offset=off, seqlens_q=lq, seqlens_k=lk)
    return inp, kw


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_rope_attention_parity(case):
    torch = pytest.importorskip("torch")
    name, dtype, n_pos, d_h = case[0], case[1], case[-1], case[7]
    P.say(f"[rope] {name}")
    inp, kw = _inputs(case)
    cs_host, cs = _table(n_pos, d_h)
    q, k, v, do = (P.to_device(inp.Q), P.to_device(inp.K), P.to_device(inp.V), P.to_device(inp.GO))
    o = P.poison(torch.empty(q.shape[:3] + (v.shape[-1],), dtype=q.dtype, device=q.device))
    lse = P.poison(torch.empty(q.shape[:3], dtype=torch.float32, device=q.device))
    A.fwd_rope(q, k, v, cs, out=o, lse=lse, **kw)
    dq, dk, dv = (P.poison(torch.empty_like(q)), P.poison(torch.empty_like(k)), P.poison(torch.empty_like(v)))
    prob = A._problem_from(q, k, v, A._strides(o))
    ws = torch.full((A.rope_workspace_size(prob, backward=True),), 0xFF, dtype=torch.uint8, device=q.device)
    A.bwd_rope(q, k, v, o, lse, do, cs, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)
    torch.cuda.synchronize()
    f64 = W.payload_to_f64
    ref = oracle.attention_backward_rope(f64(inp.Q), f64(inp.K), f64(inp.V), f64(inp.GO), cs_host, **kw)
    gpu = {"O": o, "lse": lse, "GQ": dq, "GK": dk, "GV": dv}
    errs = {nm: P.rel_err(P.to_f64(t), ref[nm]) for nm, t in gpu.items()}
    P.assert_within(errs, dtype, name)
    # inactive rows and padded keys stay exact zeros
    lq, lk = kw["seqlens_q"], kw["seqlens_k"]
    for b in range(q.shape[0]):
        L_q = q.shape[2] if lq is None else lq[b]
        L_k = k.shape[2] if lk is None else lk[b]
        assert (P.to_f64(dq[b, :, L_q:]) == 0).all() and (P.to_f64(o[b, :, L_q:]) == 0).all()
        assert (P.to_f64(dk[b, :, L_k:]) == 0).all() and (P.to_f64(dv[b, :, L_k:]) == 0).all()


@pytest.mark.parametrize("case", [CASES[1], CASES[3], CASES[6]], ids=lambda c: c[0])
def test_rope_fused_equals_unfused(case):
    torch = pytest.importorskip("torch")
    name, dtype, n_pos, d_h = case[0], case[1], case[-1], case[7]
    P.say(f"[rope] fused vs unfused {name}")
    inp, kw = _inputs(case)
    _, cs = _table(n_pos, d_h)
    q, k, v, do = (P.to_device(inp.Q), P.to_device(inp.K), P.to_device(inp.V), P.to_device(inp.GO))
    o_f, lse_f = A.fwd_rope(q, k, v, cs, **kw)
    qt = A.rope_apply(q, k, v, cs, operand="q", **kw)
    kt = A.rope_apply(q, k, v, cs, operand="k", **kw)
    lq, lk = kw["seqlens_q"], kw["seqlens_k"]
    # rows past the active ones are not written by the rotation: give them zeros
    for b in range(q.shape[0]):
        if lq is not None:
            qt[b, :, lq[b]:] = 0
        if lk is not None:
            kt[b, :, lk[b]:] = 0
    o_u, lse_u = A.fwd(qt, kt, v, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_f, o_u) and torch.equal(lse_f, lse_u)
    dq_f, dk_f, dv_f = A.bwd_rope(q, k, v, o_f, lse_f, do, cs, **kw)
    dqt, dkt, dv_u = A.bwd(qt, kt, v, o_u, lse_u, do, **kw)
    dq_u = A.rope_apply(dqt, k, v, cs, operand="q", inverse=True, **kw)
    dk_u = A.rope_apply(q, dkt, v, cs, operand="k", inverse=True, **kw)
    torch.cuda.synchronize()
    # G_V: the same sums, but the unrotated backward may divide a small grid's
    # passes (float32 partials summed in another order), so to rounding
    tol = 1e-2 if dtype == W.BF16 else 1e-6  # one bf16 rounding of G_Q~ / G_K~
    for got, want, lens in ((dq_f, dq_u, lq), (dk_f, dk_u, lk), (dv_f, dv_u, lk)):
        g, w = P.to_f64(got), P.to_f64(want)
        for b in range(q.shape[0]):
            n = got.shape[2] if lens is None else lens[b]
            gb, wb = g[b, :, :n], w[b, :, :n]
            assert np.max(np.abs(gb - wb), initial=0.0) <= tol * np.max(np.abs(wb), initial=1e-30)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_rope_apply_parity(dtype):
    """The standalone rotation against the oracle's, its inverse, in place."""
    torch = pytest.importorskip("torch")
    B, H_q, H_kv, n_q, n_k, d = 2, 4, 2, 90, 120, 128
    wl = W.custom_workload(dtype, B, H_q, H_kv, n_q, n_k, d, d, True, 0, "rope_apply")
    inp = W.make_custom_inputs(wl, seed=77, seqlens_q=[90, 33], seqlens_k=[120, 63], with_grad=False)
    offs = [30, 7]
    kw = dict(causal=True, offset=offs, seqlens_q=[90, 33], seqlens_k=[120, 63])
    cs_host, cs = _table(128, d)
    q, k, v = P.to_device(inp.Q), P.to_device(inp.K), P.to_device(inp.V)
    P.say(f"[rope] apply {dtype}")
    qt = A.rope_apply(q, k, v, cs, operand="q", out=P.poison(torch.empty_like(q)), **kw)
    kt = A.rope_apply(q, k, v, cs, operand="k", out=P.poison(torch.empty_like(k)), **kw)
    torch.cuda.synchronize()
    f64 = W.payload_to_f64
    # one rounding of a float32 rotation: 2^-8 relative for bf16
    tol = 2.0 ** -8 if dtype == W.BF16 else 1e-6
    for b in range(B):
        L_q, L_k = kw["seqlens_q"][b], kw["seqlens_k"][b]
        ref_q = oracle.rope_rotate(f64(inp.Q[b, :, :L_q]), cs_host, np.arange(L_q) + offs[b])
        ref_k = oracle.rope_rotate(f64(inp.K[b, :, :L_k]), cs_host, np.arange(L_k))
        for got, ref in ((P.to_f64(qt[b, :, :L_q]), ref_q), (P.to_f64(kt[b, :, :L_k]), ref_k)):
            assert np.all(np.abs(got - ref) <= tol * np.abs(ref) + 1e-6 * np.max(np.abs(ref)))
        # rows past the active ones are left alone
        assert torch.isnan(qt[b, :, L_q:].float()).all() and torch.isnan(kt[b, :, L_k:].float()).all()
    # turning back in place recovers the input up to two roundings
    A.rope_apply(qt, k, v, cs, operand="q", inverse=True, out=qt, **kw)
    torch.cuda.synchronize()
    for b in range(B):
        L_q = kw["seqlens_q"][b]
        got, want = P.to_f64(qt[b, :, :L_q]), f64(inp.Q[b, :, :L_q])
        assert np.max(np.abs(got - want)) <= 2 * tol * np.max(np.abs(want))


def test_rope_packed_equals_padded():
    """Packed rotary attention equals the padded call with the same lengths."""
    torch = pytest.importorskip("torch")
    lq, offs = [37, 150, 1, 96], [0, 20, 7, 3]
    lk = [L + o for L, o in zip(lq, offs)]
    B, H_q, H_kv, d = len(lq), 4, 2, 128
    n_q, n_k = max(lq), max(lk)
    wl = W.custom_workload(W.BF16, B, H_q, H_kv, n_q, n_k, d, d, True, 0, "rope_packed")
    inp = W.make_custom_inputs(wl, seed=5, seqlens_q=lq, seqlens_k=lk)
    _, cs = _table(256, d)
    P.say("[rope] packed vs padded")
    kw = dict(causal=True, offset=offs, seqlens_q=lq, seqlens_k=lk)
    q, k, v, do = (P.to_device(inp.Q), P.to_device(inp.K), P.to_device(inp.V), P.to_device(inp.GO))
    o, lse = A.fwd_rope(q, k, v, cs, **kw)
    dq, dk, dv = A.bwd_rope(q, k, v, o, lse, do, cs, **kw)

    def pack(t, lens):
        return torch.cat([t[b, :, :L].transpose(0, 1) for b, L in enumerate(lens)], 0).contiguous()

    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(int).tolist()
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(int).tolist()
    pk = dict(causal=True, offset=offs, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)
    qp, kp, vp, dop = pack(q, lq), pack(k, lk), pack(v, lk), pack(do, lq)
    op, lsep = A.fwd_rope(qp, kp, vp, cs, **pk)
    dqp, dkp, dvp = A.bwd_rope(qp, kp, vp, op, lsep, dop, cs, **pk)
    torch.cuda.synchronize()
    for b in range(B):
        rq, rk = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        assert torch.equal(op[rq].transpose(0, 1), o[b, :, :lq[b]])
        assert torch.equal(lsep[:, rq], lse[b, :, :lq[b]])
        assert torch.equal(dqp[rq].transpose(0, 1), dq[b, :, :lq[b]])
        assert torch.equal(dkp[rk].transpose(0, 1), dk[b, :, :lk[b]])
        assert torch.equal(dvp[rk].transpose(0, 1), dv[b, :, :lk[b]])


SPLIT_CASES = [
    # decoding: one new row per sequence at position L_k[b] - 1, GQA, a long ragged cache
    ("bf16_decode_gqa", W.BF16, 3, 8, 2, 1, 700, 128, 128, True, [699, 411, 522], [1, 1, 1], [700, 412, 523], 700),
    # a chunk of new rows against its history, per-sequence offsets
    ("bf16_chunk_mqa", W.BF16, 2, 8, 1, 48, 640, 128, 128, True, [592, 300], [48, 20], [640, 320], 640),
    ("f32_decode_d64", W.F32, 2, 4, 4, 1, 300, 64, 64, True, [299, 99], [1, 1], [300, 100], 300),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("parts", [0, 5])
def test_rope_decoding_through_the_split_forward(case, parts):
    """Rotary positions with the forward split over the keys, as a decoding
    step composes them: Q and K turned by attn_rope_apply (in practice new K
    rows are turned once as they enter the cache), then attn_fwd_splitkv on
    the turned tensors (automatic part count, or 5 parts); O and lse against
    the oracle's attention on rotated q, k."""
    torch = pytest.importorskip("torch")
    name, dtype, n_pos, d_h = case[0], case[1], case[-1], case[7]
    P.say(f"[rope] split forward {name} parts={parts}")
    inp, kw = _inputs(case)
    cs_host, cs = _table(n_pos, d_h)
    q, k, v = P.to_device(inp.Q), P.to_device(inp.K), P.to_device(inp.V)
    qt = A.rope_apply(q, k, v, cs, operand="q", **kw)
    kt = A.rope_apply(q, k, v, cs, operand="k", **kw)
    lq, lk = kw["seqlens_q"], kw["seqlens_k"]
    for b in range(q.shape[0]):  # rows past the active ones are not written by the rotation
        qt[b, :, lq[b]:] = 0
        kt[b, :, lk[b]:] = 0
    o, lse = A.fwd_splitkv(qt, kt, v, num_splits=parts, **kw)
    torch.cuda.synchronize()
    f64 = W.payload_to_f64
    go = np.zeros(inp.Q.shape[:3] + (inp.V.shape[-1],))
    ref = oracle.attention_backward_rope(f64(inp.Q), f64(inp.K), f64(inp.V), go, cs_host, **kw)
    errs = {"O": P.rel_err(P.to_f64(o), ref["O"]), "lse": P.rel_err(P.to_f64(lse), ref["lse"])}
    P.assert_within(errs, dtype, f"{name} parts={parts}")
    for b in range(q.shape[0]):
        assert (P.to_f64(o[b, :, lq[b]:]) == 0).all() and (P.to_f64(lse[b, :, lq[b]:]) == 0).all()
