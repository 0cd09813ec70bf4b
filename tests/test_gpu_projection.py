"""GPU parity of the projections (attn_linear_fwd / attn_linear_bwd) and of
self-attention with its projections (attn_self_attention_fwd / _bwd) through
the C ABI, against the float64 oracle (oracle/projection.py) on the same
seeded, rounded inputs.

Tolerance: max|gpu - ref| / max|ref| per tensor, 1e-5 for float32 I/O and
2e-2 for bf16 I/O (as for the core; the bf16 path also rounds the projected
Q, K, V and the gradients G_Q, G_K, G_V to bf16 between the products).
Rows of padding get exact zeros in G_X, and a poisoned output buffer must not
leak into a result that overwrites it."""

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


def _draw(rng, shape, dtype, scale=1.0):
    x = rng.standard_normal(shape) * scale
    if dtype == W.BF16:
        return W.bf16_bits(W.round_to_bf16(x))
    return x.astype(np.float32)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_linear_parity(dtype):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(17)
    rows, d_in, d_out = 300, 192, 136
    P.say(f"[proj] linear {dtype}")
    # X is a column block of a wider matrix (row stride > width)
    Xw = _draw(rng, (rows, d_in + 64), dtype)
    Wm = _draw(rng, (d_in, d_out), dtype, 1 / np.sqrt(d_in))
    GY = _draw(rng, (rows, d_out), dtype)
    xw, w, gy = P.to_device(Xw), P.to_device(Wm), P.to_device(GY)
    x = xw[:, 32:32 + d_in]
    y = A.linear_fwd(x, w, out=P.poison(torch.empty(rows, d_out, dtype=x.dtype, device=x.device)))
    gx_buf = P.poison(torch.empty_like(xw))
    gx = gx_buf[:, 32:32 + d_in]
    gw = P.poison(torch.empty_like(w))
    A.linear_bwd(x, w, gy, gx=gx, gw=gw)
    torch.cuda.synchronize()
    f64 = W.payload_to_f64
    X64, W64, G64 = f64(Xw)[:, 32:32 + d_in], f64(Wm), f64(GY)
    errs = {"Y": P.rel_err(P.to_f64(y), X64 @ W64), "G_X": P.rel_err(P.to_f64(gx), G64 @ W64.T),
            "G_W": P.rel_err(P.to_f64(gw), X64.T @ G64)}
    P.assert_within(errs, dtype, f"linear {dtype}")
    # columns outside the block are untouched
    assert torch.isnan(gx_buf[:, :32].float()).all() and torch.isnan(gx_buf[:, 32 + d_in:].float()).all()
    # accumulate adds a second contribution
    gx2, gw2 = gx_buf.clone()[:, 32:32 + d_in], gw.clone()
    A.linear_bwd(x, w, gy, gx=gx2, gw=gw2, accumulate=True)
    torch.cuda.synchronize()
    e2 = {"G_X": P.rel_err(P.to_f64(gx2), 2 * (G64 @ W64.T)), "G_W": P.rel_err(P.to_f64(gw2), 2 * (X64.T @ G64))}
    P.assert_within(e2, dtype, f"linear accumulate {dtype}")


def test_caller_owned_gemm_context():
    """The projections run on a GEMM context the caller creates and destroys:
    a context made explicitly gives the same products as the default one,
    and a destroyed context's replacement works on the same stream."""
    torch = pytest.importorskip("torch")
    P.say("[proj] caller-owned GEMM context")
    rng = np.random.default_rng(3)
    x = P.to_device(_draw(rng, (130, 64), W.BF16))
    w = P.to_device(_draw(rng, (64, 96), W.BF16, 1 / 8))
    ref = A.linear_fwd(x, w)
    for _ in range(2):
        ctx = A.GemmContext()
        y = A.linear_fwd(x, w, gemm=ctx, out=P.poison(torch.empty_like(ref)))
        gx, gw = A.linear_bwd(x, w, y, gemm=ctx)
        torch.cuda.synchronize()
        ctx.close()
        assert torch.equal(y, ref)
        assert torch.isfinite(gx.float()).all() and torch.isfinite(gw.float()).all()


SELF_CASES = [
    # (name, dtype, B, n, d_model, H_q, H_kv, d_h, d_v, causal, lens)
    ("bf16_gqa_causal_lens", W.BF16, 2, 200, 256, 4, 2, 128, 128, True, [200, 131]),
    ("bf16_mha_full_dv64", W.BF16, 2, 96, 128, 2, 2, 128, 64, False, None),
    ("f32_d64_causal", W.F32, 1, 80, 64, 2, 1, 64, 64, True, None),
]


@pytest.mark.parametrize("case", SELF_CASES, ids=lambda c: c[0])
def test_self_attention_parity(case):
    torch = pytest.importorskip("torch")
    name, dtype, B, n, d_model, H_q, H_kv, d_h, d_v, causal, lens = case
    P.say(f"[proj] self-attention {name}")
    wl = W.custom_workload(dtype, B, H_q, H_kv, n, n, d_h, d_v, causal, 0, name)
    inp = W.make_projection_inputs(wl, d_model, seed=zlib.crc32(name.encode()) % 10000, seqlens=lens)
    x, w, do = P.to_device(inp.X), P.to_device(inp.W), P.to_device(inp.GO)
    kw = dict(H_q=H_q, H_kv=H_kv, d_h=d_h, d_v=d_v, causal=causal, seqlens_q=lens, seqlens_k=lens)
    qkv, o, lse = A.self_attention_fwd(x, w, **kw)
    gx, gw = A.self_attention_bwd(x, w, qkv, o, lse, do, gx=P.poison(torch.empty_like(x)),
                                  gw=P.poison(torch.empty_like(w)), **kw)
    torch.cuda.synchronize()
    f64 = W.payload_to_f64
    ref = oracle.self_attention_backward(f64(inp.X), f64(inp.W), f64(inp.GO), H_q=H_q, H_kv=H_kv, d_h=d_h, d_v=d_v,
                                         causal=causal, seqlens_q=lens, seqlens_k=lens)
    errs = {"O": P.rel_err(P.to_f64(o), ref["O"]), "lse": P.rel_err(P.to_f64(lse), ref["lse"]),
            "G_X": P.rel_err(P.to_f64(gx), ref["G_X"]), "G_W": P.rel_err(P.to_f64(gw), ref["G_W"])}
    P.assert_within(errs, dtype, name)
    if lens is not None:
        for b, L in enumerate(lens):
            assert (P.to_f64(gx[b, L:]) == 0).all()


def test_self_attention_packed_parity():
    torch = pytest.importorskip("torch")
    lens = [37, 150, 1, 96]
    B, n, d_model, H_q, H_kv, d_h = len(lens), max(lens), 256, 4, 2, 128
    wl = W.custom_workload(W.BF16, B, H_q, H_kv, n, n, d_h, d_h, True, 0, "proj_packed")
    inp = W.make_projection_inputs(wl, d_model, seed=31, seqlens=lens)
    P.say("[proj] self-attention packed")
    cu = [0] + np.cumsum(lens).astype(int).tolist()
    Xp = np.concatenate([inp.X[b, :L] for b, L in enumerate(lens)], axis=0)
    GOp = np.ascontiguousarray(np.concatenate([inp.GO[b, :, :L].transpose(1, 0, 2) for b, L in enumerate(lens)],
                                              axis=0))
    x, w, do = P.to_device(Xp), P.to_device(inp.W), P.to_device(GOp)
    kw = dict(H_q=H_q, H_kv=H_kv, d_h=d_h, d_v=d_h, causal=True, cu_seqlens=cu)
    qkv, o, lse = A.self_attention_fwd(x, w, **kw)
    gx, gw = A.self_attention_bwd(x, w, qkv, o, lse, do, **kw)
    torch.cuda.synchronize()
    f64 = W.payload_to_f64
    ref = oracle.self_attention_backward(f64(Xp), f64(inp.W), f64(GOp), H_q=H_q, H_kv=H_kv, d_h=d_h, d_v=d_h,
                                         causal=True, cu_seqlens=cu)
    errs = {"O": P.rel_err(P.to_f64(o), ref["O"]), "lse": P.rel_err(P.to_f64(lse), ref["lse"]),
            "G_X": P.rel_err(P.to_f64(gx), ref["G_X"]), "G_W": P.rel_err(P.to_f64(gw), ref["G_W"])}
    P.assert_within(errs, W.BF16, "packed self-attention")


def _heads(t2d, B, n, H, d, col0):
    """Column block [col0, col0 + H d) of a [B n, C] matrix as [B, H, n, d]."""
    return t2d[:, col0:col0 + H * d].view(B, n, H, d).permute(0, 2, 1, 3)


@pytest.mark.parametrize("causal", [False, True])
def test_cross_attention_recipe(causal):
    """Cross-attention from the parts: Q = X_q W_q and [K | V] = X_kv W_kv by
    attn_linear_fwd, the core on strided views of those products, the core's
    gradients written into views of two gradient matrices, and one
    attn_linear_bwd per input (each input's branches only)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(41 + causal)
    B, n_q, n_k, d_q, d_kv, H_q, H_kv, d_h, d_v = 2, 64, 160, 192, 128, 4, 2, 128, 64
    dt = W.BF16
    Xq, Xkv = _draw(rng, (B * n_q, d_q), dt), _draw(rng, (B * n_k, d_kv), dt)
    Wq = _draw(rng, (d_q, H_q * d_h), dt, 1 / np.sqrt(d_q))
    Wkv = _draw(rng, (d_kv, H_kv * (d_h + d_v)), dt, 1 / np.sqrt(d_kv))
    GO = _draw(rng, (B, H_q, n_q, d_v), dt)
    lens_k = [160, 97]
    kw = dict(causal=causal, offset=n_k - n_q if causal else 0, seqlens_k=lens_k)
    P.say(f"[proj] cross-attention recipe causal={causal}")
    xq, xkv, wq, wkv, do = (P.to_device(a) for a in (Xq, Xkv, Wq, Wkv, GO))
    qm = A.linear_fwd(xq, wq)
    kvm = A.linear_fwd(xkv, wkv)
    q = _heads(qm, B, n_q, H_q, d_h, 0)
    k = _heads(kvm, B, n_k, H_kv, d_h, 0)
    v = _heads(kvm, B, n_k, H_kv, d_v, H_kv * d_h)
    o, lse = A.fwd(q, k, v, **kw)
    gqm, gkvm = torch.empty_like(qm), torch.empty_like(kvm)
    A.bwd(q, k, v, o, lse, do, dq=_heads(gqm, B, n_q, H_q, d_h, 0), dk=_heads(gkvm, B, n_k, H_kv, d_h, 0),
          dv=_heads(gkvm, B, n_k, H_kv, d_v, H_kv * d_h), **kw)
    gxq, gwq = A.linear_bwd(xq, wq, gqm)
    gxkv, gwkv = A.linear_bwd(xkv, wkv, gkvm)
    torch.cuda.synchronize()
    f64 = W.payload_to_f64
    ref = oracle.cross_attention_backward(f64(Xq).reshape(B, n_q, d_q), f64(Xkv).reshape(B, n_k, d_kv), f64(Wq),
                                          f64(Wkv), f64(GO), H_q=H_q, H_kv=H_kv, d_h=d_h, d_v=d_v, **kw)
    errs = {"O": P.rel_err(P.to_f64(o), ref["O"]),
            "G_Xq": P.rel_err(P.to_f64(gxq).reshape(B, n_q, d_q), ref["G_Xq"]),
            "G_Xkv": P.rel_err(P.to_f64(gxkv).reshape(B, n_k, d_kv), ref["G_Xkv"]),
            "G_Wq": P.rel_err(P.to_f64(gwq), ref["G_Wq"]), "G_Wkv": P.rel_err(P.to_f64(gwkv), ref["G_Wkv"])}
    P.assert_within(errs, dt, f"cross causal={causal}")


def test_separate_weights_sum_through_accumulate():
    """Three weights held apart: G_X summed with accumulate equals the fused
    product over [W_Q | W_K | W_V] (to float32 summation order)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    rows, d, widths = 256, 128, (256, 128, 128)
    dt = W.F32
    X = _draw(rng, (rows, d), dt)
    Ws = [_draw(rng, (d, c), dt, 1 / np.sqrt(d)) for c in widths]
    Gs = [_draw(rng, (rows, c), dt) for c in widths]
    P.say("[proj] separate weights")
    x = P.to_device(X)
    gx = P.poison(torch.empty_like(x))
    for i, (Wi, Gi) in enumerate(zip(Ws, Gs)):
        A.linear_bwd(x, P.to_device(Wi), P.to_device(Gi), gx=gx, accumulate=i > 0, want_gw=False)
    fused, _ = A.linear_bwd(x, P.to_device(np.concatenate(Ws, axis=1)), P.to_device(np.concatenate(Gs, axis=1)),
                            want_gw=False)
    torch.cuda.synchronize()
    assert P.rel_err(P.to_f64(gx), P.to_f64(fused)) <= 1e-5
