"""GPU parity where element offsets leave the 32-bit range.

Two layouts, each checked element by element against the float64 oracle
(max|gpu - ref| / max|ref| <= 1e-5 float32, <= 2e-2 bf16) through the forward,
the forward split over the keys and the backward:

* a batch stride of 2^31 + 256 elements, so every address of the second
  sequence lies past 2^31 elements (past 4 GiB of bf16, 8 GiB of float32);
* rows 2^24 + 512 elements apart with the heads interleaved inside a row
  ([B, n, H, d] storage), so a 64-row tile spans more than 2^31 bytes and the
  forward takes its general copy path, and the last rows of each tensor lie
  past 4 GiB;
* rows 2^26 + 512 elements apart in the same storage, so even a 32-row block
  of Q or G_O spans more than 4 GiB and the bf16 dK/dV pass takes its 64-bit
  copy path instead of buffer copies.

Each tensor sits in one large allocation with only its strided rows written
(about 35-70 GB of device memory per case, freed between cases)."""

import zlib

import numpy as np
import pytest

from exact_masked_scaled_amd import attn as A
from exact_masked_scaled_amd import workloads as W

import parity as P

pytestmark = pytest.mark.gpu

BATCH_STRIDE = 2 ** 31 + 256
ROW_STRIDE = 2 ** 24 + 512
ROW_STRIDE_HUGE = 2 ** 26 + 512
NEED_BYTES = 100 * 2 ** 30  # device memory the largest case needs, with margin

CASES = [
    # name, layout, dtype, B, H_q, H_kv, n_q, n_k, d, causal, offset, seqlens_q, seqlens_k
    ("batch_bf16", "batch", W.BF16, 2, 4, 2, 200, 200, 128, True, [0, 30], [200, 137], [200, 181]),
    ("batch_f32", "batch", W.F32, 2, 2, 1, 130, 150, 64, False, 0, [130, 77], [150, 99]),
    ("rows_bf16", "rows", W.BF16, 1, 4, 2, 160, 160, 128, True, 0, None, None),
    ("rows_huge_bf16", "rows_huge", W.BF16, 1, 4, 2, 40, 40, 128, True, 0, None, None),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if torch.cuda.get_device_properties(0).total_memory < NEED_BYTES:
        pytest.skip("needs about 100 GB of device memory")
    A.lib()


def _strided(torch, layout, dtype, B, H, n, d):
    """A [B, H, n, d] view into one allocation with 64-bit offsets."""
    if layout == "batch":
        size, strides = (B - 1) * BATCH_STRIDE + H * n * d, (BATCH_STRIDE, n * d, d, 1)
    else:
        rs = ROW_STRIDE if layout == "rows" else ROW_STRIDE_HUGE
        assert H * d <= rs
        size, strides = B * n * rs, (n * rs, d, rs, 1)
    buf = torch.empty(size, dtype=dtype, device="cuda")
    return torch.as_strided(buf, (B, H, n, d), strides)


def _put(view, host):
    """Write a host [B, H, n, d] array row by row (each piece small and dense)."""
    src = P.to_device(host)
    for b in range(view.shape[0]):
        for i in range(view.shape[2]):
            view[b, :, i].copy_(src[b, :, i])


def _get(view):
    out = np.empty(tuple(view.shape), dtype=np.float64)
    for b in range(view.shape[0]):
        for i in range(view.shape[2]):
            out[b, :, i] = P.to_f64(view[b, :, i])
    return out


def _poison(view):
    for b in range(view.shape[0]):
        for i in range(view.shape[2]):
            view[b, :, i].fill_(float("nan"))


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_offsets_beyond_32_bits(case):
    import torch
    name, layout, dtype, B, H_q, H_kv, n_q, n_k, d, causal, off, lq, lk = case
    label = f"[large offsets] {name} layout={layout} {dtype} B={B} H_q={H_q} H_kv={H_kv} n_q={n_q} n_k={n_k} d={d}"
    P.say(label)
    wl = W.custom_workload(dtype, B, H_q, H_kv, n_q, n_k, d, d, causal, 0, name)
    inp = W.make_custom_inputs(wl, seed=zlib.crc32(name.encode()) % 10000, seqlens_q=lq, seqlens_k=lk)
    kw = dict(causal=causal, offset=off, seqlens_q=lq, seqlens_k=lk)
    inp.mask_kwargs = lambda: kw
    f64 = W.payload_to_f64
    ref = P.oracle.attention_backward(f64(inp.Q), f64(inp.K), f64(inp.V), f64(inp.GO), **kw)

    tdt = torch.bfloat16 if dtype == W.BF16 else torch.float32
    shapes = {"q": (H_q, n_q), "k": (H_kv, n_k), "v": (H_kv, n_k), "o": (H_q, n_q)}
    try:
        t = {}
        for key, (H, n) in shapes.items():
            t[key] = _strided(torch, layout, tdt, B, H, n, d)
            t["d" + key] = _strided(torch, layout, tdt, B, H, n, d)
        _put(t["q"], inp.Q), _put(t["k"], inp.K), _put(t["v"], inp.V), _put(t["do"], inp.GO)
        for key in ("o", "dq", "dk", "dv"):
            _poison(t[key])
        lse = P.poison(torch.empty(B, H_q, n_q, dtype=torch.float32, device="cuda"))
        o, lse = A.fwd(t["q"], t["k"], t["v"], out=t["o"], lse=lse, **kw)
        dq, dk, dv = A.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], dq=t["dq"], dk=t["dk"], dv=t["dv"], **kw)
        torch.cuda.synchronize()
        got = {"O": _get(o), "lse": P.to_f64(lse), "GQ": _get(dq), "GK": _get(dk), "GV": _get(dv)}
        errs = {n: P.rel_err(got[n], ref[n]) for n in P.TENSORS}
        P.assert_within(errs, dtype, label)

        _poison(t["o"])
        lse2 = P.poison(torch.empty(B, H_q, n_q, dtype=torch.float32, device="cuda"))
        o2, lse2 = A.fwd_splitkv(t["q"], t["k"], t["v"], num_splits=3, out=t["o"], lse=lse2, **kw)
        torch.cuda.synchronize()
        errs = {"O": P.rel_err(_get(o2), ref["O"]), "lse": P.rel_err(P.to_f64(lse2), ref["lse"])}
        P.assert_within(errs, dtype, label + " split forward, 3 parts")
    finally:
        t = o = o2 = dq = dk = dv = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
