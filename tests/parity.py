"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the float64 oracle on the same seeded (rounded) inputs, compare.

Tolerance metric, per tensor over the compared elements:
    max|gpu - ref| / max|ref|  <= 1e-5 (float32 I/O) or 2e-2 (bf16 I/O).
"""

from __future__ import annotations

import sys

import numpy as np

import oracle
from exact_masked_scaled_amd import attn as A
from exact_masked_scaled_amd import workloads as W

TOL = {W.F32: 1e-5, W.BF16: 2e-2}
TENSORS = ("O", "lse", "GQ", "GK", "GV")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def poison(t):
    import torch
    t.fill_(float("nan"))
    return t


def bench_forward_splits(prob) -> int:
    """The forward the benchmark times: split over the keys (automatic part
    count, 0) when the library's automatic count divides the problem,
    otherwise unsplit (1)."""
    return 0 if A.splitkv_workspace_size(prob, 0) > A.splitkv_workspace_size(prob, 1) else 1


def run_gpu(inp: W.Inputs, backward=True, poison_outputs=True, num_splits=1, keep_gs=False):
    """Forward (+ backward) on the GPU; returns device tensors.  num_splits 1
    runs attn_fwd; any other value runs attn_fwd_splitkv with that part count
    (0: automatic, the benchmark's choice).  keep_gs runs the backward as
    attn_bwd_gs."""
    import torch
    wl = inp.wl
    q, k, v = to_device(inp.Q), to_device(inp.K), to_device(inp.V)
    kw = inp.mask_kwargs()
    out = torch.empty(wl.B, wl.H_q, wl.n_q, wl.d_v, dtype=q.dtype, device=q.device)
    lse = torch.empty(wl.B, wl.H_q, wl.n_q, dtype=torch.float32, device=q.device)
    if poison_outputs:
        poison(out), poison(lse)
    if num_splits == 1:
        o, lse = A.fwd(q, k, v, out=out, lse=lse, **kw)
    else:
        prob = A._problem_from(q, k, v, A._strides(out))
        wsf = torch.full((max(A.splitkv_workspace_size(prob, num_splits), 1),), 0xFF, dtype=torch.uint8,
                         device=q.device)
        o, lse = A.fwd_splitkv(q, k, v, num_splits=num_splits, out=out, lse=lse, workspace=wsf, **kw)
    res = {"O": o, "lse": lse}
    if backward:
        do = to_device(inp.GO)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        prob = A._problem_from(q, k, v, A._strides(o))
        need = A.gs_workspace_size(prob) if keep_gs else A.workspace_size(prob)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        if poison_outputs:
            poison(dq), poison(dk), poison(dv)
            ws.fill_(0xFF)  # NaN bit patterns in the float32 workspace (and in kept G_S)
        dq, dk, dv = A.bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, keep_gs=keep_gs, **kw)
        res.update({"GQ": dq, "GK": dk, "GV": dv})
    torch.cuda.synchronize()
    return res


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    denom = float(np.max(np.abs(ref))) if ref.size else 0.0
    diff = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if not np.all(np.isfinite(got)):
        return float("inf")
    if denom == 0.0:
        return diff
    return diff / denom


def compare_full(inp: W.Inputs, gpu: dict, backward=True) -> dict:
    """Whole-tensor comparison against the oracle (small problems)."""
    f64 = W.payload_to_f64
    kw = inp.mask_kwargs()
    if backward:
        ref = oracle.attention_backward(f64(inp.Q), f64(inp.K), f64(inp.V), f64(inp.GO), **kw)
    else:
        ref = oracle.attention_forward(f64(inp.Q), f64(inp.K), f64(inp.V), **kw)
    errs = {}
    for name in TENSORS if backward else ("O", "lse"):
        errs[name] = rel_err(to_f64(gpu[name]), ref[name])
    return errs, ref


def compare_groups(inp: W.Inputs, gpu: dict, groups=None, progress=None, workers=4) -> dict:
    """Comparison per (sequence, KV head) group: every output of the query
    heads of the group and G_K/G_V of its KV head, against the oracle
    restricted to that group.  groups=None compares every group of the
    problem, i.e. every element of every output.  The error of a tensor is
    max|gpu - ref| / max|ref| over all compared elements."""
    wl = inp.wl
    kw = inp.mask_kwargs()
    if groups is None:
        groups = [(b, g) for b in range(wl.B) for g in range(wl.H_kv)]
    diff = {n: 0.0 for n in TENSORS}
    top = {n: 0.0 for n in TENSORS}
    finite = {n: True for n in TENSORS}
    Qf, Kf, Vf, GOf = _Lazy(inp.Q), _Lazy(inp.K), _Lazy(inp.V), _Lazy(inp.GO)
    host = {n: t.detach().float().cpu().numpy() for n, t in gpu.items()}

    def one(bg):
        b, g = bg
        o = oracle.attention_group(Qf, Kf, Vf, GOf, b, g, **kw)
        heads = o["heads"]
        res = {}
        for name in TENSORS:
            if name in ("GK", "GV"):
                got = host[name][b, g].astype(np.float64)
            else:
                got = host[name][b, heads[0]:heads[-1] + 1].astype(np.float64)
            ref = o[name]
            res[name] = (bool(np.all(np.isfinite(got))),
                         float(np.max(np.abs(got - ref))) if ref.size else 0.0,
                         float(np.max(np.abs(ref))) if ref.size else 0.0)
        return res

    # groups are independent: a few host threads (numpy's products and large
    # element-wise operations release the interpreter lock)
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(max_workers=min(workers, len(groups)) or 1) as ex:
        for idx, res in enumerate(ex.map(one, groups)):
            for name, (fin, d, t) in res.items():
                finite[name] &= fin
                diff[name] = max(diff[name], d)
                top[name] = max(top[name], t)
            if progress is not None and (idx + 1) % progress == 0:
                say(f"  compared {idx + 1}/{len(groups)} groups")
    out = {}
    for n in TENSORS:
        if not finite[n]:
            out[n] = float("inf")
        else:
            out[n] = diff[n] / top[n] if top[n] > 0 else diff[n]
    return out


def record(label: str, errs: dict, **extra):
    """Append one parity row (per-tensor errors) to the JSON-lines file named
    by ATTN_PARITY_TABLE, when that variable is set."""
    import json
    import os
    path = os.environ.get("ATTN_PARITY_TABLE")
    if not path:
        return
    with open(path, "a") as f:
        f.write(json.dumps({"case": label, **{k: float(v) for k, v in errs.items()}, **extra}) + "\n")


class _Lazy:
    """[b, h] indexing that widens one payload slice to float64 on demand."""

    def __init__(self, a):
        self.a = a
        self.shape = a.shape

    def __getitem__(self, idx):
        return W.payload_to_f64(self.a[idx])


def assert_within(errs: dict, dtype: str, label: str):
    tol = TOL[dtype]
    say(f"{label}: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f" (tol {tol:g})")
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    assert not bad, f"{label}: over tolerance {tol}: {bad}"
