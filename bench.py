#!/usr/bin/env python3
"""Throughput of exact masked scaled dot-product attention, forward + backward.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--uniform-len N]

One step = the whole hot path over one batch of synthetic input: the forward
(O and lse; split over the keys where the library's automatic part count
divides it) and the backward's two passes (the query-stationary pass: D and
G_Q; the key-stationary pass: G_K and G_V), all through the C ABI on one HIP
stream, inputs resident in HBM.  Default workload: bf16 causal GQA with key and
row padding, B=8, H_q=32, H_kv=8, n=4096, d=128 (lengths drawn in [2048, 4096]).
The other configurations (and this one with every length 4096, and this one
with its sequences packed without padding rows) follow in `other_workloads`,
timed over fewer steps.

Prints ONE JSON line.  `value` is algorithmic TFLOP/s: only visible
(query, key) pairs are credited, 2(d_h + d_v) FLOPs per pair forward and
2(3 d_h + 2 d_v) backward.  `roofline` describes the dominant kernel, timed
with HIP events on the stream it is launched on; `cpu_baseline` times the
float64 oracle on a bounded sample of the same workload on the host cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense MFMA, published
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd+bwd TFLOP/s and % of MFMA peak (bf16 causal GQA, n=4096)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_dkdv_causal_gqa_b8_n4096_traffic.txt")
KERNEL_SOURCES = ("attn_bwd_quad.hip", "attn_device.h", "attn_internal.h")
DOMINANT = "bwd_dkdv"
BACKWARD_KIND = {True: "score gradients kept (per-row pass, dK/dV pass storing G_S, dQ product)",
                 False: "two passes (dQ pass and dK/dV pass, both recomputing S and dP)"}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_masked_scaled_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(units_per_launch_bytes):
    """HBM bytes per launch of the backward main kernel from the committed
    rocprofv3 counter summary, or None when the kernel source has changed
    since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, seconds: float):
    """The float64 oracle as it stands, on whole (sequence, query head) pairs of
    the same workload until about `seconds` of host time is spent."""
    import numpy as np

    import oracle
    from exact_masked_scaled_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = len(os.sched_getaffinity(0))
    wl = inp.wl
    lq = inp.seqlens_q or [wl.n_q] * wl.B
    lk = inp.seqlens_k or [wl.n_k] * wl.B
    done_pairs, heads, t_used = 0, [], 0.0
    order = [(b, r) for b in range(wl.B) for r in range(wl.H_q)]
    t_start = time.perf_counter()
    for b, r in order:
        g = oracle.kv_group(r, wl.H_q, wl.H_kv)
        M = oracle.visible_mask(wl.n_q, wl.n_k, lq[b], lk[b], wl.causal, wl.offset)
        q = W.payload_to_f64(inp.Q[b, r])
        k = W.payload_to_f64(inp.K[b, g])
        v = W.payload_to_f64(inp.V[b, g])
        go = W.payload_to_f64(inp.GO[b, r])
        t0 = time.perf_counter()
        f = oracle.head_forward(q, k, v, M)
        oracle.head_backward(q, k, v, f["A"], M, go)
        t_used += time.perf_counter() - t0
        done_pairs += int(M.sum())
        heads.append((b, r))
        if time.perf_counter() - t_start >= seconds:
            break
    flop = 2 * done_pairs * (wl.d_h + wl.d_v) + 2 * done_pairs * (3 * wl.d_h + 2 * wl.d_v)
    return {
        "value": flop / t_used / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle, forward+backward of {len(heads)} whole (sequence, query head) "
                   f"pairs of the same workload (first: {heads[0]}, last: {heads[-1]}), "
                   f"{t_used:.1f} s; algorithmic FLOPs of the visible pairs / oracle time"),
    }


def kernel_report(wl, work, kern_ms):
    """Per kernel of a step: time, algorithmic and executed TFLOP/s and
    fractions of the dtype's dense MFMA peak; the dominant (longest) kernel
    and its algorithmic rate.  Algorithmic FLOPs are credited without double
    counting the recomputed products: the dQ pass gets the G_Q product only,
    the dK/dV pass the recomputed scores, dP, G_V and G_K.  With the score
    gradients kept, the per-row pass has no products and the dQ product
    from the stored gradients is credited 2 d_h per pair."""
    peak = PEAK_TFLOPS[wl.dtype]
    P, dh, dv_ = work["pairs"], wl.d_h, wl.d_v
    alg = {"fwd": 2 * P * (dh + dv_), "bwd_dq": 2 * P * dh, "bwd_dkdv": 2 * P * (2 * dh + 2 * dv_),
           "bwd_rows": 0, "bwd_dq_gs": 2 * P * dh}
    executed = {"fwd": 2 * P * (dh + dv_), "bwd_dq": 2 * P * (2 * dh + dv_), "bwd_dkdv": 2 * P * (2 * dh + 2 * dv_),
                "bwd_rows": 0, "bwd_dq_gs": 2 * P * dh}
    # the two passes of the G_S backward that are bound by HBM: algorithmic
    # bytes (per-row pass: O and G_O read, lse read, -D and lse log2 e
    # written; G_Q product: 2 bytes of G_S per visible pair, K read once,
    # G_Q written), against the 8 TB/s peak
    s = 2 if wl.dtype == "bf16" else 4
    hbm_bytes = {"bwd_rows": work["active_q_rows"] * (2 * dv_ * s + 4 + 8),
                 "bwd_dq_gs": 2 * P + (work["active_k_rows"] + work["active_q_rows"]) * dh * s}
    kernels = {}
    for n, t in kern_ms.items():
        sec = t * 1e-3
        kernels[n] = {"ms": round(t, 4),
                      "algorithmic_TFLOP/s": round(alg[n] / sec / 1e12, 2),
                      "frac_of_peak": round(alg[n] / sec / 1e12 / peak, 4),
                      "executed_MFMA_TFLOP/s": round(executed[n] / sec / 1e12, 2),
                      "executed_frac_of_peak": round(executed[n] / sec / 1e12 / peak, 4)}
        if n in hbm_bytes:
            kernels[n]["algorithmic_GB/s"] = round(hbm_bytes[n] / sec / 1e9, 1)
            kernels[n]["frac_of_hbm_peak"] = round(hbm_bytes[n] / sec / 1e9 / PEAK_HBM_GBS, 4)
    dominant = max(kern_ms, key=kern_ms.get)
    return kernels, dominant, alg[dominant] / (kern_ms[dominant] * 1e-3) / 1e12


def measure(torch, attn, W, wl, uniform_len, steps, warmup, packed=False, keep_gs=True):
    """Time `steps` steps (forward, then the backward) of one workload with
    its inputs resident; returns (inputs, work, ms per step, ms per kernel,
    device, forward split?, score gradients kept?).  The backward keeps the
    score gradients G_S (per-row pass, dK/dV pass storing G_S, dQ product)
    where the library supports it and ``keep_gs`` is set, else it runs the
    dQ pass and the dK/dV pass, both recomputing S and dP.
    With ``packed`` the same sequences are stored one after another without
    padding rows ([rows, H, d] tensors and row offsets): same visible pairs."""
    import numpy as np

    inp = W.make_inputs(wl, uniform_len=uniform_len)
    kw = inp.mask_kwargs()
    work = W.work(wl, inp.seqlens_q, inp.seqlens_k)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    if packed:
        lq = inp.seqlens_q or [wl.n_q] * wl.B
        lk = inp.seqlens_k or [wl.n_k] * wl.B

        def pack(X, lens):  # [B, H, n, d] -> [sum(lens), H, d]
            return np.ascontiguousarray(np.concatenate([X[b, :, :L].transpose(1, 0, 2)
                                                        for b, L in enumerate(lens)], axis=0))
        cu_q = [0] + np.cumsum(lq).astype(int).tolist()
        cu_k = [0] + np.cumsum(lk).astype(int).tolist()
        q, do = dev(pack(inp.Q, lq)), dev(pack(inp.GO, lq))
        k, v = dev(pack(inp.K, lk)), dev(pack(inp.V, lk))
        o = torch.empty(cu_q[-1], wl.H_q, wl.d_v, dtype=q.dtype, device=q.device)
        lse = torch.empty(wl.H_q, cu_q[-1], dtype=torch.float32, device=q.device)
        kw = dict(causal=wl.causal, offset=wl.offset, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
                  max_seqlen_q=wl.n_q, max_seqlen_k=wl.n_k)
    else:
        q, k, v, do = dev(inp.Q), dev(inp.K), dev(inp.V), dev(inp.GO)
        o = torch.empty(wl.B, wl.H_q, wl.n_q, wl.d_v, dtype=q.dtype, device=q.device)
        lse = torch.empty(wl.B, wl.H_q, wl.n_q, dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    pf = attn._problem_from(q, k, v, attn._strides(o), kw.get("cu_seqlens_q"), kw.get("cu_seqlens_k"),
                            kw.get("max_seqlen_q"), kw.get("max_seqlen_k"))
    gs = keep_gs and attn.gs_workspace_size(pf) > attn.workspace_size(pf)
    need = attn.gs_workspace_size(pf) if gs else attn.workspace_size(pf)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    staged = attn.StagedBackward(q, k, v, o, lse, do, dq, dk, dv, ws, **kw)
    stream = torch.cuda.current_stream()
    if gs:
        names = ("fwd", "bwd_rows", "bwd_dkdv", "bwd_dq_gs")
        backward = [lambda: staged.gs_stage(0, stream), lambda: staged.gs_stage(1, stream),
                    lambda: staged.gs_stage(2, stream)]
    else:
        names = ("fwd", "bwd_dq", "bwd_dkdv")
        backward = [lambda: staged.dq(stream), lambda: staged.dkdv(stream)]
    # the forward split over the keys where the library's automatic part
    # count divides it (few query rows per KV head against long key ranges)
    split_fwd = attn.splitkv_workspace_size(pf, 0) > attn.splitkv_workspace_size(pf, 1)
    ws_f = torch.empty(max(attn.splitkv_workspace_size(pf, 0), 1), dtype=torch.uint8, device=q.device) \
        if split_fwd else None

    def forward():
        if split_fwd:
            attn.fwd_splitkv(q, k, v, num_splits=0, out=o, lse=lse, workspace=ws_f, stream=stream, **kw)
        else:
            attn.fwd(q, k, v, out=o, lse=lse, stream=stream, **kw)

    def step(events=None):
        if events is not None:
            events[0].record(stream)
        forward()
        if events is not None:
            events[1].record(stream)
        for j, run in enumerate(backward):
            run()
            if events is not None:
                events[j + 2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    kern_ms = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j, n in enumerate(names)}
    device = q.device
    del q, k, v, do, o, lse, dq, dk, dv, ws, staged, ws_f, backward
    torch.cuda.synchronize()
    return inp, work, ms_per_step, kern_ms, device, split_fwd, gs


def measure_forward_split(torch, attn, W, wl, steps, warmup):
    """Forward only, unsplit (attn_fwd) against split over the keys
    (attn_fwd_splitkv, automatic part count), inputs resident; median ms per
    call."""
    import numpy as np

    inp = W.make_inputs(wl, with_grad=False) if wl.wid in W.WORKLOADS else \
        W.make_custom_inputs(wl, seed=2000, with_grad=False)
    kw = inp.mask_kwargs()

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()
    q, k, v = dev(inp.Q), dev(inp.K), dev(inp.V)
    o = torch.empty(wl.B, wl.H_q, wl.n_q, wl.d_v, dtype=q.dtype, device=q.device)
    lse = torch.empty(wl.B, wl.H_q, wl.n_q, dtype=torch.float32, device=q.device)
    prob = attn._problem_from(q, k, v, attn._strides(o))
    ws = torch.empty(max(attn.splitkv_workspace_size(prob, 0), 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream()
    calls = {"unsplit": lambda: attn.fwd(q, k, v, out=o, lse=lse, stream=stream, **kw),
             "split": lambda: attn.fwd_splitkv(q, k, v, num_splits=0, out=o, lse=lse, workspace=ws,
                                               stream=stream, **kw)}
    out = {}
    for name, fn in calls.items():
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        # one event pair per call and the median: these calls last tens of
        # microseconds, so a stall of the submitting thread would otherwise
        # count as GPU time
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        out[name] = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
    work = W.work(wl, inp.seqlens_q, inp.seqlens_k)
    del q, k, v, o, lse, ws
    return out, work


def measure_rope(torch, attn, W, wl, steps, warmup):
    """Rotary positions on the same workload: forward and backward with the
    rotation (attn_fwd_rope, attn_bwd_rope) against without (attn_fwd,
    attn_bwd), and the standalone rotation of Q; ms per call, inputs resident."""
    import numpy as np

    inp = W.make_inputs(wl)
    kw = inp.mask_kwargs()

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()
    q, k, v, do = dev(inp.Q), dev(inp.K), dev(inp.V), dev(inp.GO)
    cs = torch.from_numpy(W.rotary_table(max(wl.n_q, wl.n_k) + max(wl.offset, 0), wl.d_h)).cuda()
    # each backward reads the O and lse of its own forward
    o, o_r = (torch.empty(wl.B, wl.H_q, wl.n_q, wl.d_v, dtype=q.dtype, device=q.device) for _ in range(2))
    lse, lse_r = (torch.empty(wl.B, wl.H_q, wl.n_q, dtype=torch.float32, device=q.device) for _ in range(2))
    dq, dk, dv, qt = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(q)
    prob = attn._problem_from(q, k, v, attn._strides(o))
    ws = torch.empty(max(attn.rope_workspace_size(prob, backward=True), 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream()
    calls = {
        "fwd": lambda: attn.fwd(q, k, v, out=o, lse=lse, stream=stream, **kw),
        "bwd": lambda: attn.bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, stream=stream, **kw),
        "fwd_rope": lambda: attn.fwd_rope(q, k, v, cs, out=o_r, lse=lse_r, workspace=ws, stream=stream, **kw),
        "bwd_rope": lambda: attn.bwd_rope(q, k, v, o_r, lse_r, do, cs, dq=dq, dk=dk, dv=dv, workspace=ws,
                                          stream=stream, **kw),
        "rotate_q": lambda: attn.rope_apply(q, k, v, cs, operand="q", out=qt, stream=stream, **kw),
    }
    # the calls interleaved, one event pair each, medians over the steps (so
    # clock and cache state drift affects every variant alike)
    for _ in range(warmup):
        for fn in calls.values():
            fn()
    evs = {n: [] for n in calls}
    for _ in range(steps):
        for name, fn in calls.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            evs[name].append((e0, e1))
    torch.cuda.synchronize()
    out = {n: float(np.median([a.elapsed_time(b) for a, b in ev])) for n, ev in evs.items()}
    rows_q = sum(inp.seqlens_q) if inp.seqlens_q else wl.B * wl.n_q
    es = 2 if wl.dtype == W.BF16 else 4
    rot_bytes = 2 * rows_q * wl.H_q * wl.d_h * es  # each active Q element read and written once
    del q, k, v, do, o, lse, o_r, lse_r, dq, dk, dv, qt, ws, cs
    return {"workload": wl.name,
            "fwd_ms": round(out["fwd"], 4), "fwd_rope_ms": round(out["fwd_rope"], 4),
            "bwd_ms": round(out["bwd"], 4), "bwd_rope_ms": round(out["bwd_rope"], 4),
            "step_overhead_pct": round(100 * (out["fwd_rope"] + out["bwd_rope"] - out["fwd"] - out["bwd"])
                                       / (out["fwd"] + out["bwd"]), 2),
            "rotate_q_ms": round(out["rotate_q"], 4),
            "rotate_q_GB/s_algorithmic": round(rot_bytes / (out["rotate_q"] * 1e-3) / 1e9, 1),
            "steps": steps, "warmup": warmup}


def measure_projected(torch, attn, W, wl, d_model, steps, warmup):
    """Self-attention with its projections on the same sequences, packed (no
    padding rows enter the products): forward = [Q|K|V] = X W_qkv then the
    core; backward = the core's backward into [G_Q|G_K|G_V], then G_W and G_X
    (the three branches summed by one product).  Interleaved per-call medians,
    inputs resident; the products alone are timed too."""
    import numpy as np

    rng = np.random.default_rng(W.default_seed(wl.wid))
    lq, lk = W.draw_lengths(wl, rng)
    lens = lq or [wl.n_q] * wl.B
    inp = W.make_projection_inputs(wl, d_model, seed=W.default_seed(wl.wid) + 500, seqlens=lens)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()
    cu = [0] + np.cumsum(lens).astype(int).tolist()
    rows = cu[-1]
    x = dev(np.ascontiguousarray(np.concatenate([inp.X[b, :L] for b, L in enumerate(lens)], axis=0)))
    do = dev(np.ascontiguousarray(np.concatenate([inp.GO[b, :, :L].transpose(1, 0, 2)
                                                  for b, L in enumerate(lens)], axis=0)))
    w = dev(inp.W)
    del inp
    C = w.shape[1]
    kw = dict(H_q=wl.H_q, H_kv=wl.H_kv, d_h=wl.d_h, d_v=wl.d_v, causal=wl.causal, offset=wl.offset, cu_seqlens=cu,
              max_seqlen=wl.n_q)
    qkv = torch.empty(rows, C, dtype=x.dtype, device=x.device)
    o = torch.empty(rows, wl.H_q, wl.d_v, dtype=x.dtype, device=x.device)
    lse = torch.empty(wl.H_q, rows, dtype=torch.float32, device=x.device)
    gx, gw = torch.empty_like(x), torch.empty_like(w)
    prob = attn._self_problem(x, w, wl.H_q, wl.H_kv, wl.d_h, wl.d_v, attn._strides(o), cu, wl.n_q)
    ws = torch.empty(attn.self_attention_workspace_size(prob), dtype=torch.uint8, device=x.device)
    gqkv = torch.empty_like(qkv)
    stream = torch.cuda.current_stream()
    calls = {
        "fwd": lambda: attn.self_attention_fwd(x, w, qkv=qkv, out=o, lse=lse, stream=stream, **kw),
        "bwd": lambda: attn.self_attention_bwd(x, w, qkv, o, lse, do, gx=gx, gw=gw, workspace=ws, stream=stream,
                                               **kw),
        "gemm_qkv": lambda: attn.linear_fwd(x, w, out=qkv, stream=stream),
        "gemm_grads": lambda: attn.linear_bwd(x, w, gqkv, gx=gx, gw=gw, stream=stream),
    }
    for _ in range(warmup):
        for fn in calls.values():
            fn()
    evs = {n: [] for n in calls}
    for _ in range(steps):
        for name, fn in calls.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            evs[name].append((e0, e1))
    torch.cuda.synchronize()
    t = {n: float(np.median([a.elapsed_time(b) for a, b in ev])) for n, ev in evs.items()}
    work = W.work(wl, lq, lk)
    gemm_fwd = 2.0 * rows * d_model * C
    total = 3 * gemm_fwd + work["fwd_flop"] + work["bwd_flop"]
    del x, do, w, qkv, o, lse, gx, gw, ws, gqkv
    return {"workload": wl.name + f"_packed_dmodel{d_model}", "rows": rows, "d_model": d_model, "qkv_width": C,
            "fwd_ms": round(t["fwd"], 4), "bwd_ms": round(t["bwd"], 4),
            "step_TFLOP/s": round(total / ((t["fwd"] + t["bwd"]) * 1e-3) / 1e12, 2),
            "gemm_qkv_ms": round(t["gemm_qkv"], 4),
            "gemm_qkv_TFLOP/s": round(gemm_fwd / (t["gemm_qkv"] * 1e-3) / 1e12, 2),
            "gemm_grads_ms": round(t["gemm_grads"], 4),
            "gemm_grads_TFLOP/s": round(2 * gemm_fwd / (t["gemm_grads"] * 1e-3) / 1e12, 2),
            "steps": steps, "warmup": warmup}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--uniform-len", type=int, default=None,
                    help="replace the drawn sequence lengths by this length (e.g. 4096: unpadded)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="time only the selected workload (default: also every other configuration, briefly)")
    ap.add_argument("--two-pass", action="store_true",
                    help="run the backward as the dQ pass and the dK/dV pass (both recompute S and dP) "
                         "instead of keeping the score gradients")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after timing, run a plain elementwise copy of this many MiB (3 launches) "
                         "so HBM byte counters can be scaled against a kernel of known traffic")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this build has no multi-GPU path", file=sys.stderr)
        return 2

    import torch

    from exact_masked_scaled_amd import attn
    from exact_masked_scaled_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    attn.lib()  # fail loudly without the library
    wl = W.WORKLOADS[args.workload]
    inp, work, ms_per_step, kern_ms, dev_of, split_fwd, gs = measure(torch, attn, W, wl, args.uniform_len,
                                                                     args.steps, args.warmup,
                                                                     keep_gs=not args.two_pass)

    flop = work["fwd_flop"] + work["bwd_flop"]
    value = flop / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl.dtype]
    kernels, dominant, ach = kernel_report(wl, work, kern_ms)
    roof = {"kernel": dominant, "bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(ach / peak, 4),
            "traffic": load_traffic(None) if dominant == DOMINANT else None}

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "pct_of_peak": round(100 * value / peak, 2),
        "config": {
            "workload": wl.name, "B": wl.B, "H_q": wl.H_q, "H_kv": wl.H_kv, "n_q": wl.n_q,
            "n_k": wl.n_k, "d_h": wl.d_h, "d_v": wl.d_v, "causal": wl.causal, "offset": wl.offset,
            "seqlens_k": inp.seqlens_k, "seqlens_q": inp.seqlens_q, "seed": inp.seed,
            "visible_pairs": work["pairs"], "fwd_gflop": round(work["fwd_flop"] / 1e9, 3),
            "bwd_gflop": round(work["bwd_flop"] / 1e9, 3),
            "literal_formula_fwd_gflop": round(work["literal_fwd_flop"] / 1e9, 3),
        },
        "kernels": kernels,
        "forward": "split over keys" if split_fwd else "unsplit",
        "backward": BACKWARD_KIND[gs],
        "roofline": roof,
        "cpu_baseline": None,
    }
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev_of)
        c = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=c)  # reads and writes exactly n * 4 bytes
        torch.cuda.synchronize()
        result["copy_calibration"] = {"bytes_read": n * 4, "bytes_written": n * 4, "launches": 3}
    if not args.no_other_workloads:
        # every other configuration, shorter runs (the headline target is the one above)
        others = []
        # float32 at a size that is not launch-bound (the float32 workload is 16 K pairs)
        f32_large = W.custom_workload(W.F32, 4, 16, 16, 2048, 2048, 64, 64, False, 0,
                                      "mha_fp32_b4_h16_n2048_d64")
        for owl, ulen, pk in [(W.WORKLOADS[1], None, False), (f32_large, None, False),
                              (W.WORKLOADS[2], None, False), (W.WORKLOADS[4], None, False),
                              (W.WORKLOADS[5], None, False), (W.WORKLOADS[3], 4096, False),
                              (W.WORKLOADS[3], None, True)]:
            if owl.wid == args.workload and ulen == args.uniform_len and not pk:
                continue
            _, ow, oms, okern, _, osplit, ogs = measure(torch, attn, W, owl, ulen, 10, 3, packed=pk,
                                                        keep_gs=not args.two_pass)
            oflop = ow["fwd_flop"] + ow["bwd_flop"]
            ov = oflop / (oms * 1e-3) / 1e12
            label = owl.name + (f"_uniform{ulen}" if ulen else "") + ("_packed" if pk else "")
            okernels, odom, oach = kernel_report(owl, ow, okern)
            others.append({"workload": label, "dtype": owl.dtype,
                           "value": round(ov, 2), "unit": "TFLOP/s", "ms_per_step": round(oms, 4),
                           "pct_of_peak": round(100 * ov / PEAK_TFLOPS[owl.dtype], 2),
                           "visible_pairs": ow["pairs"], "kernels": okernels,
                           "roofline": {"kernel": odom, "bound": "mfma", "achieved": round(oach, 2),
                                        "peak": PEAK_TFLOPS[owl.dtype], "unit": "TFLOP/s",
                                        "frac": round(oach / PEAK_TFLOPS[owl.dtype], 4)},
                           "forward": "split over keys" if osplit else "unsplit",
                           "backward": BACKWARD_KIND[ogs], "steps": 10, "warmup": 3})
        result["other_workloads"] = others
        # forward only, split over the keys, where few query rows meet a long key range
        fsplit = []
        decode = W.custom_workload(W.BF16, 8, 32, 8, 1, 8192, 128, 128, True, 8191,
                                   "decode_gqa_bf16_b8_hq32_hkv8_nq1_nk8192_d128")
        for fwl in (W.WORKLOADS[5], W.WORKLOADS[4], decode):
            t, fw = measure_forward_split(torch, attn, W, fwl, 20, 3)
            s_ = 2 if fwl.dtype == W.BF16 else 4
            byts = s_ * (fwl.B * fwl.H_kv * fwl.n_k * (fwl.d_h + fwl.d_v)
                         + fwl.B * fwl.H_q * fwl.n_q * (fwl.d_h + fwl.d_v)) + 4 * fwl.B * fwl.H_q * fwl.n_q
            ent = {"workload": fwl.name, "unsplit_ms": round(t["unsplit"], 4), "split_ms": round(t["split"], 4),
                   "split_TFLOP/s": round(fw["fwd_flop"] / (t["split"] * 1e-3) / 1e12, 2),
                   "split_GB/s_algorithmic": round(byts / (t["split"] * 1e-3) / 1e9, 1),
                   "unsplit_TFLOP/s": round(fw["fwd_flop"] / (t["unsplit"] * 1e-3) / 1e12, 2)}
            fsplit.append(ent)
        result["forward_splitkv"] = fsplit
        # rotary positions on the headline workload
        result["rotary"] = measure_rope(torch, attn, W, wl, 10, 3)
        # with the Q/K/V projections (model width = the query heads' width)
        result["projected"] = measure_projected(torch, attn, W, wl, wl.H_q * wl.d_h, 10, 3)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
