"""Graph capture of the attention calls, and the empty-sum case of the
projection GEMMs.

The forward, the split forward and the backward allocate nothing and record
no memset, so a caller can capture them in a HIP graph.  The graph is replayed
several times with eager work between replays (new input values copied in,
outputs poisoned with NaN); every replay must reproduce the eager call on the
same inputs bit for bit (the kernels are deterministic), and the eager call
itself matches the float64 oracle (max|gpu - ref| / max|ref| <= 2e-2 bf16)."""

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


def test_forward_and_backward_replay_in_a_graph():
    import torch
    B, H_q, H_kv, n, d = 2, 8, 2, 300, 128
    kw = dict(causal=True, offset=[0, 17], seqlens_q=[300, 211], seqlens_k=[300, 240])
    P.say(f"[graph] bf16 B={B} H_q={H_q} H_kv={H_kv} n={n} d={d} {kw}")
    wl = W.custom_workload(W.BF16, B, H_q, H_kv, n, n, d, d, True, 0, "graph")
    sets = [W.make_custom_inputs(wl, seed=zlib.crc32(f"graph{i}".encode()) % 10000, **{
        "seqlens_q": kw["seqlens_q"], "seqlens_k": kw["seqlens_k"]}) for i in range(2)]
    for s in sets:
        s.mask_kwargs = lambda: kw
    host = [{k: P.to_device(getattr(s, k)) for k in ("Q", "K", "V", "GO")} for s in sets]

    q, k, v, do = (torch.empty_like(host[0][x]) for x in ("Q", "K", "V", "GO"))
    o, o_split = torch.empty_like(do), torch.empty_like(do)
    lse = torch.empty(B, H_q, n, dtype=torch.float32, device="cuda")
    lse_split = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    prob = A._problem_from(q, k, v, A._strides(o))
    ws = torch.empty(max(A.workspace_size(prob), 1), dtype=torch.uint8, device="cuda")
    ws_split = torch.empty(max(A.splitkv_workspace_size(prob, 4), 1), dtype=torch.uint8, device="cuda")

    def step():
        A.fwd(q, k, v, out=o, lse=lse, **kw)
        A.fwd_splitkv(q, k, v, num_splits=4, out=o_split, lse=lse_split, workspace=ws_split, **kw)
        A.bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)

    def load(i):
        for dst, key in ((q, "Q"), (k, "K"), (v, "V"), (do, "GO")):
            dst.copy_(host[i][key])
        for t in (o, o_split, lse, lse_split, dq, dk, dv):
            P.poison(t)

    outs = (o, lse, o_split, lse_split, dq, dk, dv)
    eager = []
    for i in range(2):
        load(i)
        step()
        torch.cuda.synchronize()
        eager.append([t.clone() for t in outs])
        got = {"O": P.to_f64(o), "lse": P.to_f64(lse), "GQ": P.to_f64(dq), "GK": P.to_f64(dk),
               "GV": P.to_f64(dv)}
        _, ref = P.compare_full(sets[i], {"O": o, "lse": lse, "GQ": dq, "GK": dk, "GV": dv})
        errs = {name: P.rel_err(got[name], ref[name]) for name in got}
        errs["O split"] = P.rel_err(P.to_f64(o_split), ref["O"])
        P.assert_within(errs, W.BF16, f"graph eager set {i}")

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep, i in enumerate([0, 1, 1, 0]):
        load(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("O", "lse", "O split", "lse split", "GQ", "GK", "GV"), outs, eager[i]):
            assert torch.equal(got, want), f"replay {rep} (input set {i}): {name} differs from the eager call"
        P.say(f"[graph] replay {rep} matches")


def test_gs_backward_replays_in_a_graph():
    """attn_bwd_gs (G_S kept in the workspace, three launches, no memset)
    captured with the forward: every replay reproduces the eager call."""
    import torch
    B, H_q, H_kv, n, d = 4, 32, 8, 800, 128
    kw = dict(causal=True, offset=0, seqlens_q=[800, 513, 700, 64], seqlens_k=[800, 513, 700, 64])
    prob0 = A.make_problem(B, H_q, H_kv, n, n, d, d, A.BF16)
    assert A.gs_workspace_size(prob0) > A.workspace_size(prob0)  # the G_S path, not its fallback
    P.say(f"[graph] G_S backward bf16 B={B} H_q={H_q} H_kv={H_kv} n={n} d={d}")
    wl = W.custom_workload(W.BF16, B, H_q, H_kv, n, n, d, d, True, 0, "graph_gs")
    sets = [W.make_custom_inputs(wl, seed=zlib.crc32(f"graph_gs{i}".encode()) % 10000,
                                 seqlens_q=kw["seqlens_q"], seqlens_k=kw["seqlens_k"]) for i in range(2)]
    host = [{k: P.to_device(getattr(s, k)) for k in ("Q", "K", "V", "GO")} for s in sets]
    q, k, v, do = (torch.empty_like(host[0][x]) for x in ("Q", "K", "V", "GO"))
    o = torch.empty_like(do)
    lse = torch.empty(B, H_q, n, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    prob = A._problem_from(q, k, v, A._strides(o))
    ws = torch.empty(A.gs_workspace_size(prob), dtype=torch.uint8, device="cuda")

    def step():
        A.fwd(q, k, v, out=o, lse=lse, **kw)
        A.bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, keep_gs=True, **kw)

    def load(i):
        for dst, key in ((q, "Q"), (k, "K"), (v, "V"), (do, "GO")):
            dst.copy_(host[i][key])
        for t in (o, lse, dq, dk, dv):
            P.poison(t)
        ws.fill_(0xFF)  # stale G_S would show as NaN

    outs = (o, lse, dq, dk, dv)
    eager = []
    for i in range(2):
        load(i)
        step()
        torch.cuda.synchronize()
        eager.append([t.clone() for t in outs])
        sets[i].mask_kwargs = lambda: kw
        errs, _ = P.compare_full(sets[i], {"O": o, "lse": lse, "GQ": dq, "GK": dk, "GV": dv})
        P.assert_within(errs, W.BF16, f"G_S graph eager set {i}")

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep, i in enumerate([0, 1, 1, 0]):
        load(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("O", "lse", "GQ", "GK", "GV"), outs, eager[i]):
            assert torch.equal(got, want), f"replay {rep} (input set {i}): {name} differs from the eager call"
        P.say(f"[graph] G_S replay {rep} matches")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_linear_backward_over_no_rows_gives_zero_weight_gradient(dtype):
    """With no rows, G_W = X^T G_Y is an empty sum: exactly zero (or left
    unchanged when accumulating)."""
    import torch
    P.say(f"[proj] linear over no rows {dtype}")
    tdt = torch.bfloat16 if dtype == W.BF16 else torch.float32
    d_in, d_out = 96, 40
    x = torch.empty(0, d_in, dtype=tdt, device="cuda")
    gy = torch.empty(0, d_out, dtype=tdt, device="cuda")
    w = torch.randn(d_in, d_out, device="cuda").to(tdt)
    gw = P.poison(torch.empty(d_in, d_out, dtype=tdt, device="cuda"))
    A.linear_bwd(x, w, gy, gw=gw, want_gx=False)
    torch.cuda.synchronize()
    assert (gw.float() == 0).all()
    gw.fill_(1.5)
    A.linear_bwd(x, w, gy, gw=gw, want_gx=False, accumulate=True)
    torch.cuda.synchronize()
    assert (gw.float() == 1.5).all()
