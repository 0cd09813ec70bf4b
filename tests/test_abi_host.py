"""Host-only checks of the C ABI: the library loads, exports every function the
header declares, its structs match the header, and every argument error is
reported before anything touches a device (so these run without a GPU)."""

import ctypes
import os
import re

import pytest

from exact_masked_scaled_amd import attn as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def lib_or_skip():
    if not os.path.exists(A.LIB_PATH):
        pytest.fail(f"{A.LIB_PATH} not built (run __graft_entry__.build())")
    return A.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function():
    L = lib_or_skip()
    names = declared_functions()
    assert set(names) == set(A.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n
    assert L.attn_version() >= 100


def test_struct_layouts_match_header():
    # attn_mask: int32, int32, int64, ptr, ptr, ptr
    # attn_problem: 8 x int32 + 12 x int64 + 2 ptr
    assert ctypes.sizeof(A.Mask) == 40
    assert A.Mask.causal_offsets.offset == 32
    assert ctypes.sizeof(A.Problem) == 8 * 4 + 12 * 8 + 2 * 8
    assert A.Problem.q_stride.offset == 32
    assert A.Problem.cu_seqlens_q.offset == 128
    assert A.Problem.cu_seqlens_k.offset == 136


def prob(**kw):
    base = dict(B=2, H_q=4, H_kv=2, n_q=100, n_k=130, d_h=128, d_v=64, dtype=A.BF16)
    base.update(kw)
    return A.make_problem(**base)


def status(p, **mk):
    lib_or_skip()
    m, keep = A.make_mask(**mk)
    return A.validate(p, m)


def test_validation_codes():
    assert status(prob()) == A.OK
    assert status(prob(), causal=True, offset=0) == A.OK
    assert status(prob(H_q=3, H_kv=2)) == A.INVALID_ARG
    assert status(prob(d_h=96)) == A.UNSUPPORTED
    assert status(prob(d_v=32)) == A.UNSUPPORTED
    assert status(prob(dtype=7)) == A.UNSUPPORTED
    assert status(prob(B=-1)) == A.INVALID_ARG
    # empty visible sets of active rows
    assert status(prob(), causal=True, offset=-1) == A.EMPTY_ROW
    assert status(prob(), seqlens_k=[130, 0]) == A.EMPTY_ROW
    assert status(prob(n_k=0)) == A.EMPTY_ROW
    # ...but sequences without active rows are fine
    assert status(prob(), seqlens_q=[100, 0], seqlens_k=[130, 0]) == A.OK
    assert status(prob(n_q=0, n_k=0)) == A.OK
    # lengths out of range
    assert status(prob(), seqlens_q=[101, 3]) == A.INVALID_ARG
    assert status(prob(), seqlens_k=[-1, 3]) == A.INVALID_ARG
    # strides: multiples of 8, rows hold d elements
    assert status(prob(q_stride=(4 * 100 * 128, 100 * 128, 132))) == A.INVALID_ARG
    assert status(prob(k_stride=(2 * 130 * 64, 130 * 64, 64))) == A.INVALID_ARG
    assert status(prob(q_stride=(4 * 100 * 136, 100 * 136, 136))) == A.OK


def test_calls_reject_before_any_launch():
    """attn_fwd / attn_bwd return the validation or pointer error without
    enqueuing work: here no device exists, so reaching a launch would fail
    differently (ATTN_ERR_HIP) or crash."""
    L = lib_or_skip()
    p = prob()
    m, keep = A.make_mask(causal=True, offset=-3)
    null = ctypes.c_void_p(0)
    st = L.attn_fwd(ctypes.byref(p), ctypes.byref(m), null, null, null, null, null, null)
    assert st == A.EMPTY_ROW
    m2, keep2 = A.make_mask()
    st = L.attn_fwd(ctypes.byref(p), ctypes.byref(m2), null, null, null, null, null, null)
    assert st == A.INVALID_ARG  # null pointers
    bad = ctypes.c_void_p(0x1004)  # misaligned (never dereferenced)
    st = L.attn_fwd(ctypes.byref(p), ctypes.byref(m2), bad, bad, bad, bad, bad, null)
    assert st == A.INVALID_ARG
    fake = ctypes.c_void_p(0x10000)  # aligned but never dereferenced: workspace check comes first
    st = L.attn_bwd(ctypes.byref(p), ctypes.byref(m2), fake, fake, fake, fake, fake, fake, fake, fake,
                    fake, null, ctypes.c_size_t(0), null)
    assert st == A.WORKSPACE
    st = L.attn_bwd(ctypes.byref(p), ctypes.byref(m2), fake, fake, fake, fake, fake, fake, fake, fake,
                    fake, fake, ctypes.c_size_t(16), null)
    assert st == A.WORKSPACE
    assert A.status_string(A.EMPTY_ROW).startswith("an active query row")


def test_gs_backward_errors_before_any_device_work():
    """attn_bwd_gs and attn_bwd_gs_stage check the stage, the problem and the
    workspace (which must also hold G_S) on the host before any launch."""
    L = lib_or_skip()
    fake = ctypes.c_void_p(0x10000)
    null = ctypes.c_void_p(0)
    p = A.make_problem(8, 32, 8, 4096, 4096, 128, 128, A.BF16)  # a grid the passes do not divide
    m, keep = A.make_mask(causal=True)
    args = [fake] * 9
    small = ctypes.c_size_t(A.workspace_size(p))  # enough for attn_bwd, not for G_S
    assert A.gs_workspace_size(p) > small.value
    assert L.attn_bwd_gs(ctypes.byref(p), ctypes.byref(m), *args, fake, small, null) == A.WORKSPACE
    for stage in (0, 1, 2):
        assert L.attn_bwd_gs_stage(ctypes.byref(p), ctypes.byref(m), *args, fake, small,
                                   ctypes.c_int32(stage), null) == A.WORKSPACE
    for stage in (-1, 3):
        assert L.attn_bwd_gs_stage(ctypes.byref(p), ctypes.byref(m), *args, fake,
                                   ctypes.c_size_t(A.gs_workspace_size(p)), ctypes.c_int32(stage),
                                   null) == A.INVALID_ARG
    m2, keep2 = A.make_mask(causal=True, offset=-1)  # an active row with no visible key
    assert L.attn_bwd_gs(ctypes.byref(p), ctypes.byref(m2), *args, fake,
                         ctypes.c_size_t(A.gs_workspace_size(p)), null) == A.EMPTY_ROW


def test_noalloc_backward_errors_before_any_device_work():
    """attn_bwd_noalloc checks the problem and its fixed workspace's size on
    the host before it touches a device (so these run without a GPU)."""
    L = lib_or_skip()
    fake = ctypes.c_void_p(0x10000)
    null = ctypes.c_void_p(0)
    m, keep = A.make_mask(causal=True, offset=-1)
    p = A.make_problem(1, 4, 2, 64, 64, 128, 128, A.BF16)
    args = [fake] * 9 + [null]
    assert L.attn_bwd_noalloc(ctypes.byref(p), ctypes.byref(m), *args) == A.EMPTY_ROW
    m2, keep2 = A.make_mask()
    bad = A.make_problem(1, 3, 2, 64, 64, 128, 128, A.BF16)  # H_q not a multiple of H_kv
    assert L.attn_bwd_noalloc(ctypes.byref(bad), ctypes.byref(m2), *args) == A.INVALID_ARG
    # D alone over the fixed array: B * H_q * n_q floats > 64 MiB
    big = A.make_problem(64, 64, 8, 8192, 64, 128, 128, A.BF16)
    assert A.workspace_size(big) > A.NOALLOC_MAX_WORKSPACE
    assert L.attn_bwd_noalloc(ctypes.byref(big), ctypes.byref(m2), *args) == A.WORKSPACE
    # the limit the header states
    text = open(HEADER).read()
    assert re.search(r"#define ATTN_BWD_NOALLOC_MAX_WORKSPACE \(\(size_t\)64 << 20\)", text)


def _al(x):
    return (x + 255) // 256 * 256


def test_workspace_size():
    lib_or_skip()
    # a grid that fills the GPU: the two per-row arrays (-D and lse log2 e) only
    p = prob(B=8, H_q=32, H_kv=8, n_q=4096, n_k=4096, d_h=128, d_v=128)
    assert A.workspace_size(p) == 2 * _al(8 * 32 * 4096 * 4)
    assert A.workspace_size(prob(B=0)) == 0
    # float32 (no head split) with few keys (no key split): the per-row arrays only
    assert A.workspace_size(prob(B=3, H_q=4, n_q=100, d_h=128, dtype=A.F32)) == 2 * _al(3 * 4 * 100 * 4)


def test_gs_workspace_size():
    """attn_bwd_gs keeps G_S: the per-row arrays plus one 4 KB block per
    (sequence, query head, 32-row block, 128-key block, 64-key half); float32
    problems and grids the two-pass backward would divide need only
    attn_bwd's workspace (attn_bwd_gs runs attn_bwd for them)."""
    lib_or_skip()
    p = prob(B=8, H_q=32, H_kv=8, n_q=4096, n_k=4096, d_h=128, d_v=128)
    assert A.gs_workspace_size(p) == 2 * _al(8 * 32 * 4096 * 4) + _al(8 * 32 * 128 * 32 * 8192)
    p = prob(B=2, H_q=4, H_kv=2, n_q=300, n_k=500, d_h=64, d_v=128)
    if A.workspace_size(p) == 2 * _al(2 * 4 * 300 * 4):  # not divided
        assert A.gs_workspace_size(p) == A.workspace_size(p) + _al(2 * 4 * 10 * 4 * 8192)
    f32 = prob(B=3, H_q=4, n_q=100, d_h=128, dtype=A.F32)
    assert A.gs_workspace_size(f32) == A.workspace_size(f32)
    small = prob(B=1, H_q=8, H_kv=1, n_q=128, n_k=4096, d_h=128, d_v=128)  # divided passes
    assert A.workspace_size(small) > 2 * _al(8 * 128 * 4)
    assert A.gs_workspace_size(small) == A.workspace_size(small)


def test_workspace_size_divided_passes():
    """Small grids divide the backward passes; the workspace then also holds
    their float32 partials: the dQ pass over parts of the keys when fewer than
    384 of its workgroups exist and the keys span at least 8 tiles of 64
    (parts = min(ceil(512 / workgroups), tiles / 4, 16)); the bf16 dK/dV pass
    over parts of each group's query heads when fewer than 192 of its
    workgroups exist (parts = min(ceil(256 / workgroups), group, 8))."""
    lib_or_skip()
    # chunked MQA: B=2, H_q=32, H_kv=1, n_q=256, n_k=8192, d=128
    p = prob(B=2, H_q=32, H_kv=1, n_q=256, n_k=8192, d_h=128, d_v=128)
    rows, krows = 2 * 32 * 256, 2 * 1 * 8192
    dq_wgs, kv_wgs = 2 * 32 * 2, 2 * 1 * 64
    s = min(-(-512 // dq_wgs), 128 // 4, 16)
    hs = min(-(-256 // kv_wgs), 32, 8)
    assert (s, hs) == (4, 2)
    want = 2 * _al(rows * 4) + _al(s * rows * 128 * 4) + _al(hs * krows * 256 * 4)
    assert A.workspace_size(p) == want
    # packed rows: partial rows follow the packed totals
    pk = packed([0, 100, 300], [0, 600, 1200], H_q=4, H_kv=2)
    rows_p, krows_p = 4 * 300, 2 * 1200
    dq_wgs, kv_wgs = 2 * 4 * 2, 2 * 2 * 5
    s = min(-(-512 // dq_wgs), 10 // 4, 16)
    hs = min(-(-256 // kv_wgs), 2, 8)
    assert A.workspace_size(pk) == (2 * _al(2 * 4 * 200 * 4) + _al(s * rows_p * 128 * 4)
                                    + _al(hs * krows_p * (128 + 64) * 4))


def test_validation_per_sequence_offsets():
    # each sequence's own causal offset decides whether its row 0 sees a key
    assert status(prob(), causal=True, offset=[0, 7]) == A.OK
    assert status(prob(), causal=True, offset=[3, -1]) == A.EMPTY_ROW
    # ...which only matters for sequences with active rows
    assert status(prob(), causal=True, offset=[3, -1], seqlens_q=[100, 0]) == A.OK
    # without the causal rule the offsets are unused
    assert status(prob(), causal=False, offset=[-5, -5]) == A.OK


def packed(cu_q, cu_k, **kw):
    base = dict(B=len(cu_q) - 1, H_q=4, H_kv=2, n_q=max(b - a for a, b in zip(cu_q, cu_q[1:])),
                n_k=max(b - a for a, b in zip(cu_k, cu_k[1:])), d_h=128, d_v=64, dtype=A.BF16,
                cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)
    base.update(kw)
    return A.make_problem(**base)


def test_validation_packed_layout():
    assert status(packed([0, 10, 30], [0, 20, 40])) == A.OK
    assert status(packed([0, 10, 30], [0, 20, 40]), causal=True, offset=[0, 3]) == A.OK
    # n_q / n_k must bound every length
    assert status(packed([0, 10, 30], [0, 20, 40], n_q=16)) == A.INVALID_ARG
    assert status(packed([0, 10, 30], [0, 20, 40], n_k=19)) == A.INVALID_ARG
    # offsets start at 0 and never decrease
    assert status(packed([2, 10, 30], [0, 20, 40], n_q=28)) == A.INVALID_ARG
    assert status(packed([0, 10, 5], [0, 20, 40], n_q=10)) == A.INVALID_ARG
    # both arrays or neither; no per-sequence lengths besides them; batch strides 0
    assert status(packed([0, 10, 30], [0, 20, 40], cu_seqlens_k=None)) == A.INVALID_ARG
    assert status(packed([0, 10, 30], [0, 20, 40]), seqlens_q=[10, 20]) == A.INVALID_ARG
    assert status(packed([0, 10, 30], [0, 20, 40], q_stride=(8, 128, 512))) == A.INVALID_ARG
    # empty key range under active rows; empty sequences are fine
    assert status(packed([0, 10, 30], [0, 20, 20])) == A.EMPTY_ROW
    assert status(packed([0, 10, 10, 30], [0, 20, 20, 40])) == A.OK
    # the workspace bound covers the packed rows
    p = packed([0, 10, 30], [0, 20, 40])
    assert A.workspace_size(p) >= 4 * 30 * 4


def test_splitkv_workspace_and_errors():
    L = lib_or_skip()
    p = prob(B=2, H_q=4, n_q=100, n_k=130, d_v=64)
    rows = 2 * 4 * 100
    # float32 partial outputs and logsumexps for every part, two aligned sections
    for s in (1, 3, 8):
        want = (s * rows * 64 * 4 + 255) // 256 * 256 + (s * rows * 4 + 255) // 256 * 256
        assert A.splitkv_workspace_size(p, s) == want
    auto = A.splitkv_workspace_size(p, 0)
    assert auto >= A.splitkv_workspace_size(p, 1)
    # packed layout: rows = H_q * total rows
    pk = packed([0, 10, 30], [0, 20, 40])
    assert A.splitkv_workspace_size(pk, 2) == ((2 * 4 * 30 * 64 * 4 + 255) // 256 * 256
                                               + (2 * 4 * 30 * 4 + 255) // 256 * 256)
    m, keep = A.make_mask()
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x10000)
    # too many parts, then a missing workspace: rejected before any launch
    st = L.attn_fwd_splitkv(ctypes.byref(p), ctypes.byref(m), fake, fake, fake, fake, fake, 2000, fake,
                            ctypes.c_size_t(1 << 30), null)
    assert st == A.INVALID_ARG
    st = L.attn_fwd_splitkv(ctypes.byref(p), ctypes.byref(m), fake, fake, fake, fake, fake, 4, null,
                            ctypes.c_size_t(0), null)
    assert st == A.WORKSPACE
    m2, keep2 = A.make_mask(causal=True, offset=-1)
    st = L.attn_fwd_splitkv(ctypes.byref(p), ctypes.byref(m2), fake, fake, fake, fake, fake, 4, fake,
                            ctypes.c_size_t(1 << 30), null)
    assert st == A.EMPTY_ROW


def test_rope_struct_and_workspace():
    lib_or_skip()
    assert ctypes.sizeof(A.Rope) == 16 and A.Rope.n_pos.offset == 8
    p = prob(B=2, H_q=4, H_kv=2, n_q=100, n_k=130, d_h=128, d_v=64)
    kt = 2 * 2 * 130 * 128 * 2  # rotated keys, bf16, contiguous
    qt = 2 * 4 * 100 * 128 * 2
    al = lambda x: (x + 255) // 256 * 256
    assert A.rope_workspace_size(p, backward=False) == al(kt)
    assert A.rope_workspace_size(p, backward=True) == A.workspace_size(p) + al(qt) + al(kt)
    pk = packed([0, 10, 30], [0, 20, 40])
    assert A.rope_workspace_size(pk, backward=False) == al(40 * 2 * 128 * 2)
    assert A.rope_workspace_size(pk, backward=True) == A.workspace_size(pk) + al(30 * 4 * 128 * 2) + al(40 * 2 * 128 * 2)


def test_rope_argument_errors():
    """Rotary-position calls reject a bad table, positions past it and bad
    operands before anything is enqueued (no device here)."""
    L = lib_or_skip()
    p = prob(B=2, n_q=100, n_k=130)
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x10000)
    big = ctypes.c_size_t(1 << 40)

    def fwd(rope, **mk):
        m, keep = A.make_mask(**mk)
        return L.attn_fwd_rope(ctypes.byref(p), ctypes.byref(m), ctypes.byref(rope), fake, fake, fake, fake, fake,
                               fake, big, null)

    def apply(rope, operand=0, inverse=0, **mk):
        m, keep = A.make_mask(**mk)
        return L.attn_rope_apply(ctypes.byref(p), ctypes.byref(m), ctypes.byref(rope), operand, inverse, fake,
                                 fake, null)

    assert fwd(A.make_rope(0, 200)) == A.INVALID_ARG                  # no table
    assert fwd(A.make_rope(0x10004, 200)) == A.INVALID_ARG            # misaligned table
    assert fwd(A.Rope(fake, 200, 1)) == A.INVALID_ARG                 # reserved != 0
    assert fwd(A.make_rope(0x10000, 129)) == A.INVALID_ARG            # keys past the table
    # query positions i + offset_b must fit: 100 rows at offset 30 need 130
    assert fwd(A.make_rope(0x10000, 130), causal=True, offset=31) == A.INVALID_ARG
    assert fwd(A.make_rope(0x10000, 130), causal=False, offset=[0, -1]) == A.INVALID_ARG
    # ...except for sequences without active rows
    assert apply(A.make_rope(0x10000, 130), 0, 2, offset=[0, 500], seqlens_q=[100, 0]) == A.INVALID_ARG  # bad flag
    assert apply(A.make_rope(0x10000, 130), 2, 0) == A.INVALID_ARG   # bad operand
    # the attention checks still come first
    assert fwd(A.make_rope(0x10000, 10), causal=True, offset=-1) == A.EMPTY_ROW
    # backward: too small a workspace
    m, keep = A.make_mask()
    st = L.attn_bwd_rope(ctypes.byref(p), ctypes.byref(m), ctypes.byref(A.make_rope(0x10000, 200)), fake, fake,
                         fake, fake, fake, fake, fake, fake, fake, fake, ctypes.c_size_t(A.workspace_size(p)), null)
    assert st == A.WORKSPACE


def test_linear_struct_and_errors():
    L = lib_or_skip()
    assert ctypes.sizeof(A.Linear) == 40 and A.Linear.ld_x.offset == 16
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x10000)

    ctx = fake  # a context is only used once a product is enqueued

    def fwd(lin, x=fake, w=fake, y=fake, c=ctx):
        return L.attn_linear_fwd(ctypes.byref(lin), c, x, w, y, null)

    assert fwd(A.make_linear(10, 64, 96, A.BF16, ld_x=32)) == A.INVALID_ARG          # row stride < width
    assert fwd(A.make_linear(10, 64, 96, 7)) == A.UNSUPPORTED
    assert fwd(A.make_linear(-1, 64, 96, A.BF16)) == A.INVALID_ARG
    assert fwd(A.make_linear(10, 64, 96, A.BF16), x=null) == A.INVALID_ARG
    assert fwd(A.make_linear(10, 64, 96, A.BF16), y=ctypes.c_void_p(0x10002)) == A.INVALID_ARG
    assert fwd(A.make_linear(0, 64, 96, A.BF16), x=null, w=null, y=null) == A.OK     # nothing to do
    # the GEMM context is the caller's: a call without one is an argument error
    assert fwd(A.make_linear(10, 64, 96, A.BF16), c=null) == A.INVALID_ARG
    assert fwd(A.make_linear(0, 64, 96, A.BF16), x=null, w=null, y=null, c=null) == A.INVALID_ARG
    lin = A.make_linear(10, 64, 96, A.BF16)
    assert L.attn_linear_bwd(ctypes.byref(lin), ctx, fake, fake, fake, fake, fake, 2, null) == A.INVALID_ARG
    assert L.attn_linear_bwd(ctypes.byref(lin), ctx, fake, fake, null, fake, null, 0, null) == A.INVALID_ARG
    assert L.attn_linear_bwd(ctypes.byref(lin), null, fake, fake, fake, fake, fake, 0, null) == A.INVALID_ARG
    # nothing requested: nothing to check or do
    assert L.attn_linear_bwd(ctypes.byref(lin), ctx, null, null, null, null, null, 0, null) == A.OK
    # destroying no context is a no-op
    assert L.attn_gemm_destroy(null) == A.OK
    assert L.attn_gemm_create(None) == A.INVALID_ARG


def test_self_attention_workspace_and_errors():
    L = lib_or_skip()
    p = A.make_problem(2, 4, 2, 100, 100, 128, 64, A.BF16)
    C = 4 * 128 + 2 * 128 + 2 * 64
    assert A.self_attention_workspace_size(p) == A.workspace_size(p) + (2 * 100 * C * 2 + 255) // 256 * 256
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x10000)
    m, keep = A.make_mask(causal=True)
    ctx = fake
    # self-attention needs n_k == n_q
    p2 = A.make_problem(2, 4, 2, 100, 120, 128, 64, A.BF16)
    assert L.attn_self_attention_fwd(ctypes.byref(p2), ctypes.byref(m), ctx, 256, fake, fake, fake, fake, fake,
                                     null) == A.INVALID_ARG
    assert L.attn_self_attention_fwd(ctypes.byref(p), ctypes.byref(m), ctx, 0, fake, fake, fake, fake, fake,
                                     null) == A.INVALID_ARG
    # no GEMM context
    assert L.attn_self_attention_fwd(ctypes.byref(p), ctypes.byref(m), null, 256, fake, fake, fake, fake, fake,
                                     null) == A.INVALID_ARG
    # packed: the same rows for queries and keys
    pk = A.make_problem(2, 4, 2, 20, 20, 128, 64, A.BF16, cu_seqlens_q=[0, 10, 30], cu_seqlens_k=[0, 20, 30])
    assert L.attn_self_attention_fwd(ctypes.byref(pk), ctypes.byref(m), ctx, 256, fake, fake, fake, fake, fake,
                                     null) == A.INVALID_ARG
    # attention checks still apply
    m2, keep2 = A.make_mask(causal=True, offset=-1)
    assert L.attn_self_attention_fwd(ctypes.byref(p), ctypes.byref(m2), ctx, 256, fake, fake, fake, fake, fake,
                                     null) == A.EMPTY_ROW
    st = L.attn_self_attention_bwd(ctypes.byref(p), ctypes.byref(m), ctx, 256, fake, fake, fake, fake, fake, fake,
                                   fake, fake, fake, ctypes.c_size_t(16), null)
    assert st == A.WORKSPACE
    st = L.attn_self_attention_bwd(ctypes.byref(p), ctypes.byref(m), null, 256, fake, fake, fake, fake, fake, fake,
                                   fake, fake, fake, ctypes.c_size_t(1 << 30), null)
    assert st == A.INVALID_ARG
