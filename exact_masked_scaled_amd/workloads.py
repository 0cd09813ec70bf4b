"""Seeded synthetic workloads and algorithmic work counts.

This module holds no step of the attention method itself: it only draws the
seeded inputs (sequence lengths, Q, K, V and the upstream gradient G_O), rounds
them once to the I/O dtype, and counts visible (query, key) pairs for FLOP
accounting.  Both the GPU path's tests/benchmark and the float64 oracle consume
the same draws from here; neither side's arithmetic lives here.

Input recipe (every workload):
  * generator numpy.random.default_rng(seed), PCG64; default seed 1000 + id;
  * draw order: (i) per-sequence lengths, (ii) Q, (iii) K, (iv) V, (v) G_O,
    each a float64 standard normal array in B,H,n,d C-order;
  * each array is rounded ONCE to the I/O dtype (round-to-nearest-even); the
    oracle consumes exactly those rounded values widened to float64.
Standard normal entries give unit-variance scaled logits q.k/sqrt(d_h) at any
d_h (the variance model of [A.10, eq. A.10.4]), so no extra scale is applied.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    dtype: str
    B: int
    H_q: int
    H_kv: int
    n_q: int
    n_k: int
    d_h: int
    d_v: int
    causal: bool = False
    offset: int = 0
    # inclusive uniform range of per-sequence key lengths (None = unpadded)
    len_k_range: Optional[tuple] = None
    # when True the query rows are padded with the same length as the keys
    pad_rows_like_keys: bool = False

    def describe(self) -> str:
        return (f"{self.name}: {self.dtype} B={self.B} H_q={self.H_q} H_kv={self.H_kv} "
                f"n_q={self.n_q} n_k={self.n_k} d_h={self.d_h} d_v={self.d_v} "
                f"causal={self.causal} offset={self.offset} len_k={self.len_k_range}")


WORKLOADS = {
    1: Workload(1, "mha_fp32_n128_d64", F32, 1, 1, 1, 128, 128, 64, 64),
    2: Workload(2, "causal_mha_bf16_b4_h16_n2048_d128", BF16, 4, 16, 16, 2048, 2048, 128, 128,
                causal=True),
    3: Workload(3, "causal_gqa_padded_bf16_b8_hq32_hkv8_n4096_d128", BF16, 8, 32, 8, 4096, 4096,
                128, 128, causal=True, len_k_range=(2048, 4096), pad_rows_like_keys=True),
    4: Workload(4, "cross_bf16_b4_h16_nq512_nk4096_dh128_dv64", BF16, 4, 16, 16, 512, 4096,
                128, 64, len_k_range=(2048, 4096)),
    5: Workload(5, "chunked_mqa_bf16_b2_hq32_nq256_nk8192_off7936_d128", BF16, 2, 32, 1, 256, 8192,
                128, 128, causal=True, offset=7936),
}

# the throughput headline: bf16 causal GQA at n = 4096, d = 128
HEADLINE = 3


def default_seed(wid: int) -> int:
    return 1000 + wid


# ----------------------------------------------------------------------------
# rounding to the I/O dtype (data preparation, not the method)
# ----------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), returned as float64.

    bf16 keeps 8 significant bits.  With x = m * 2**e, 0.5 <= |m| < 1, rounding
    m * 2**8 to the nearest integer (numpy.rint rounds half to even) keeps 8
    bits in one rounding step.  Valid for the normal bf16 range, which covers
    every drawn value (|x| between 1e-38 and 3e38)."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def bf16_bits(x_rounded: np.ndarray) -> np.ndarray:
    """Bit patterns (uint16) of float64 values that are already bf16-exact."""
    f = np.asarray(x_rounded, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _draw_rounded(rng: np.random.Generator, shape, dtype: str, chunk: int = 1 << 24):
    """Standard normal draw of ``shape`` rounded once to ``dtype``.

    Returns the device payload: uint16 bf16 bits, or float32 values.  Drawing in
    chunks consumes the generator exactly as one big draw would."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == BF16 else np.float32)
    for s in range(0, n, chunk):
        x = rng.standard_normal(min(chunk, n - s))
        if dtype == BF16:
            out[s:s + x.size] = bf16_bits(round_to_bf16(x))
        else:
            out[s:s + x.size] = x.astype(np.float32)
    return out.reshape(shape)


def payload_to_f64(a: np.ndarray) -> np.ndarray:
    """Device payload (uint16 bf16 bits or float32) -> float64 values."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Inputs:
    wl: Workload
    seed: int
    seqlens_q: Optional[list]
    seqlens_k: Optional[list]
    Q: np.ndarray
    K: np.ndarray
    V: np.ndarray
    GO: Optional[np.ndarray]

    def mask_kwargs(self) -> dict:
        return dict(causal=self.wl.causal, offset=self.wl.offset,
                    seqlens_q=self.seqlens_q, seqlens_k=self.seqlens_k)


def draw_lengths(wl: Workload, rng: np.random.Generator):
    if wl.len_k_range is None:
        return None, None
    lo, hi = wl.len_k_range
    lk = [int(x) for x in rng.integers(lo, hi + 1, size=wl.B)]
    lq = list(lk) if wl.pad_rows_like_keys else None
    return lq, lk


def make_inputs(wl, seed: Optional[int] = None, with_grad: bool = True,
                uniform_len: Optional[int] = None) -> Inputs:
    """Seeded inputs of a workload (payload arrays: uint16 bf16 bits or float32).

    ``uniform_len`` replaces the drawn lengths (after drawing them, so the value
    stream is unchanged) -- e.g. the unpadded n = 4096 variant of workload 3."""
    if isinstance(wl, int):
        wl = WORKLOADS[wl]
    if seed is None:
        seed = default_seed(wl.wid)
    rng = np.random.default_rng(seed)
    lq, lk = draw_lengths(wl, rng)
    if uniform_len is not None and lk is not None:
        lk = [uniform_len] * wl.B
        lq = list(lk) if wl.pad_rows_like_keys else None
    Q = _draw_rounded(rng, (wl.B, wl.H_q, wl.n_q, wl.d_h), wl.dtype)
    K = _draw_rounded(rng, (wl.B, wl.H_kv, wl.n_k, wl.d_h), wl.dtype)
    V = _draw_rounded(rng, (wl.B, wl.H_kv, wl.n_k, wl.d_v), wl.dtype)
    GO = _draw_rounded(rng, (wl.B, wl.H_q, wl.n_q, wl.d_v), wl.dtype) if with_grad else None
    return Inputs(wl, seed, lq, lk, Q, K, V, GO)


@dataclasses.dataclass
class ProjectionInputs:
    wl: Workload
    seed: int
    d_model: int
    seqlens: Optional[list]
    X: np.ndarray       # [B, n, d_model] payload
    W: np.ndarray       # [d_model, H_q d_h + H_kv d_h + H_kv d_v] payload, [W_Q | W_K | W_V]
    GO: np.ndarray      # [B, H_q, n, d_v] payload


def make_projection_inputs(wl: Workload, d_model: int, seed: int, seqlens=None) -> ProjectionInputs:
    """Inputs of self-attention with its projections (n_q == n_k): X ~ N(0, 1),
    W ~ N(0, 1/d_model) so the projected Q, K, V have unit-variance entries
    (the variance model of [A.10, eq. A.10.4] again), G_O ~ N(0, 1); each
    rounded once to the I/O dtype.  Draw order: X, W, G_O."""
    if wl.n_q != wl.n_k:
        raise ValueError("self-attention needs n_q == n_k")
    rng = np.random.default_rng(seed)
    C = wl.H_q * wl.d_h + wl.H_kv * wl.d_h + wl.H_kv * wl.d_v
    X = _draw_rounded(rng, (wl.B, wl.n_q, d_model), wl.dtype)
    W = _draw_rounded_scaled(rng, (d_model, C), wl.dtype, 1.0 / np.sqrt(d_model))
    GO = _draw_rounded(rng, (wl.B, wl.H_q, wl.n_q, wl.d_v), wl.dtype)
    return ProjectionInputs(wl, seed, d_model, seqlens, X, W, GO)


def _draw_rounded_scaled(rng: np.random.Generator, shape, dtype: str, scale: float):
    """N(0, scale^2) drawn in float64, rounded once to the I/O dtype."""
    x = rng.standard_normal(shape) * scale
    if dtype == BF16:
        return bf16_bits(round_to_bf16(x))
    return x.astype(np.float32)


def rotary_table(n_pos: int, d_h: int, base: float = 10000.0) -> np.ndarray:
    """The cos/sin table a caller hands to the rotary-position calls, an input
    like Q or K: [n_pos, d_h/2, 2] float32 of (cos, sin) of the angle
    t * base^(-2k/d_h) for position t and column pair k (geometric
    frequencies, one common choice of the fixed per-pair frequency)."""
    k = np.arange(d_h // 2)
    theta = np.arange(n_pos)[:, None] * (base ** (-2.0 * k / d_h))[None, :]
    return np.stack([np.cos(theta), np.sin(theta)], axis=-1).astype(np.float32)


def custom_workload(dtype=BF16, B=1, H_q=1, H_kv=1, n_q=64, n_k=64, d_h=128, d_v=128,
                    causal=False, offset=0, name="custom") -> Workload:
    return Workload(0, name, dtype, B, H_q, H_kv, n_q, n_k, d_h, d_v, causal, offset)


def make_custom_inputs(wl: Workload, seed: int, seqlens_q=None, seqlens_k=None,
                       with_grad=True) -> Inputs:
    rng = np.random.default_rng(seed)
    Q = _draw_rounded(rng, (wl.B, wl.H_q, wl.n_q, wl.d_h), wl.dtype)
    K = _draw_rounded(rng, (wl.B, wl.H_kv, wl.n_k, wl.d_h), wl.dtype)
    V = _draw_rounded(rng, (wl.B, wl.H_kv, wl.n_k, wl.d_v), wl.dtype)
    GO = _draw_rounded(rng, (wl.B, wl.H_q, wl.n_q, wl.d_v), wl.dtype) if with_grad else None
    return Inputs(wl, seed, seqlens_q, seqlens_k, Q, K, V, GO)


# ----------------------------------------------------------------------------
# work accounting
# ----------------------------------------------------------------------------

def visible_pairs_per_sequence(n_q, n_k, causal, offset, seqlens_q, seqlens_k, B):
    """Number of visible (query, key) pairs of each sequence (one query head);
    ``offset`` is one causal offset or one per sequence."""
    lq = [n_q] * B if seqlens_q is None else list(seqlens_q)
    lk = [n_k] * B if seqlens_k is None else list(seqlens_k)
    offs = [int(offset)] * B if np.ndim(offset) == 0 else [int(x) for x in offset]
    out = []
    for b in range(B):
        i = np.arange(lq[b], dtype=np.int64)
        if causal:
            cnt = np.clip(np.minimum(lk[b], i + offs[b] + 1), 0, None)
        else:
            cnt = np.full(lq[b], lk[b], dtype=np.int64)
        out.append(int(cnt.sum()))
    return out


def work(wl: Workload, seqlens_q=None, seqlens_k=None) -> dict:
    """Algorithmic FLOPs and bytes of one forward and one backward.

    Only visible pairs are credited: forward 2*(d_h + d_v) FLOPs per pair
    (QK^T and PV), backward 2*(3*d_h + 2*d_v) (recomputed QK^T, dV, dP, dK, dQ).
    Bytes: forward reads Q, K, V once and writes O and lse; backward reads
    Q, K, V, O, G_O, lse, writes and re-reads D, and writes G_Q, G_K, G_V."""
    pairs_b = visible_pairs_per_sequence(wl.n_q, wl.n_k, wl.causal, wl.offset,
                                         seqlens_q, seqlens_k, wl.B)
    pairs = sum(pairs_b) * wl.H_q
    s = 2 if wl.dtype == BF16 else 4
    q = wl.B * wl.H_q * wl.n_q * wl.d_h * s
    k = wl.B * wl.H_kv * wl.n_k * wl.d_h * s
    v = wl.B * wl.H_kv * wl.n_k * wl.d_v * s
    o = wl.B * wl.H_q * wl.n_q * wl.d_v * s
    rows = wl.B * wl.H_q * wl.n_q * 4
    lq = seqlens_q if seqlens_q is not None else [wl.n_q] * wl.B
    lk = seqlens_k if seqlens_k is not None else [wl.n_k] * wl.B
    return {
        # rows the kernels read or write: active query rows of every query
        # head, key rows below L_k of every KV head
        "active_q_rows": sum(lq) * wl.H_q,
        "active_k_rows": sum(lk) * wl.H_kv,
        "pairs": pairs,
        "pairs_per_sequence": pairs_b,
        "fwd_flop": 2 * pairs * (wl.d_h + wl.d_v),
        "bwd_flop": 2 * pairs * (3 * wl.d_h + 2 * wl.d_v),
        "fwd_bytes": q + k + v + o + rows,
        "bwd_bytes": q + k + v + o + o + rows + 2 * rows + q + k + v,
        # the literal count 4*n_q*n_k*d per head, halved for causal (d = d_h)
        "literal_fwd_flop": wl.B * wl.H_q * 4 * wl.n_q * wl.n_k * wl.d_h // (2 if wl.causal else 1),
    }
