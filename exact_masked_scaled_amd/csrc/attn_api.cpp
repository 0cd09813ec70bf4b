// Host side of the C ABI declared in include/attn.h: argument checks, kernel
// argument packing, batch chunking and launch order.  Pure C++; the HIP
// launches live in the kernel translation units.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "attn_internal.h"

using namespace attn;

namespace {

constexpr size_t kWsAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t esize(int dtype) { return dtype == ATTN_BF16 ? 2 : 4; }

// Fill everything but pointers and lengths.
void fill_common(KernelParams& kp, const attn_problem& p, const attn_mask& m) {
  memset(&kp, 0, sizeof(kp));
  kp.q_sb = p.q_stride[0]; kp.q_sh = p.q_stride[1]; kp.q_sr = p.q_stride[2];
  kp.k_sb = p.k_stride[0]; kp.k_sh = p.k_stride[1]; kp.k_sr = p.k_stride[2];
  kp.v_sb = p.v_stride[0]; kp.v_sh = p.v_stride[1]; kp.v_sr = p.v_stride[2];
  kp.o_sb = p.o_stride[0]; kp.o_sh = p.o_stride[1]; kp.o_sr = p.o_stride[2];
  kp.dq_sb = kp.q_sb; kp.dq_sh = kp.q_sh; kp.dq_sr = kp.q_sr;
  kp.dk_sb = kp.k_sb; kp.dk_sh = kp.k_sh; kp.dk_sr = kp.k_sr;
  kp.H_q = p.H_q; kp.H_kv = p.H_kv; kp.n_q = p.n_q; kp.n_k = p.n_k;
  kp.group = p.H_q / p.H_kv;
  kp.causal = m.causal;
  // j <= i + off with off >= n_k is no restriction at all; offsets below zero
  // only reach here when no row is active.
  kp.offset = (int32_t)std::min<int64_t>(std::max<int64_t>(m.causal_offset, 0), p.n_k);
  kp.scale = (float)(1.0 / sqrt((double)p.d_h));
  kp.scale_log2 = (float)(1.4426950408889634 / sqrt((double)p.d_h));
  kp.varlen = p.cu_seqlens_q != nullptr ? 1 : 0;
  kp.has_lens = (m.seqlens_q != nullptr || m.seqlens_k != nullptr || kp.varlen) ? 1 : 0;
  kp.has_offs = (m.causal && m.causal_offsets != nullptr) ? 1 : 0;
  if (kp.varlen) {  // lse / D: [H_q][total rows]; the row offsets carry the sequence
    kp.lse_sb = 0;
    kp.lse_sh = p.cu_seqlens_q[p.B];
    kp.krow_sb = 0;
    kp.krow_sh = p.cu_seqlens_k[p.B];
  } else {
    kp.lse_sb = (int64_t)p.H_q * p.n_q;
    kp.lse_sh = p.n_q;
    kp.krow_sb = (int64_t)p.H_kv * p.n_k;
    kp.krow_sh = p.n_k;
  }
  kp.hsplits = 1;
}

int32_t clamp_offset(int64_t off, int32_t n_k) {
  return (int32_t)std::min<int64_t>(std::max<int64_t>(off, 0), n_k);
}

// Active rows / valid keys of sequence b and its offset_b.
int64_t seq_len_q(const attn_problem& p, const attn_mask& m, int b) {
  if (p.cu_seqlens_q) return (int64_t)p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b];
  return m.seqlens_q ? m.seqlens_q[b] : p.n_q;
}
int64_t seq_len_k(const attn_problem& p, const attn_mask& m, int b) {
  if (p.cu_seqlens_k) return (int64_t)p.cu_seqlens_k[b + 1] - p.cu_seqlens_k[b];
  return m.seqlens_k ? m.seqlens_k[b] : p.n_k;
}
int64_t seq_offset(const attn_mask& m, int b) { return m.causal_offsets ? m.causal_offsets[b] : m.causal_offset; }

// Sequence chunk [b0, b0 + nb): per-sequence data and unit counts.
void fill_chunk(KernelParams& kp, const attn_problem& p, const attn_mask& m, int b0, int nb) {
  kp.B = nb;
  for (int i = 0; i < nb; ++i) {
    const int b = b0 + i;
    if (kp.varlen) {
      kp.row0_q[i] = p.cu_seqlens_q[b];
      kp.row0_k[i] = p.cu_seqlens_k[b];
      kp.lens_q[i] = p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b];
      kp.lens_k[i] = p.cu_seqlens_k[b + 1] - p.cu_seqlens_k[b];
    } else if (kp.has_lens) {
      kp.lens_q[i] = m.seqlens_q ? m.seqlens_q[b] : p.n_q;
      kp.lens_k[i] = m.seqlens_k ? m.seqlens_k[b] : p.n_k;
    }
    if (kp.has_offs) kp.offs[i] = clamp_offset(m.causal_offsets[b], p.n_k);
    // rotary positions of the query rows start at offset_b (checked to fit
    // the table for sequences with active rows)
    if (kp.rope) kp.rope_pos[i] = seq_len_q(p, m, b) > 0 ? (int32_t)seq_offset(m, b) : 0;
  }
  kp.groups = nb * p.H_kv;
  kp.xcd_map = (kp.groups % 8 == 0) ? 1 : 0;
}

template <typename T>
const T* off(const T* base, int64_t elems, size_t es) {
  return base ? (const T*)((const char*)base + elems * (int64_t)es) : nullptr;
}
template <typename T>
T* off(T* base, int64_t elems, size_t es) {
  return base ? (T*)((char*)base + elems * (int64_t)es) : nullptr;
}

// Forward work items per (sequence, KV head) unit.  With packed heads a
// workgroup's rows are the unit's (position, head) pairs, group * n_q rows in
// blocks; otherwise each query head has its own blocks of n_q rows.
bool fwd_pack(const attn_problem& p) {
  const int64_t group = p.H_q / p.H_kv;
  return group > 1 && group * p.n_q <= INT32_MAX;
}
int64_t fwd_items(const attn_problem& p, bool pack) {
  const int64_t bm = fwd_block_rows(p.dtype), group = p.H_q / p.H_kv;
  return pack ? (group * p.n_q + bm - 1) / bm : group * ((p.n_q + bm - 1) / bm);
}

int chunk_size(const KernelParams& kp, int B) {
  return (kp.has_lens || kp.has_offs || kp.rope) ? kMaxBatchChunk : std::max(B, 1);
}

// How the backward passes are divided when their grids alone would leave
// most of the GPU idle (few sequences and heads, short query blocks): the
// dQ pass over parts of the keys (float32 partial G_Q summed by a combine
// kernel), the bf16 dK/dV pass over parts of each group's query heads
// (partial G_K / G_V likewise).  Fixed by the sizes alone, so the workspace
// size and the call agree; not used with rotary positions.
struct BwdPlan {
  int32_t dq_splits = 1, hsplits = 1;
  // G_S kept (attn_bwd_gs): one 4 KB block per (sequence, query head,
  // 32-row block, 128-key block, 64-key half)
  bool gs = false;
  int32_t gs_nqb = 0, gs_nkb = 0;
  size_t gs_bytes = 0;
  int64_t q_rows = 0, k_rows = 0;      // rows of lse / D, and of the key partials
  size_t row_bytes = 0;                 // one float per row of lse: the -D array, then the lse2 array
  size_t d_bytes = 0, dq_bytes = 0, kv_bytes = 0;
};
BwdPlan bwd_plan(const attn_problem& p, bool rope, bool keep_gs = false) {
  BwdPlan pl;
  const bool packed = p.cu_seqlens_q != nullptr;
  pl.q_rows = packed ? (int64_t)p.H_q * std::max(p.cu_seqlens_q[p.B], 0) : (int64_t)p.B * p.H_q * p.n_q;
  pl.k_rows = packed ? (int64_t)p.H_kv * std::max(p.cu_seqlens_k[p.B], 0) : (int64_t)p.B * p.H_kv * p.n_k;
  pl.row_bytes = align_up((size_t)p.B * (size_t)p.H_q * (size_t)p.n_q * sizeof(float), kWsAlign);
  pl.d_bytes = 2 * pl.row_bytes;
  if (p.B <= 0 || p.H_kv <= 0 || rope) return pl;
  const int64_t nb = std::min(p.B, kMaxBatchChunk);
  const int64_t group = p.H_q / p.H_kv;
  const int64_t dq_wgs = nb * p.H_q * ((p.n_q + bwd_dq_block_rows(p.dtype) - 1) / bwd_dq_block_rows(p.dtype));
  const int64_t key_tiles = (p.n_k + 63) / 64;
  if (dq_wgs > 0 && dq_wgs < 384 && key_tiles >= 8)  // two workgroups per CU want 512
    pl.dq_splits = (int32_t)std::min<int64_t>({(512 + dq_wgs - 1) / dq_wgs, key_tiles / 4, 16});
  const int64_t kv_wgs = nb * p.H_kv * ((p.n_k + bwd_dkdv_block_keys(p.dtype) - 1) / bwd_dkdv_block_keys(p.dtype));
  if (p.dtype == ATTN_BF16 && kv_wgs > 0 && kv_wgs < 192 && group > 1)  // one per CU wants 256
    pl.hsplits = (int32_t)std::min<int64_t>({(256 + kv_wgs - 1) / kv_wgs, group, 8});
  if (pl.dq_splits > 1) pl.dq_bytes = align_up((size_t)pl.dq_splits * pl.q_rows * p.d_h * sizeof(float), kWsAlign);
  if (pl.hsplits > 1)
    pl.kv_bytes = align_up((size_t)pl.hsplits * pl.k_rows * (p.d_h + p.d_v) * sizeof(float), kWsAlign);
  // G_S kept: bf16 grids that need no division (the divided passes stay two-pass)
  // (the product pass addresses a sequence's K rows with 32-bit offsets)
  const bool k_fits = p.k_stride[2] >= 0 &&
                      (p.n_k - 1) * (int64_t)p.k_stride[2] * 2 + (int64_t)p.d_h * 2 <= (int64_t)0xffffffff;
  if (keep_gs && p.dtype == ATTN_BF16 && pl.dq_splits == 1 && pl.hsplits == 1 && p.n_q > 0 && p.n_k > 0 &&
      (p.d_h == 64 || p.d_h == 128) && (p.d_v == 64 || p.d_v == 128) && k_fits) {
    pl.gs = true;
    pl.gs_nqb = (int32_t)((p.n_q + 31) / 32);
    pl.gs_nkb = (int32_t)((p.n_k + 127) / 128);
    pl.gs_bytes = align_up((size_t)p.B * p.H_q * pl.gs_nqb * pl.gs_nkb * 8192, kWsAlign);
  }
  return pl;
}

}  // namespace

extern "C" {

attn_status attn_validate(const attn_problem* prob, const attn_mask* mask) {
  return validate_problem(prob, mask);
}

size_t attn_bwd_workspace_size(const attn_problem* prob) {
  if (prob == nullptr || prob->B < 0 || prob->H_q < 0 || prob->H_kv < 0 || prob->n_q < 0 || prob->n_k < 0 ||
      prob->d_h < 0 || prob->d_v < 0)
    return 0;
  if ((prob->cu_seqlens_q == nullptr) != (prob->cu_seqlens_k == nullptr)) return 0;
  const BwdPlan pl = bwd_plan(*prob, false);
  return pl.d_bytes + pl.dq_bytes + pl.kv_bytes;
}

size_t attn_bwd_gs_workspace_size(const attn_problem* prob) {
  if (prob == nullptr || prob->B < 0 || prob->H_q < 0 || prob->H_kv < 0 || prob->n_q < 0 || prob->n_k < 0 ||
      prob->d_h < 0 || prob->d_v < 0)
    return 0;
  if ((prob->cu_seqlens_q == nullptr) != (prob->cu_seqlens_k == nullptr)) return 0;
  const BwdPlan pl = bwd_plan(*prob, false, true);
  return pl.d_bytes + pl.dq_bytes + pl.kv_bytes + pl.gs_bytes;
}

attn_status attn_fwd(const attn_problem* prob, const attn_mask* mask, const void* Q, const void* K,
                     const void* V, void* O, float* lse, void* stream) {
  attn_status st = validate_problem(prob, mask);
  if (st != ATTN_OK) return st;
  const attn_problem& p = *prob;
  const attn_mask& m = *mask;
  if (p.B == 0 || p.n_q == 0) return ATTN_OK;
  if (!Q || !O || !lse || !aligned16(Q) || !aligned16(O) || !aligned16(lse)) return ATTN_ERR_INVALID_ARG;
  if (p.n_k > 0 && (!K || !V || !aligned16(K) || !aligned16(V))) return ATTN_ERR_INVALID_ARG;
  const size_t es = esize(p.dtype);
  KernelParams kp;
  fill_common(kp, p, m);
  kp.pack = fwd_pack(p) ? 1 : 0;
  const int cs = chunk_size(kp, p.B);
  for (int b0 = 0; b0 < p.B; b0 += cs) {
    const int nb = std::min(cs, p.B - b0);
    fill_chunk(kp, p, m, b0, nb);
    kp.per_group = (int32_t)fwd_items(p, kp.pack != 0);
    kp.q = off(Q, b0 * p.q_stride[0], es);
    kp.k = off(K, b0 * p.k_stride[0], es);
    kp.v = off(V, b0 * p.v_stride[0], es);
    kp.o_out = off(O, b0 * p.o_stride[0], es);
    kp.lse = lse + b0 * kp.lse_sb;
    if (launch_fwd(kp, p.dtype, p.d_h, p.d_v, stream) != 0) return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

// ---------------------------------------------------------------- split forward

namespace {

// rows of the lse array (padded: B * H_q * n_q; packed: H_q * total rows)
int64_t lse_rows(const attn_problem& p) {
  if (p.cu_seqlens_q != nullptr) return (int64_t)p.H_q * p.cu_seqlens_q[p.B];
  return (int64_t)p.B * p.H_q * p.n_q;
}

// Parts per row block: enough workgroups to give every CU two (the forward
// runs two per CU), at most one part per key tile and at most 64.
int32_t auto_splits(const attn_problem& p) {
  const int64_t base =
      std::max<int64_t>(1, (int64_t)std::min(p.B, kMaxBatchChunk) * p.H_kv * fwd_items(p, fwd_pack(p)));
  const int64_t want = (512 + base - 1) / base;
  const int64_t tiles = std::max<int64_t>(1, (p.n_k + 63) / 64);
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>({want, tiles, 64}));
}

int32_t resolve_splits(const attn_problem& p, int32_t num_splits) {
  return num_splits > 0 ? num_splits : auto_splits(p);
}

}  // namespace

size_t attn_fwd_splitkv_workspace_size(const attn_problem* prob, int32_t num_splits) {
  if (prob == nullptr || prob->B < 0 || prob->H_q < 0 || prob->n_q < 0 || prob->n_k < 0 || prob->d_v < 0 ||
      num_splits > 1024)
    return 0;
  if (prob->cu_seqlens_q != nullptr && prob->B > 0 && prob->cu_seqlens_q[prob->B] < 0) return 0;
  const size_t rows = (size_t)lse_rows(*prob);
  const size_t s = (size_t)resolve_splits(*prob, num_splits);
  return align_up(s * rows * (size_t)prob->d_v * sizeof(float), kWsAlign) +
         align_up(s * rows * sizeof(float), kWsAlign);
}

attn_status attn_fwd_splitkv(const attn_problem* prob, const attn_mask* mask, const void* Q, const void* K,
                             const void* V, void* O, float* lse, int32_t num_splits, void* workspace,
                             size_t workspace_bytes, void* stream) {
  attn_status st = validate_problem(prob, mask);
  if (st != ATTN_OK) return st;
  if (num_splits > 1024) return ATTN_ERR_INVALID_ARG;
  const attn_problem& p = *prob;
  const attn_mask& m = *mask;
  if (p.B == 0 || p.n_q == 0) return ATTN_OK;
  if (!Q || !O || !lse || !aligned16(Q) || !aligned16(O) || !aligned16(lse)) return ATTN_ERR_INVALID_ARG;
  if (p.n_k > 0 && (!K || !V || !aligned16(K) || !aligned16(V))) return ATTN_ERR_INVALID_ARG;
  const int32_t splits = resolve_splits(p, num_splits);
  const size_t need = attn_fwd_splitkv_workspace_size(prob, num_splits);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace % kWsAlign) != 0))
    return ATTN_ERR_WORKSPACE;
  const size_t es = esize(p.dtype);
  const int64_t rows = lse_rows(p);
  float* part_o = (float*)workspace;
  float* part_lse = (float*)((char*)workspace + align_up((size_t)splits * rows * p.d_v * sizeof(float), kWsAlign));
  KernelParams kp;
  fill_common(kp, p, m);
  kp.splits = splits;
  kp.part_rows = rows;
  kp.pack = fwd_pack(p) ? 1 : 0;
  const int cs = chunk_size(kp, p.B);
  for (int b0 = 0; b0 < p.B; b0 += cs) {
    const int nb = std::min(cs, p.B - b0);
    fill_chunk(kp, p, m, b0, nb);
    kp.per_group = (int32_t)(fwd_items(p, kp.pack != 0) * splits);
    kp.q = off(Q, b0 * p.q_stride[0], es);
    kp.k = off(K, b0 * p.k_stride[0], es);
    kp.v = off(V, b0 * p.v_stride[0], es);
    kp.o_out = off(O, b0 * p.o_stride[0], es);
    kp.lse = lse + b0 * kp.lse_sb;
    kp.part_o = part_o + b0 * kp.lse_sb * p.d_v;
    kp.part_lse = part_lse + b0 * kp.lse_sb;
    if (launch_fwd_split(kp, p.dtype, p.d_h, p.d_v, stream) != 0) return ATTN_ERR_HIP;
    if (launch_fwd_combine(kp, p.dtype, p.d_v, stream) != 0) return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // extern "C"

namespace {

enum : int { kDq = 1, kDkdv = 2 };

struct BwdPtrs {
  const void *Q, *K, *V, *O, *dO;
  const float* lse;
  void *dQ, *dK, *dV;
};

// Rotated copies of Q and K the backward passes read instead of the caller's
// (rotary positions): their element strides, and the rope flags.
struct RopeCtx {
  const float* cos_sin;
  const void* Qt;
  const void* Kt;
  int64_t qt_s[3], kt_s[3];
};

// Checks of attn_bwd and its two passes: validate, then the pointers the
// requested passes read or write and the workspace.
attn_status bwd_check(const attn_problem* prob, const attn_mask* mask, const BwdPtrs& t, void* workspace,
                      size_t workspace_bytes, int passes, bool keep_gs = false) {
  attn_status st = validate_problem(prob, mask);
  if (st != ATTN_OK) return st;
  const attn_problem& p = *prob;
  if (p.B == 0 || (p.n_q == 0 && p.n_k == 0)) return ATTN_OK;
  const bool has_q = p.n_q > 0, has_k = p.n_k > 0;
  auto ok = [](const void* ptr) { return ptr != nullptr && aligned16(ptr); };
  if (has_q) {
    if ((passes & kDq) && !(ok(t.Q) && ok(t.O) && ok(t.lse) && ok(t.dO) && ok(t.dQ)))
      return ATTN_ERR_INVALID_ARG;
    if ((passes & kDkdv) && !(ok(t.Q) && ok(t.lse) && ok(t.dO))) return ATTN_ERR_INVALID_ARG;
  }
  if (has_k && (passes & kDkdv) && !(ok(t.K) && ok(t.V) && ok(t.dK) && ok(t.dV)))
    return ATTN_ERR_INVALID_ARG;
  if (has_k && has_q && (passes & kDq) && !(ok(t.K) && ok(t.V))) return ATTN_ERR_INVALID_ARG;
  const size_t need_ws = keep_gs ? attn_bwd_gs_workspace_size(prob) : attn_bwd_workspace_size(prob);
  if (need_ws > 0 &&
      (workspace == nullptr || workspace_bytes < need_ws || ((uintptr_t)workspace % kWsAlign) != 0))
    return ATTN_ERR_WORKSPACE;
  return ATTN_OK;
}

// Enqueue the requested passes per sequence chunk (arguments checked).
attn_status bwd_enqueue(const attn_problem& p, const attn_mask& m, const BwdPtrs& t, float* delta, void* stream,
                        int passes, const RopeCtx* rc, bool keep_gs = false, int stage = -1) {
  if (p.B == 0 || (p.n_q == 0 && p.n_k == 0)) return ATTN_OK;
  const bool has_q = p.n_q > 0, has_k = p.n_k > 0;
  const size_t es = esize(p.dtype);
  KernelParams kp;
  fill_common(kp, p, m);
  const void* Qsrc = t.Q;
  const void* Ksrc = t.K;
  int64_t q_sb = p.q_stride[0], k_sb = p.k_stride[0];
  if (rc) {  // read the rotated copies; G_Q and G_K keep the caller's strides
    kp.rope = kRopeDQ | kRopeDK;
    kp.rope_cs = rc->cos_sin;
    Qsrc = rc->Qt;
    Ksrc = rc->Kt;
    q_sb = rc->qt_s[0]; kp.q_sb = rc->qt_s[0]; kp.q_sh = rc->qt_s[1]; kp.q_sr = rc->qt_s[2];
    k_sb = rc->kt_s[0]; kp.k_sb = rc->kt_s[0]; kp.k_sh = rc->kt_s[1]; kp.k_sr = rc->kt_s[2];
  }
  const int nqblk = (p.n_q + bwd_dq_block_rows(p.dtype) - 1) / bwd_dq_block_rows(p.dtype);
  const int nkblk = (p.n_k + bwd_dkdv_block_keys(p.dtype) - 1) / bwd_dkdv_block_keys(p.dtype);
  // workspace: -D, lse2, then the partials of divided passes
  const BwdPlan pl = bwd_plan(p, rc != nullptr, keep_gs && passes == (kDq | kDkdv));
  float* part_q = delta ? (float*)((char*)delta + pl.d_bytes) : nullptr;
  float* part_kv = delta ? (float*)((char*)delta + pl.d_bytes + pl.dq_bytes) : nullptr;
  void* gs_buf = delta && pl.gs ? (void*)((char*)delta + pl.d_bytes + pl.dq_bytes + pl.kv_bytes) : nullptr;
  kp.splits = pl.dq_splits;
  kp.part_rows = pl.q_rows;
  kp.hsplits = pl.hsplits;
  kp.part_krows = pl.k_rows;
  const int cs = chunk_size(kp, p.B);
  for (int b0 = 0; b0 < p.B; b0 += cs) {
    const int nb = std::min(cs, p.B - b0);
    fill_chunk(kp, p, m, b0, nb);
    const int64_t row0 = b0 * kp.lse_sb;
    kp.q = off(Qsrc, b0 * q_sb, es);
    kp.k = off(Ksrc, b0 * k_sb, es);
    kp.v = off(t.V, b0 * p.v_stride[0], es);
    kp.o = off(t.O, b0 * p.o_stride[0], es);
    kp.dout = off(t.dO, b0 * p.o_stride[0], es);
    kp.lse = t.lse ? const_cast<float*>(t.lse) + row0 : nullptr;
    kp.delta = delta ? delta + row0 : nullptr;
    kp.lse2 = delta ? (float*)((char*)delta + pl.row_bytes) + row0 : nullptr;
    kp.dq = off(t.dQ, b0 * p.q_stride[0], es);
    kp.dk = off(t.dK, b0 * p.k_stride[0], es);
    kp.dv = off(t.dV, b0 * p.v_stride[0], es);
    if (pl.dq_splits > 1) kp.part_o = part_q + b0 * kp.lse_sb * p.d_h;
    if (pl.hsplits > 1) {
      kp.part_dk = part_kv + b0 * kp.krow_sb * p.d_h;
      kp.part_dv = part_kv + (int64_t)pl.hsplits * pl.k_rows * p.d_h + b0 * kp.krow_sb * p.d_v;
    }
    if (pl.gs) {
      // -D and lse log2 e first (stage 0), then the dK/dV pass writing G_S
      // (stage 1), then G_Q from it (stage 2); the chunk's G_S blocks start
      // at its first sequence's
      const int rqblk = (p.n_q + bwd_gs_block_rows() - 1) / bwd_gs_block_rows();
      kp.gs = (char*)gs_buf + (size_t)b0 * p.H_q * pl.gs_nqb * pl.gs_nkb * 8192;
      kp.gs_nqb = pl.gs_nqb;
      kp.gs_nkb = pl.gs_nkb;
      if (stage < 0 || stage == 0) {
        KernelParams kr = kp;
        kr.gs = nullptr;
        kr.per_group = kr.group * rqblk;
        if (launch_bwd_rows(kr, p.d_v, stream) != 0) return ATTN_ERR_HIP;
      }
      if (stage < 0 || stage == 1) {
        kp.per_group = nkblk;
        if (launch_bwd_dkdv(kp, p.dtype, p.d_h, p.d_v, stream) != 0) return ATTN_ERR_HIP;
      }
      if (stage < 0 || stage == 2) {
        kp.per_group = (int32_t)bwd_dq_gs_items(p.n_q, kp.group);
        if (launch_bwd_dq_gs(kp, p.d_h, stream) != 0) return ATTN_ERR_HIP;
      }
      kp.gs = nullptr;
      continue;
    }
    if ((passes & kDq) && has_q) {
      kp.per_group = kp.group * nqblk * pl.dq_splits;
      if (rc) {  // the dQ pass reads the caller's Q, turns it as it loads it and writes q~
        KernelParams kq = kp;
        kq.q = off(t.Q, b0 * p.q_stride[0], es);
        kq.q_sb = p.q_stride[0]; kq.q_sh = p.q_stride[1]; kq.q_sr = p.q_stride[2];
        kq.qt = off((void*)rc->Qt, b0 * rc->qt_s[0], es);
        kq.qt_sb = rc->qt_s[0]; kq.qt_sh = rc->qt_s[1]; kq.qt_sr = rc->qt_s[2];
        if (launch_bwd_dq(kq, p.dtype, p.d_h, p.d_v, stream) != 0) return ATTN_ERR_HIP;
      } else if (launch_bwd_dq(kp, p.dtype, p.d_h, p.d_v, stream) != 0) {
        return ATTN_ERR_HIP;
      }
    }
    if ((passes & kDkdv) && has_k) {
      kp.per_group = nkblk * pl.hsplits;
      if (launch_bwd_dkdv(kp, p.dtype, p.d_h, p.d_v, stream) != 0) return ATTN_ERR_HIP;
      if (pl.hsplits > 1 && launch_dkdv_combine(kp, p.dtype, p.d_h, p.d_v, stream) != 0) return ATTN_ERR_HIP;
    }
  }
  return ATTN_OK;
}

attn_status bwd_passes(const attn_problem* prob, const attn_mask* mask, const BwdPtrs& t, void* workspace,
                       size_t workspace_bytes, void* stream, int passes, bool keep_gs = false, int stage = -1) {
  const attn_status st = bwd_check(prob, mask, t, workspace, workspace_bytes, passes, keep_gs);
  if (st != ATTN_OK) return st;
  return bwd_enqueue(*prob, *mask, t, (float*)workspace, stream, passes, nullptr, keep_gs, stage);
}

}  // namespace

extern "C" {

attn_status attn_bwd(const attn_problem* prob, const attn_mask* mask, const void* Q, const void* K,
                     const void* V, const void* O, const float* lse, const void* dO, void* dQ, void* dK,
                     void* dV, void* workspace, size_t workspace_bytes, void* stream) {
  const BwdPtrs t{Q, K, V, O, dO, lse, dQ, dK, dV};
  return bwd_passes(prob, mask, t, workspace, workspace_bytes, stream, kDq | kDkdv);
}

attn_status attn_bwd_gs(const attn_problem* prob, const attn_mask* mask, const void* Q, const void* K,
                        const void* V, const void* O, const float* lse, const void* dO, void* dQ, void* dK,
                        void* dV, void* workspace, size_t workspace_bytes, void* stream) {
  const BwdPtrs t{Q, K, V, O, dO, lse, dQ, dK, dV};
  return bwd_passes(prob, mask, t, workspace, workspace_bytes, stream, kDq | kDkdv, true);
}

attn_status attn_bwd_gs_stage(const attn_problem* prob, const attn_mask* mask, const void* Q, const void* K,
                              const void* V, const void* O, const float* lse, const void* dO, void* dQ, void* dK,
                              void* dV, void* workspace, size_t workspace_bytes, int32_t stage, void* stream) {
  if (stage < 0 || stage > 2) return ATTN_ERR_INVALID_ARG;
  const BwdPtrs t{Q, K, V, O, dO, lse, dQ, dK, dV};
  if (attn_bwd_gs_workspace_size(prob) > attn_bwd_workspace_size(prob)) {
    return bwd_passes(prob, mask, t, workspace, workspace_bytes, stream, kDq | kDkdv, true, stage);
  }
  // the two-pass backward: its dQ pass (with D) as stage 0, its dK/dV pass as stage 1
  if (stage == 2) {
    const attn_status st = validate_problem(prob, mask);
    return st;
  }
  return bwd_passes(prob, mask, t, workspace, workspace_bytes, stream, stage == 0 ? kDq : kDkdv);
}

attn_status attn_bwd_dq(const attn_problem* prob, const attn_mask* mask, const void* Q, const void* K,
                        const void* V, const void* O, const float* lse, const void* dO, void* dQ,
                        void* workspace, size_t workspace_bytes, void* stream) {
  const BwdPtrs t{Q, K, V, O, dO, lse, dQ, nullptr, nullptr};
  return bwd_passes(prob, mask, t, workspace, workspace_bytes, stream, kDq);
}

attn_status attn_bwd_dkdv(const attn_problem* prob, const attn_mask* mask, const void* Q, const void* K,
                          const void* V, const float* lse, const void* dO, void* dK, void* dV,
                          void* workspace, size_t workspace_bytes, void* stream) {
  const BwdPtrs t{Q, K, V, nullptr, dO, lse, nullptr, dK, dV};
  return bwd_passes(prob, mask, t, workspace, workspace_bytes, stream, kDkdv);
}

}  // extern "C"

// ---------------------------------------------------------------- rotary positions

namespace {

attn_status validate_rope(const attn_problem& p, const attn_mask& m, const attn_rope* r) {
  if (r == nullptr || r->cos_sin == nullptr || !aligned16(r->cos_sin) || r->n_pos < 1 || r->reserved != 0)
    return ATTN_ERR_INVALID_ARG;
  for (int b = 0; b < p.B; ++b) {
    if (seq_len_k(p, m, b) > r->n_pos) return ATTN_ERR_INVALID_ARG;
    const int64_t lq = seq_len_q(p, m, b);
    if (lq == 0) continue;
    const int64_t off = seq_offset(m, b);
    if (off < 0 || off > (int64_t)r->n_pos - lq) return ATTN_ERR_INVALID_ARG;
  }
  return ATTN_OK;
}

// A rotated copy in the workspace: rows of H heads x d columns, contiguous
// ([B][H][n][d], or [total rows][H][d] in the packed layout).
struct Rotated {
  int64_t s[3];
  size_t bytes;
};
Rotated rotated_layout(const attn_problem& p, bool keys) {
  const int64_t H = keys ? p.H_kv : p.H_q, n = keys ? p.n_k : p.n_q, d = p.d_h;
  const int32_t* cu = keys ? p.cu_seqlens_k : p.cu_seqlens_q;
  Rotated r;
  if (cu != nullptr) {
    r.s[0] = 0; r.s[1] = d; r.s[2] = H * d;
    r.bytes = (size_t)(p.B > 0 ? std::max(cu[p.B], 0) : 0) * H * d * esize(p.dtype);
  } else {
    r.s[0] = H * n * d; r.s[1] = n * d; r.s[2] = d;
    r.bytes = (size_t)p.B * H * n * d * esize(p.dtype);
  }
  r.bytes = align_up(r.bytes, kWsAlign);
  return r;
}

bool sizes_ok(const attn_problem* prob) {
  return prob != nullptr && prob->B >= 0 && prob->H_q >= 0 && prob->H_kv >= 0 && prob->n_q >= 0 &&
         prob->n_k >= 0 && prob->d_h >= 0;
}

// Rotate the active rows of every sequence (operand 0: Q rows at positions
// i + offset_b; 1: K rows at positions j), per chunk of sequences.
attn_status rope_enqueue(const attn_problem& p, const attn_mask& m, const float* cs, int operand, int inverse,
                         const void* X, const int64_t xs[3], void* Y, const int64_t ys[3], void* stream) {
  const bool keys = operand == 1;
  const int32_t* cu = keys ? p.cu_seqlens_k : p.cu_seqlens_q;
  const size_t es = esize(p.dtype);
  RopeParams rp;
  memset(&rp, 0, sizeof(rp));
  rp.cs = cs;
  rp.inverse = inverse;
  rp.x_sb = xs[0]; rp.x_sh = xs[1]; rp.x_sr = xs[2];
  rp.y_sb = ys[0]; rp.y_sh = ys[1]; rp.y_sr = ys[2];
  rp.H = keys ? p.H_kv : p.H_q;
  for (int b0 = 0; b0 < p.B; b0 += kMaxBatchChunk) {
    const int nb = std::min(kMaxBatchChunk, p.B - b0);
    rp.B = nb;
    int32_t nmax = 0;
    for (int i = 0; i < nb; ++i) {
      const int b = b0 + i;
      rp.len[i] = (int32_t)(keys ? seq_len_k(p, m, b) : seq_len_q(p, m, b));
      rp.row0[i] = cu ? cu[b] : 0;
      rp.pos0[i] = (!keys && rp.len[i] > 0) ? (int32_t)seq_offset(m, b) : 0;
      nmax = std::max(nmax, rp.len[i]);
    }
    rp.n = nmax;
    rp.x = off(X, b0 * xs[0], es);
    rp.y = off(Y, b0 * ys[0], es);
    if (launch_rope(rp, p.dtype, p.d_h, stream) != 0) return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_rope_apply(const attn_problem* prob, const attn_mask* mask, const attn_rope* rope,
                            int32_t operand, int32_t inverse, const void* X, void* Y, void* stream) {
  attn_status st = validate_problem(prob, mask);
  if (st != ATTN_OK) return st;
  const attn_problem& p = *prob;
  const attn_mask& m = *mask;
  if ((operand != 0 && operand != 1) || (inverse != 0 && inverse != 1)) return ATTN_ERR_INVALID_ARG;
  st = validate_rope(p, m, rope);
  if (st != ATTN_OK) return st;
  if (p.B == 0 || (operand == 0 ? p.n_q : p.n_k) == 0) return ATTN_OK;
  if (!X || !Y || !aligned16(X) || !aligned16(Y)) return ATTN_ERR_INVALID_ARG;
  const int64_t* s = operand == 0 ? p.q_stride : p.k_stride;
  return rope_enqueue(p, m, rope->cos_sin, operand, inverse, X, s, Y, s, stream);
}

size_t attn_fwd_rope_workspace_size(const attn_problem* prob) {
  if (!sizes_ok(prob)) return 0;
  return rotated_layout(*prob, true).bytes;
}

attn_status attn_fwd_rope(const attn_problem* prob, const attn_mask* mask, const attn_rope* rope, const void* Q,
                          const void* K, const void* V, void* O, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  attn_status st = validate_problem(prob, mask);
  if (st != ATTN_OK) return st;
  const attn_problem& p = *prob;
  const attn_mask& m = *mask;
  st = validate_rope(p, m, rope);
  if (st != ATTN_OK) return st;
  if (p.B == 0 || p.n_q == 0) return ATTN_OK;
  if (!Q || !O || !lse || !aligned16(Q) || !aligned16(O) || !aligned16(lse)) return ATTN_ERR_INVALID_ARG;
  if (p.n_k > 0 && (!K || !V || !aligned16(K) || !aligned16(V))) return ATTN_ERR_INVALID_ARG;
  const Rotated kt = rotated_layout(p, true);
  if (kt.bytes > 0 && (workspace == nullptr || workspace_bytes < kt.bytes || ((uintptr_t)workspace % kWsAlign) != 0))
    return ATTN_ERR_WORKSPACE;
  // keys turned once into the workspace; queries turn in the forward's loads
  if (p.n_k > 0) {
    st = rope_enqueue(p, m, rope->cos_sin, 1, 0, K, p.k_stride, workspace, kt.s, stream);
    if (st != ATTN_OK) return st;
  }
  const size_t es = esize(p.dtype);
  KernelParams kp;
  fill_common(kp, p, m);
  kp.rope = kRopeQ;
  kp.rope_cs = rope->cos_sin;
  kp.k_sb = kt.s[0]; kp.k_sh = kt.s[1]; kp.k_sr = kt.s[2];
  kp.pack = fwd_pack(p) ? 1 : 0;
  const int cs = chunk_size(kp, p.B);
  for (int b0 = 0; b0 < p.B; b0 += cs) {
    const int nb = std::min(cs, p.B - b0);
    fill_chunk(kp, p, m, b0, nb);
    kp.per_group = (int32_t)fwd_items(p, kp.pack != 0);
    kp.q = off(Q, b0 * p.q_stride[0], es);
    kp.k = off((const void*)workspace, b0 * kt.s[0], es);
    kp.v = off(V, b0 * p.v_stride[0], es);
    kp.o_out = off(O, b0 * p.o_stride[0], es);
    kp.lse = lse + b0 * kp.lse_sb;
    if (launch_fwd(kp, p.dtype, p.d_h, p.d_v, stream) != 0) return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

size_t attn_bwd_rope_workspace_size(const attn_problem* prob) {
  if (!sizes_ok(prob)) return 0;
  return attn_bwd_workspace_size(prob) + rotated_layout(*prob, false).bytes + rotated_layout(*prob, true).bytes;
}

attn_status attn_bwd_rope(const attn_problem* prob, const attn_mask* mask, const attn_rope* rope, const void* Q,
                          const void* K, const void* V, const void* O, const float* lse, const void* dO, void* dQ,
                          void* dK, void* dV, void* workspace, size_t workspace_bytes, void* stream) {
  const BwdPtrs t{Q, K, V, O, dO, lse, dQ, dK, dV};
  attn_status st = bwd_check(prob, mask, t, workspace, workspace_bytes, kDq | kDkdv);
  if (st != ATTN_OK) return st;
  const attn_problem& p = *prob;
  const attn_mask& m = *mask;
  st = validate_rope(p, m, rope);
  if (st != ATTN_OK) return st;
  if (p.B == 0 || (p.n_q == 0 && p.n_k == 0)) return ATTN_OK;
  const size_t need = attn_bwd_rope_workspace_size(prob);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace % kWsAlign) != 0))
    return ATTN_ERR_WORKSPACE;
  const Rotated qt = rotated_layout(p, false), kt = rotated_layout(p, true);
  char* ws = (char*)workspace;
  RopeCtx rc;
  rc.cos_sin = rope->cos_sin;
  rc.Qt = ws + attn_bwd_workspace_size(prob);
  rc.Kt = ws + attn_bwd_workspace_size(prob) + qt.bytes;
  for (int i = 0; i < 3; ++i) { rc.qt_s[i] = qt.s[i]; rc.kt_s[i] = kt.s[i]; }
  // q~ is written by the dQ pass as it turns the rows it loads; k~ here
  if (p.n_k > 0) {
    st = rope_enqueue(p, m, rope->cos_sin, 1, 0, K, p.k_stride, (void*)rc.Kt, kt.s, stream);
    if (st != ATTN_OK) return st;
  }
  return bwd_enqueue(p, m, t, (float*)workspace, stream, kDq | kDkdv, &rc);
}

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_EMPTY_ROW: return "an active query row has an empty visible set";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head width or dtype";
    case ATTN_ERR_WORKSPACE: return "backward workspace missing, too small or misaligned";
    case ATTN_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t attn_version(void) { return 200; }

}  // extern "C"
