// Host-side argument validation of the attention ABI (pure C++, no HIP).
//
// The rules resolve the visible sets of "Appendix A.10 - Attention matrices
// and backpropagation" (glenzli.com), secs. A.10.1 and A.10.6: row i of
// sequence b sees keys j < L_k[b], and with the causal rule only
// j <= i + offset.  Softmax over an empty set is undefined (sec. A.10.1) and
// such rows are rejected, as "Chapter 31: attention backpropagation"
// (eonloom handbook), sec. 3 does.  Row 0 has the smallest visible set of its
// sequence, so the check is O(B): every sequence with an active row needs
// L_k[b] >= 1 and, under the causal rule, its offset >= 0.
#include <stdint.h>

#include "attn_internal.h"

namespace attn {

static bool stride_ok(const int64_t s[3]) {
  for (int i = 0; i < 3; ++i)
    if (s[i] < 0 || (s[i] % 8) != 0) return false;
  return true;
}

static bool width_ok(int d) { return d == 64 || d == 128; }

attn_status validate_problem(const attn_problem* prob, const attn_mask* mask) {
  if (prob == nullptr || mask == nullptr) return ATTN_ERR_INVALID_ARG;
  const attn_problem& p = *prob;
  if (p.B < 0 || p.n_q < 0 || p.n_k < 0 || p.H_q < 1 || p.H_kv < 1) return ATTN_ERR_INVALID_ARG;
  if (p.H_q % p.H_kv != 0) return ATTN_ERR_INVALID_ARG;
  if (p.dtype != ATTN_F32 && p.dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!width_ok(p.d_h) || !width_ok(p.d_v)) return ATTN_ERR_UNSUPPORTED;
  if (!stride_ok(p.q_stride) || !stride_ok(p.k_stride) || !stride_ok(p.v_stride) ||
      !stride_ok(p.o_stride))
    return ATTN_ERR_INVALID_ARG;
  // a row must hold its d elements
  if ((p.n_q > 0 && (p.q_stride[2] < p.d_h || p.o_stride[2] < p.d_v)) ||
      (p.n_k > 0 && (p.k_stride[2] < p.d_h || p.v_stride[2] < p.d_v)))
    return ATTN_ERR_INVALID_ARG;
  const attn_mask& m = *mask;
  if (m.causal != 0 && m.causal != 1) return ATTN_ERR_INVALID_ARG;
  if (m.reserved != 0) return ATTN_ERR_INVALID_ARG;
  // packed layout: both row-offset arrays, no per-sequence lengths besides
  // them, no batch strides, monotone offsets starting at 0
  const bool packed = p.cu_seqlens_q != nullptr || p.cu_seqlens_k != nullptr;
  if (packed) {
    if (p.cu_seqlens_q == nullptr || p.cu_seqlens_k == nullptr) return ATTN_ERR_INVALID_ARG;
    if (m.seqlens_q != nullptr || m.seqlens_k != nullptr) return ATTN_ERR_INVALID_ARG;
    if (p.q_stride[0] != 0 || p.k_stride[0] != 0 || p.v_stride[0] != 0 || p.o_stride[0] != 0)
      return ATTN_ERR_INVALID_ARG;
    if (p.cu_seqlens_q[0] != 0 || p.cu_seqlens_k[0] != 0) return ATTN_ERR_INVALID_ARG;
  }
  for (int b = 0; b < p.B; ++b) {
    int64_t lq, lk;
    if (packed) {
      lq = (int64_t)p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b];
      lk = (int64_t)p.cu_seqlens_k[b + 1] - p.cu_seqlens_k[b];
    } else {
      lq = m.seqlens_q ? (int64_t)m.seqlens_q[b] : (int64_t)p.n_q;
      lk = m.seqlens_k ? (int64_t)m.seqlens_k[b] : (int64_t)p.n_k;
    }
    if (lq < 0 || lq > p.n_q || lk < 0 || lk > p.n_k) return ATTN_ERR_INVALID_ARG;
    if (lq == 0) continue;             // no active row: nothing to define
    if (lk == 0) return ATTN_ERR_EMPTY_ROW;
    const int64_t off = m.causal_offsets ? m.causal_offsets[b] : m.causal_offset;
    if (m.causal && off < 0) return ATTN_ERR_EMPTY_ROW;  // row 0 sees nothing
  }
  // row offsets are int32 in the kernels (cu_seqlens_*[B] < 2^31 by type;
  // the element offsets they scale are 64-bit)
  return ATTN_OK;
}

}  // namespace attn
