/*
 * attn.h -- C ABI of the MI355X (gfx950) exact masked scaled dot-product
 * attention library (libattn_mi355x.so).
 *
 * Operation ("Appendix A.10 - Attention matrices and backpropagation",
 * glenzli.com, secs. A.10.1-A.10.6, eqs. A.10.1-A.10.9):
 *   for every sequence b, query head r (KV head g = r / (H_q / H_kv)),
 *   active query row i < L_q[b] and its visible set
 *       V_i = { j : j < L_k[b] and (causal == 0 or j <= i + causal_offset) },
 *   S_ij = q_i . k_j / sqrt(d_h)                          (eq. A.10.1)
 *   A_ij = exp(S_ij - m_i) / sum_{r in V_i} exp(S_ir - m_i) on V_i, else 0
 *                                                        (eq. A.10.2)
 *   O = A V                                               (eq. A.10.3)
 *   lse_i = m_i + ln sum_{j in V_i} exp(S_ij - m_i)
 * and given G_O = dL/dO:
 *   G_V = A^T G_O, G_A = G_O V^T                          (eqs. A.10.5-6)
 *   G_S = A o (G_A - c_i), c_i = sum_j A_ij (G_A)_ij       (eq. A.10.7)
 *   G_Q = G_S K / sqrt(d_h), G_K = G_S^T Q / sqrt(d_h)     (eqs. A.10.8-9)
 * with G_K, G_V summed over the query heads that share a KV head
 * (sec. A.10.5).  The chunked-query form (n_q != n_k, a block of new queries
 * against the full history) is the one of "Chapter 31: attention
 * backpropagation" (eonloom handbook), sec. 1; that chapter's sec. 3 also
 * rejects fully masked rows, as this library does.
 *
 * Rows i >= L_q[b] are inactive padding rows: their O, lse and G_Q rows are
 * written as 0 and they contribute nothing to G_K / G_V.  Keys j >= L_k[b]
 * get G_K = G_V = 0 exactly.  The causal offset may differ per sequence
 * (attn_mask.causal_offsets), and the sequences may be stored packed, one
 * after the other with no padding rows (attn_problem.cu_seqlens_q/_k).
 *
 * Layout: every tensor is [B][H][n][d] with unit stride in d; the three outer
 * strides (batch, head, row) are given in ELEMENTS.  G_O and G_Q use the
 * strides of O and Q, G_K and G_V those of K and V.  lse (forward output,
 * backward input) is a contiguous float32 [B][H_q][n_q] array.
 *
 * Ownership and execution: the caller owns every buffer and the stream.  All
 * data pointers are DEVICE pointers except the seqlens arrays, which are HOST
 * arrays read during the call (copied by value into the kernel arguments).
 * Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 * stream); nothing synchronises the host.  The library allocates no device
 * memory on any call except attn_gemm_create (which makes a caller-owned
 * context for the projections' vendor GEMM), and keeps no global mutable
 * state: calls are re-entrant.  The attention calls enqueue kernels only (no
 * memset or copy), so a caller may
 * capture them in a HIP graph; the host arrays are read when the call is
 * made, so every replay of a captured call uses the lengths and offsets it
 * was captured with.
 *
 * The per-sequence arrays (seqlens, causal_offsets, cu_seqlens) are HOST
 * arrays read during the call.
 *
 * Errors: every argument check runs on the host before anything is enqueued;
 * on any error the outputs are untouched.  Calls on different streams that
 * share output buffers race (as any two kernels would).
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad stride, length out of
                               range, H_q not a multiple of H_kv, negative size */
  ATTN_ERR_EMPTY_ROW = 2,   /* an active query row has an empty visible set:
                               L_k[b] == 0 with L_q[b] > 0, or causal with a
                               negative offset (row 0 sees nothing)            */
  ATTN_ERR_UNSUPPORTED = 3, /* head width not in {64, 128}, unknown dtype      */
  ATTN_ERR_WORKSPACE = 4,   /* backward workspace missing or too small         */
  ATTN_ERR_HIP = 5          /* a HIP launch failed                             */
} attn_status;

typedef enum {
  ATTN_F32 = 0,  /* float32 I/O, float32 MFMA, float32 accumulation           */
  ATTN_BF16 = 1  /* bfloat16 I/O, bf16 MFMA with float32 accumulation; P and
                    G_S are rounded to bf16 (nearest-even) before the second
                    products                                                  */
} attn_dtype;

/* The visible sets V_i (see above). */
typedef struct {
  int32_t causal;            /* 0: no causal rule; 1: j <= i + offset_b        */
  int32_t reserved;          /* must be 0                                      */
  int64_t causal_offset;     /* offset_b of every sequence when causal_offsets
                                is NULL: 0 = square top-left causal; n_k - n_q
                                places a block of n_q new queries at the end of
                                the keys                                       */
  const int32_t* seqlens_q;  /* HOST [B] active rows per sequence, or NULL (= n_q) */
  const int32_t* seqlens_k;  /* HOST [B] valid keys per sequence, or NULL (= n_k)  */
  const int64_t* causal_offsets; /* HOST [B] per-sequence offset_b (e.g. each
                                sequence's own cached-history length), or NULL */
} attn_mask;

typedef struct {
  int32_t B, H_q, H_kv;      /* H_q % H_kv == 0; g(r) = r / (H_q / H_kv)       */
  int32_t n_q, n_k;          /* rows of Q/O and of K/V                         */
  int32_t d_h, d_v;          /* widths of Q/K and of V/O: each 64 or 128       */
  int32_t dtype;             /* attn_dtype                                      */
  int64_t q_stride[3];       /* element strides of Q (and G_Q): batch, head, row */
  int64_t k_stride[3];       /* K (and G_K)                                    */
  int64_t v_stride[3];       /* V (and G_V)                                    */
  int64_t o_stride[3];       /* O (and G_O)                                    */
  /* Packed ("varlen") layout: HOST [B + 1] arrays of row offsets, or both
   * NULL for the padded layout above.  Sequence b owns rows
   * cu_seqlens_q[b] .. cu_seqlens_q[b + 1] - 1 of Q / O / G_O / G_Q and
   * cu_seqlens_k[b] .. cu_seqlens_k[b + 1] - 1 of K / V / G_K / G_V, so
   * L_q[b] and L_k[b] are the differences (seqlens_q / seqlens_k must then be
   * NULL) and no padding rows exist.  Element (row t, head h, column c) of Q
   * is at t * q_stride[2] + h * q_stride[1] + c: q_stride[0] (and the other
   * batch strides) must be 0.  n_q and n_k are upper bounds of the lengths
   * (they size the launch grids).  lse and the workspace's per-row arrays are then
   * [H_q][cu_seqlens_q[B]] float32.  Requires cu_seqlens_*[0] == 0,
   * non-decreasing entries and row totals below 2^31. */
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
} attn_problem;

/* Host-only argument check (no device work, no pointers needed).  Returns the
 * status attn_fwd / attn_bwd would return for these sizes and masks, apart
 * from pointer and workspace checks.  It resolves the visible sets of
 * "Appendix A.10" secs. A.10.1 and A.10.6 (causal rule, padded keys and rows)
 * and rejects an active row whose visible set is empty, where the softmax of
 * eq. A.10.2 is undefined, as "Chapter 31: attention backpropagation"
 * (eonloom handbook) sec. 3 prescribes: ATTN_ERR_EMPTY_ROW.  The rule is
 * O(B): row 0 of a sequence sees the fewest keys, so the sequence is valid
 * when it has no active rows, or L_k[b] >= 1 and (not causal or
 * offset_b >= 0). */
attn_status attn_validate(const attn_problem* prob, const attn_mask* mask);

/* Bytes of device workspace attn_bwd needs for `prob` (256-byte aligned
 * base): two per-row float32 arrays of B * H_q * n_q floats each (an upper
 * bound of H_q * cu_seqlens_q[B] in the packed layout), -D_i with
 * D_i = rowsum(G_O o O), the row scalar c_i of "Appendix A.10" eq. A.10.7
 * (c_i = sum_j A_ij sum_l G_O[i,l] V[j,l] = sum_l G_O[i,l] O[i,l]), and
 * lse_i * log2(e), both written by the dQ pass for the dK/dV pass, and, when the
 * problem's grids are too small for the GPU, float32 partials of divided
 * passes: the dQ pass over parts of the keys (when it has fewer than 384
 * workgroups of 128 rows and the keys span at least 8 tiles of 64: parts =
 * min(ceil(512 / workgroups), tiles / 4, 16), each holding G_Q of every row)
 * and the bf16 dK/dV pass over parts of each group's query heads (fewer than
 * 192 workgroups of 128 keys: parts = min(ceil(256 / workgroups), H_q / H_kv,
 * 8), each holding G_K and G_V of every key row); the parts are summed in a
 * fixed order, so results stay reproducible.  Contents on entry are
 * ignored. */
size_t attn_bwd_workspace_size(const attn_problem* prob);

/* Forward ("Appendix A.10" eqs. A.10.1-A.10.3 on the visible sets of
 * secs. A.10.1 and A.10.6): S = Q K^T / sqrt(d_h), the row softmax of S
 * restricted to each row's visible set (max-shifted), O = A V, and the
 * natural-log logsumexp lse_i of the scaled scores over the visible set.
 * Q [B,H_q,n_q,d_h], K [B,H_kv,n_k,d_h], V [B,H_kv,n_k,d_v] in;
 * O [B,H_q,n_q,d_v] and lse [B,H_q,n_q] (float32, contiguous) out; query
 * head r reads KV head r / (H_q / H_kv) (sec. A.10.5).  Device pointers,
 * 16-byte aligned; row strides multiples of 8 elements.  Inactive rows get
 * O = 0 and lse = 0.  Errors: INVALID_ARG, EMPTY_ROW, UNSUPPORTED (see
 * attn_validate), HIP (launch failure); outputs untouched on any error. */
attn_status attn_fwd(const attn_problem* prob, const attn_mask* mask,
                     const void* Q, const void* K, const void* V,
                     void* O, float* lse, void* stream);

/* Forward split over the keys, for problems with few query rows per KV head
 * (a block of new queries, or single decoding rows, against a long cached
 * history: "Chapter 31: attention backpropagation" (eonloom handbook),
 * sec. 1).  Same arguments and results as attn_fwd: the key tiles of every
 * row block are divided into num_splits nearly equal parts computed by
 * separate workgroups, each giving a partial output normalised over its part
 * and its partial logsumexp l_s; a second kernel merges them exactly:
 *   lse = log sum_s exp(l_s),   O = sum_s exp(l_s - lse) O_s
 * (the parts partition each row's visible set).  num_splits <= 0 chooses the
 * count from the sizes (enough workgroups for the whole GPU); at most 1024.
 * `workspace`: device memory of attn_fwd_splitkv_workspace_size(prob,
 * num_splits) bytes, 256-byte aligned (float32 partials; contents on entry
 * ignored).  Results equal attn_fwd's up to float32 rounding order. */
size_t attn_fwd_splitkv_workspace_size(const attn_problem* prob, int32_t num_splits);
attn_status attn_fwd_splitkv(const attn_problem* prob, const attn_mask* mask,
                             const void* Q, const void* K, const void* V,
                             void* O, float* lse, int32_t num_splits,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Backward ("Appendix A.10" eqs. A.10.5-A.10.9, sec. A.10.5): given G_O,
 *   G_V = A^T G_O, G_A = G_O V^T, G_S = A o (G_A - c_i) on the visible set,
 *   G_Q = G_S K / sqrt(d_h), G_K = G_S^T Q / sqrt(d_h),
 * with A recomputed from Q, K and the forward's lse (no n_q x n_k matrix is
 * stored) and G_K, G_V summed over the query heads of each KV head.  Takes
 * the forward's inputs, its outputs O and lse, and G_O (strides of O);
 * writes G_Q (strides of Q), G_K (strides of K) and G_V (strides of V):
 * inactive rows get G_Q = 0, keys past L_k[b] get G_K = G_V = 0.
 * `workspace` is device memory of at least attn_bwd_workspace_size(prob)
 * bytes, 256-byte aligned (WORKSPACE if missing or too small); other errors
 * as attn_fwd. */
attn_status attn_bwd(const attn_problem* prob, const attn_mask* mask,
                     const void* Q, const void* K, const void* V,
                     const void* O, const float* lse, const void* dO,
                     void* dQ, void* dK, void* dV,
                     void* workspace, size_t workspace_bytes, void* stream);

/* The same backward with G_S kept instead of recomputed: G_Q = G_S K /
 * sqrt(d_h) ("Appendix A.10" eq. A.10.8) read from the G_S the dK/dV pass
 * forms for G_K (eq. A.10.9), rather than from S and G_A formed a second
 * time.  Three steps on `stream`: the per-row -D_i and lse_i * log2(e); the
 * dK/dV pass, which also writes G_S in bf16 to the workspace (2 bytes per
 * (row, key) of every 32-row block against every 128-key block it visits);
 * G_Q as one product over those blocks.  Same arguments as attn_bwd; G_K
 * and G_V are bitwise attn_bwd's, G_Q agrees up to rounding (it sums the
 * dK/dV pass's bf16 G_S, which may round differently from the G_S the
 * two-pass dQ pass recomputes).  G_S is written and read with non-temporal
 * stores and loads.
 * `workspace` must hold attn_bwd_gs_workspace_size(prob) bytes, 256-byte
 * aligned: attn_bwd's, then the G_S blocks of the whole batch (B * H_q *
 * ceil(n_q / 32) * ceil(n_k / 128) * 8 KB; 8.6 GB for B = 8, H_q = 32,
 * n = 4096).  bf16 problems with d_h, d_v in {64, 128} whose grids need no
 * division and whose K rows of one sequence span less than 4 GiB take this
 * path; for any other problem the size is attn_bwd_workspace_size's and the
 * call runs attn_bwd. */
size_t attn_bwd_gs_workspace_size(const attn_problem* prob);
attn_status attn_bwd_gs(const attn_problem* prob, const attn_mask* mask,
                        const void* Q, const void* K, const void* V,
                        const void* O, const float* lse, const void* dO,
                        void* dQ, void* dK, void* dV,
                        void* workspace, size_t workspace_bytes, void* stream);
/* attn_bwd_gs one step at a time, for callers that time or schedule them
 * apart: stage 0, 1, 2 in this order (on one stream, same arguments and
 * workspace) equals one attn_bwd_gs call.  With G_S kept they are the
 * per-row pass, the dK/dV pass and the G_Q product; otherwise stage 0 is
 * attn_bwd_dq, stage 1 attn_bwd_dkdv and stage 2 does nothing.  Other stage
 * values return ATTN_ERR_INVALID_ARG. */
attn_status attn_bwd_gs_stage(const attn_problem* prob, const attn_mask* mask,
                              const void* Q, const void* K, const void* V,
                              const void* O, const float* lse, const void* dO,
                              void* dQ, void* dK, void* dV,
                              void* workspace, size_t workspace_bytes,
                              int32_t stage, void* stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): attn_bwd with its
 * workspace in a fixed device array of the library instead of a caller
 * buffer.  Same arguments and results as attn_bwd, without the workspace.
 * The array holds ATTN_BWD_NOALLOC_MAX_WORKSPACE bytes on every device the
 * library runs on (kept until the process ends); a problem whose
 * attn_bwd_workspace_size exceeds it returns ATTN_ERR_WORKSPACE.  The array's
 * device address is resolved on the first call made with a device current
 * (make one call before capturing a graph); no call allocates.  All calls on
 * one device share its array: calls that overlap on one device (other
 * streams, or host threads without ordering) race. */
#define ATTN_BWD_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
attn_status attn_bwd_noalloc(const attn_problem* prob, const attn_mask* mask,
                             const void* Q, const void* K, const void* V,
                             const void* O, const float* lse, const void* dO,
                             void* dQ, void* dK, void* dV, void* stream);

/* The backward in its two passes, for callers that schedule or time them
 * separately; attn_bwd is exactly attn_bwd_dq followed by attn_bwd_dkdv on
 * one stream with one workspace.  Each validates like attn_bwd.
 *   dq:   forms D_i = rowsum(G_O o O) (the row scalar c_i of eq. A.10.7),
 *         stores -D_i and lse_i log2(e) in the workspace and writes G_Q
 *         (eqs. A.10.6-A.10.8);
 *   dkdv: reads those two arrays from the workspace and writes G_K and G_V
 *         (eqs. A.10.5-7, A.10.9), summed over the query heads of each KV
 *         head.
 * Each G_Q, G_K and G_V element is written exactly once (no atomics), so
 * results are bitwise reproducible. */
attn_status attn_bwd_dq(const attn_problem* prob, const attn_mask* mask,
                        const void* Q, const void* K, const void* V,
                        const void* O, const float* lse, const void* dO, void* dQ,
                        void* workspace, size_t workspace_bytes, void* stream);
attn_status attn_bwd_dkdv(const attn_problem* prob, const attn_mask* mask,
                          const void* Q, const void* K, const void* V,
                          const float* lse, const void* dO, void* dK, void* dV,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- rotary positions
 * Attention on rotated queries and keys ("Chapter 15: matrix formulas to look
 * up", math.zhuph.uk, sec. 15.6): q~_i = R_i q_i, k~_j = R_j k_j, where R_t
 * turns every adjacent column pair (2k, 2k+1) of a row at position t by the
 * angle theta(t, k):
 *   x~_2k = cos x_2k - sin x_2k+1,   x~_2k+1 = sin x_2k + cos x_2k+1,
 * so q~_i . k~_j depends on the positions only through j - i when theta is
 * position times a fixed frequency.  V is not rotated.  The backward turns the
 * gradients of q~ and k~ back by -theta ("Chapter 31: attention
 * backpropagation" (eonloom handbook), sec. 5): G_Q = R^T G_Q~, G_K = R^T G_K~.
 *
 * Positions: key j of sequence b sits at position j; query row i at
 * i + offset_b, with offset_b the sequence's causal offset (causal_offsets[b]
 * or causal_offset), used for the positions even when causal == 0.  Every
 * sequence needs L_k[b] <= n_pos and, when it has active rows,
 * 0 <= offset_b and offset_b + L_q[b] <= n_pos (else ATTN_ERR_INVALID_ARG).
 * Rows past L_q[b] and keys past L_k[b] are not rotated. */
typedef struct {
  const float* cos_sin; /* DEVICE float32 [n_pos][d_h / 2][2]: (cos theta, sin
                           theta) of position t, pair k; 16-byte aligned       */
  int32_t n_pos;        /* positions in the table, >= 1                        */
  int32_t reserved;     /* must be 0                                           */
} attn_rope;

/* Rotate the rows of a Q-shaped (operand == 0: H_q heads, n_q rows, strides
 * q_stride, positions i + offset_b, rows i < L_q[b]) or K-shaped (operand ==
 * 1: H_kv heads, n_k rows, k_stride, positions j, rows j < L_k[b]) tensor by
 * R (inverse == 0) or R^T (inverse == 1).  Y has the strides of X and may be
 * X itself (in place); rows past the active ones are not written.  The
 * rotation is computed in float32 and rounded once to the payload type. */
attn_status attn_rope_apply(const attn_problem* prob, const attn_mask* mask, const attn_rope* rope,
                            int32_t operand, int32_t inverse, const void* X, void* Y, void* stream);

/* Forward with rotary positions: O and lse of attention on q~ and k~.  The
 * queries are rotated in registers as they are loaded; the keys are rotated
 * once into the workspace (attn_fwd_rope_workspace_size(prob) bytes, 256-byte
 * aligned, contents on entry ignored).  Other arguments as attn_fwd. */
size_t attn_fwd_rope_workspace_size(const attn_problem* prob);
attn_status attn_fwd_rope(const attn_problem* prob, const attn_mask* mask, const attn_rope* rope,
                          const void* Q, const void* K, const void* V, void* O, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Backward with rotary positions: from the unrotated Q and K, the forward's O
 * and lse, and G_O, writes G_Q = R^T G_Q~, G_K = R^T G_K~ and G_V.  The
 * workspace (attn_bwd_rope_workspace_size(prob) bytes, 256-byte aligned)
 * holds attn_bwd's workspace, then q~, then k~, in contiguous layouts: k~ is rotated into it by
 * a streaming pass, q~ is written by the dQ pass, which turns each query row
 * as it loads it; the dK/dV pass reads both.  The turn back of G_Q~ and G_K~
 * happens in the two passes' stores (no rounding of the rotated gradients in
 * between).  Other arguments as attn_bwd. */
size_t attn_bwd_rope_workspace_size(const attn_problem* prob);
attn_status attn_bwd_rope(const attn_problem* prob, const attn_mask* mask, const attn_rope* rope,
                          const void* Q, const void* K, const void* V,
                          const void* O, const float* lse, const void* dO,
                          void* dQ, void* dK, void* dV,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- projections
 * The products on either side of the core ("Appendix A.10", eqs. A.10.10 and
 * A.10.11), with row-major weights W [d_in][d_out]:
 *   forward   Y = X W                       (Q = X W_Q, K = X W_K, V = X W_V)
 *   backward  G_W = X^T G_Y,  G_X = G_Y W^T
 * A shared input feeds several projections; its gradient is the SUM of their
 * branches, G_X = G_Q W_Q^T + G_K W_K^T + G_V W_V^T (and for cross-attention
 * only the branches that really share an input are summed, the same
 * section).  Storing the weights side by side, W = [W_Q | W_K | W_V], makes
 * both one product: Y = X W holds [Q | K | V] in each row, and G_Y W^T over
 * the concatenated columns is the branch sum.  Separate weights sum through
 * `accumulate`.
 *
 * Products run on the vendor GEMM (rocBLAS: bf16 or float32 operands,
 * float32 accumulation, one rounding of each result to the payload type).
 * Its state lives in a GEMM context that the CALLER creates, passes to every
 * projection call and destroys (attn_gemm_create / attn_gemm_destroy): the
 * library keeps no handle of its own.  A context belongs to the device that
 * was current when it was created (a call on another device returns
 * ATTN_ERR_INVALID_ARG) and holds the stream of its last call, so one
 * context must not be used by two host threads at once.  Errors as
 * elsewhere: checked before anything is enqueued. */
typedef struct attn_gemm_s* attn_gemm;

/* Create a GEMM context on the current device (this call allocates: the
 * vendor handle and its device workspace).  *ctx receives it, or NULL on
 * error (ATTN_ERR_HIP).  The caller owns it until attn_gemm_destroy. */
attn_status attn_gemm_create(attn_gemm* ctx);

/* Destroy a context made by attn_gemm_create (NULL: no-op).  No call may be
 * using it, and work enqueued with it should have completed. */
attn_status attn_gemm_destroy(attn_gemm ctx);

typedef struct {
  int32_t rows;              /* rows of X, Y, G_X and G_Y                      */
  int32_t d_in, d_out;       /* columns of X (rows of W) and of Y (of W)       */
  int32_t dtype;             /* attn_dtype of every operand                    */
  int64_t ld_x, ld_w, ld_y;  /* row strides in elements (G_X, G_W, G_Y share
                                those of X, W, Y); >= the row widths         */
} attn_linear;

/* Y = X W.  Device pointers, 16-byte aligned; `ctx` from attn_gemm_create
 * (NULL: ATTN_ERR_INVALID_ARG). */
attn_status attn_linear_fwd(const attn_linear* lin, attn_gemm ctx, const void* X, const void* W, void* Y,
                            void* stream);

/* G_X = G_Y W^T and G_W = X^T G_Y (either output may be NULL: not formed).
 * accumulate == 1 adds into G_X / G_W instead of overwriting them (summing
 * the branches of a shared input held in separate weights). */
attn_status attn_linear_bwd(const attn_linear* lin, attn_gemm ctx, const void* X, const void* W,
                            const void* G_Y, void* G_X, void* G_W, int32_t accumulate, void* stream);

/* Self-attention with its projections: [Q | K | V] = X W_qkv with X
 * [rows][d_model] and W_qkv [d_model][C], C = H_q d_h + H_kv d_h + H_kv d_v,
 * both contiguous; rows = B n_q (padded) or cu_seqlens_q[B] (packed).  QKV
 * [rows][C] (contiguous) receives the projections; the attention then reads
 * Q, K, V as its column blocks (head h of Q at columns h d_h .., of K at
 * H_q d_h + h d_h .., of V at H_q d_h + H_kv d_h + h d_v ..), so prob's
 * q/k/v strides are ignored; O and lse as attn_fwd (o_stride from prob).
 * Requires n_k == n_q and, packed, cu_seqlens_k equal to cu_seqlens_q. */
attn_status attn_self_attention_fwd(const attn_problem* prob, const attn_mask* mask, attn_gemm ctx,
                                    int32_t d_model, const void* X, const void* W_qkv, void* QKV, void* O,
                                    float* lse, void* stream);

/* Its backward: from X, W_qkv, the forward's QKV, O and lse, and G_O, writes
 * G_X [rows][d_model] = G_Q W_Q^T + G_K W_K^T + G_V W_V^T and G_W [d_model][C]
 * = X^T [G_Q | G_K | G_V] (either may be NULL).  The workspace
 * (attn_self_attention_bwd_workspace_size bytes, 256-byte aligned) holds attn_bwd's workspace
 * and [G_Q | G_K | G_V] [rows][C]. */
size_t attn_self_attention_bwd_workspace_size(const attn_problem* prob);
attn_status attn_self_attention_bwd(const attn_problem* prob, const attn_mask* mask, attn_gemm ctx,
                                    int32_t d_model, const void* X, const void* W_qkv, const void* QKV,
                                    const void* O, const float* lse, const void* dO,
                                    void* G_X, void* G_W,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable name of a status code. */
const char* attn_status_string(attn_status status);

/* Library version (major * 10000 + minor * 100 + patch). */
int32_t attn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ATTN_MI355X_H */
