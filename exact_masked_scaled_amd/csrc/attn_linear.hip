// The projections on either side of the attention core ("Appendix A.10 -
// Attention matrices and backpropagation", eqs. A.10.10-A.10.11): Q = X W_Q,
// K = X W_K, V = X W_V with row-major weights, and in the backward
// G_W = X^T G and G_X = sum over the branches of G W^T.
//
// Plain dense products, so they go to the vendor GEMM (rocBLAS gemm_ex: bf16
// or float32 operands, float32 accumulation).  The projected widths sit side
// by side in one weight matrix and one output matrix ([W_Q | W_K | W_V], and
// the matching [Q | K | V] rows), so one product forms all three projections
// and one product forms G_X: its inner sum over the concatenated columns IS
// the sum over the three branches.  The attention kernels read Q, K and V as
// strided views of that [Q | K | V] matrix (head stride d, row stride the
// full width), and the backward writes G_Q, G_K, G_V into the same layout:
// no transposes or copies between the products and the attention.
//
// The vendor library's handle lives in a context the caller creates
// (attn_gemm_create), passes to every projection call and destroys: the
// library itself holds no handle and allocates nothing on these calls.
//
// Row-major matrices are handed to the column-major GEMM as their transposes:
//   Y   = X W      ->  Y^T   = W^T X^T          (N, N)
//   G_X = G_Y W^T  ->  G_X^T = W G_Y^T          (T, N)
//   G_W = X^T G_Y  ->  G_W^T = G_Y^T X          (N, T)
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <stdint.h>

#include <algorithm>
#include <new>

#include "attn_internal.h"

// The caller-owned GEMM context: the vendor library's handle, bound to the
// device that was current when it was created.  The library keeps no handle
// of its own; every projection call names the context it runs on.
struct attn_gemm_s {
  rocblas_handle h;
  int device;
};

namespace attn {

namespace {

// The context's handle on `stream`, or nullptr when the context is missing or
// belongs to another device than the current one.
rocblas_handle handle_for(attn_gemm ctx, void* stream) {
  int dev = -1;
  if (ctx == nullptr || ctx->h == nullptr || hipGetDevice(&dev) != hipSuccess || dev != ctx->device) return nullptr;
  if (rocblas_set_stream(ctx->h, (hipStream_t)stream) != rocblas_status_success) return nullptr;
  return ctx->h;
}

bool fits_i32(int64_t x) { return x >= 0 && x <= INT32_MAX; }

// D(m x n, column-major, leading dimension ld) = 0 with plain stores, so a
// caller may capture it in a graph (no memset node).
template <typename E>
__global__ void zero_columns(E* D, int64_t ld, int64_t m, int64_t n) {
  const int64_t total = m * n, step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += step) {
    const int64_t c = i / m;
    D[c * ld + (i - c * m)] = E(0);
  }
}

// Column-major D(m x n) = op(A) op(B) (+ D if accumulate), on the stream.
attn_status gemm(attn_gemm ctx, void* stream, int dtype, rocblas_operation ta, rocblas_operation tb, int64_t m, int64_t n, int64_t k,
                 const void* A, int64_t lda, const void* B, int64_t ldb, void* D, int64_t ldd, bool accumulate) {
  if (m == 0 || n == 0) return ATTN_OK;
  if (k == 0) {  // an empty sum: D = 0, or D unchanged when accumulating
    if (accumulate) return ATTN_OK;
    const int64_t blocks = std::min<int64_t>((m * n + 255) / 256, 2048);
    if (dtype == ATTN_BF16)
      zero_columns<uint16_t><<<dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream>>>((uint16_t*)D, ldd, m, n);
    else
      zero_columns<uint32_t><<<dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream>>>((uint32_t*)D, ldd, m, n);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
  }
  rocblas_handle h = handle_for(ctx, stream);
  if (h == nullptr) return ATTN_ERR_INVALID_ARG;
  const rocblas_datatype t = dtype == ATTN_BF16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
  const float alpha = 1.f, beta = accumulate ? 1.f : 0.f;
  const rocblas_status st =
      rocblas_gemm_ex(h, ta, tb, (rocblas_int)m, (rocblas_int)n, (rocblas_int)k, &alpha, A, t, (rocblas_int)lda, B, t,
                      (rocblas_int)ldb, &beta, D, t, (rocblas_int)ldd, D, t, (rocblas_int)ldd, rocblas_datatype_f32_r,
                      rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success ? ATTN_OK : ATTN_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

attn_status validate_linear(const attn_linear* L) {
  if (L == nullptr) return ATTN_ERR_INVALID_ARG;
  if (L->dtype != ATTN_BF16 && L->dtype != ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (L->rows < 0 || L->d_in < 0 || L->d_out < 0) return ATTN_ERR_INVALID_ARG;
  if (L->ld_x < std::max(L->d_in, 1) || L->ld_w < std::max(L->d_out, 1) || L->ld_y < std::max(L->d_out, 1))
    return ATTN_ERR_INVALID_ARG;
  if (!fits_i32(L->ld_x) || !fits_i32(L->ld_w) || !fits_i32(L->ld_y)) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

attn_status linear_fwd(attn_gemm ctx, const attn_linear& L, const void* X, const void* W, void* Y, void* stream) {
  return gemm(ctx, stream, L.dtype, rocblas_operation_none, rocblas_operation_none, L.d_out, L.rows, L.d_in, W, L.ld_w, X,
              L.ld_x, Y, L.ld_y, false);
}

attn_status linear_bwd(attn_gemm ctx, const attn_linear& L, const void* X, const void* W, const void* G_Y, void* G_X,
                       void* G_W, bool accumulate, void* stream) {
  attn_status st = ATTN_OK;
  if (G_X)
    st = gemm(ctx, stream, L.dtype, rocblas_operation_transpose, rocblas_operation_none, L.d_in, L.rows, L.d_out, W, L.ld_w,
              G_Y, L.ld_y, G_X, L.ld_x, accumulate);
  if (st == ATTN_OK && G_W)
    st = gemm(ctx, stream, L.dtype, rocblas_operation_none, rocblas_operation_transpose, L.d_out, L.d_in, L.rows, G_Y,
              L.ld_y, X, L.ld_x, G_W, L.ld_w, accumulate);
  return st;
}

}  // namespace attn

using namespace attn;

extern "C" {

attn_status attn_gemm_create(attn_gemm* out) {
  if (out == nullptr) return ATTN_ERR_INVALID_ARG;
  *out = nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  attn_gemm ctx = new (std::nothrow) attn_gemm_s{nullptr, dev};
  if (ctx == nullptr) return ATTN_ERR_HIP;
  if (rocblas_create_handle(&ctx->h) != rocblas_status_success) {
    delete ctx;
    return ATTN_ERR_HIP;
  }
  *out = ctx;
  return ATTN_OK;
}

attn_status attn_gemm_destroy(attn_gemm ctx) {
  if (ctx == nullptr) return ATTN_OK;
  const rocblas_status st = ctx->h ? rocblas_destroy_handle(ctx->h) : rocblas_status_success;
  delete ctx;
  return st == rocblas_status_success ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_linear_fwd(const attn_linear* L, attn_gemm ctx, const void* X, const void* W, void* Y,
                            void* stream) {
  const attn_status st = validate_linear(L);
  if (st != ATTN_OK) return st;
  if (ctx == nullptr) return ATTN_ERR_INVALID_ARG;
  if (L->rows == 0 || L->d_out == 0) return ATTN_OK;
  if (!Y || !aligned16(Y) || (L->d_in > 0 && (!X || !W || !aligned16(X) || !aligned16(W))))
    return ATTN_ERR_INVALID_ARG;
  return linear_fwd(ctx, *L, X, W, Y, stream);
}

attn_status attn_linear_bwd(const attn_linear* L, attn_gemm ctx, const void* X, const void* W, const void* G_Y,
                            void* G_X, void* G_W, int32_t accumulate, void* stream) {
  const attn_status st = validate_linear(L);
  if (st != ATTN_OK) return st;
  if (ctx == nullptr) return ATTN_ERR_INVALID_ARG;
  if (accumulate != 0 && accumulate != 1) return ATTN_ERR_INVALID_ARG;
  if (G_X && !aligned16(G_X)) return ATTN_ERR_INVALID_ARG;
  if (G_W && !aligned16(G_W)) return ATTN_ERR_INVALID_ARG;
  // operands of products that are not empty
  const bool gx = G_X && L->rows > 0 && L->d_in > 0, gw = G_W && L->d_in > 0 && L->d_out > 0;
  const bool sum_x = gx && L->d_out > 0, sum_w = gw && L->rows > 0;
  if ((sum_x || sum_w) && (!G_Y || !aligned16(G_Y))) return ATTN_ERR_INVALID_ARG;
  if (sum_x && (!W || !aligned16(W))) return ATTN_ERR_INVALID_ARG;
  if (sum_w && (!X || !aligned16(X))) return ATTN_ERR_INVALID_ARG;
  return linear_bwd(ctx, *L, X, W, G_Y, gx ? G_X : nullptr, gw ? G_W : nullptr, accumulate != 0, stream);
}

// ---------------------------------------------------------------- self-attention with its projections

namespace {

// [Q | K | V] columns of one row: H_q d_h, then H_kv d_h, then H_kv d_v.
int64_t qkv_width(const attn_problem& p) {
  return (int64_t)p.H_q * p.d_h + (int64_t)p.H_kv * p.d_h + (int64_t)p.H_kv * p.d_v;
}
int64_t proj_rows(const attn_problem& p) {
  if (p.cu_seqlens_q != nullptr) return p.B > 0 ? p.cu_seqlens_q[p.B] : 0;
  return (int64_t)p.B * p.n_q;
}
size_t es_of(int dtype) { return dtype == ATTN_BF16 ? 2 : 4; }

// The attention problem over the Q / K / V column blocks of a [rows][C]
// matrix; returns false if the shapes do not describe self-attention.
bool qkv_views(const attn_problem& in, attn_problem& p, int64_t off[3]) {
  if (in.n_k != in.n_q) return false;
  if ((in.cu_seqlens_q == nullptr) != (in.cu_seqlens_k == nullptr)) return false;
  p = in;
  const int64_t C = qkv_width(in);
  const int64_t sb = in.cu_seqlens_q ? 0 : (int64_t)in.n_q * C;
  p.q_stride[0] = sb; p.q_stride[1] = in.d_h; p.q_stride[2] = C;
  p.k_stride[0] = sb; p.k_stride[1] = in.d_h; p.k_stride[2] = C;
  p.v_stride[0] = sb; p.v_stride[1] = in.d_v; p.v_stride[2] = C;
  off[0] = 0;
  off[1] = (int64_t)in.H_q * in.d_h;
  off[2] = off[1] + (int64_t)in.H_kv * in.d_h;
  return true;
}

attn_linear qkv_linear(const attn_problem& p, int32_t d_model) {
  attn_linear L;
  L.rows = (int32_t)proj_rows(p);
  L.d_in = d_model;
  L.d_out = (int32_t)qkv_width(p);
  L.dtype = p.dtype;
  L.ld_x = d_model;
  L.ld_w = L.d_out;
  L.ld_y = L.d_out;
  return L;
}

// Checks shared by the self-attention calls: the problem over the views,
// the product, and that Q, K and V come from the same rows.
attn_status prepare_self(const attn_problem* prob, const attn_mask* mask, attn_gemm ctx, int32_t d_model,
                         attn_problem& p, int64_t off[3], attn_linear& L) {
  if (prob == nullptr || mask == nullptr || ctx == nullptr || d_model < 1) return ATTN_ERR_INVALID_ARG;
  if (prob->B < 0 || prob->H_q < 1 || prob->H_kv < 1 || prob->d_h < 0 || prob->d_v < 0) return ATTN_ERR_INVALID_ARG;
  if (!qkv_views(*prob, p, off)) return ATTN_ERR_INVALID_ARG;
  if (p.cu_seqlens_q != nullptr)
    for (int b = 0; b <= p.B; ++b)
      if (p.cu_seqlens_q[b] != p.cu_seqlens_k[b]) return ATTN_ERR_INVALID_ARG;
  if (!fits_i32(qkv_width(p)) || !fits_i32(proj_rows(p))) return ATTN_ERR_INVALID_ARG;
  attn_status st = validate_problem(&p, mask);
  if (st != ATTN_OK) return st;
  L = qkv_linear(p, d_model);
  return validate_linear(&L);
}

const void* cat(const void* base, int64_t elems, size_t es) { return (const char*)base + elems * (int64_t)es; }
void* mat(void* base, int64_t elems, size_t es) { return (char*)base + elems * (int64_t)es; }

}  // namespace

attn_status attn_self_attention_fwd(const attn_problem* prob, const attn_mask* mask, attn_gemm ctx, int32_t d_model,
                                    const void* X, const void* W_qkv, void* QKV, void* O, float* lse, void* stream) {
  attn_problem p;
  int64_t off[3];
  attn_linear L;
  attn_status st = prepare_self(prob, mask, ctx, d_model, p, off, L);
  if (st != ATTN_OK) return st;
  if (L.rows == 0) return ATTN_OK;
  if (!X || !W_qkv || !QKV || !aligned16(X) || !aligned16(W_qkv) || !aligned16(QKV)) return ATTN_ERR_INVALID_ARG;
  if (!O || !lse || !aligned16(O) || !aligned16(lse)) return ATTN_ERR_INVALID_ARG;
  st = linear_fwd(ctx, L, X, W_qkv, QKV, stream);
  if (st != ATTN_OK) return st;
  const size_t es = es_of(p.dtype);
  return attn_fwd(&p, mask, cat(QKV, off[0], es), cat(QKV, off[1], es), cat(QKV, off[2], es), O, lse, stream);
}

size_t attn_self_attention_bwd_workspace_size(const attn_problem* prob) {
  if (prob == nullptr || prob->B < 0 || prob->H_q < 0 || prob->H_kv < 0 || prob->n_q < 0 || prob->d_h < 0 ||
      prob->d_v < 0)
    return 0;
  if (prob->cu_seqlens_q != nullptr && prob->B > 0 && prob->cu_seqlens_q[prob->B] < 0) return 0;
  const size_t g = (size_t)proj_rows(*prob) * (size_t)qkv_width(*prob) * es_of(prob->dtype);
  return attn_bwd_workspace_size(prob) + (g + 255) / 256 * 256;
}

attn_status attn_self_attention_bwd(const attn_problem* prob, const attn_mask* mask, attn_gemm ctx, int32_t d_model,
                                    const void* X, const void* W_qkv, const void* QKV, const void* O, const float* lse,
                                    const void* dO, void* G_X, void* G_W, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  attn_problem p;
  int64_t off[3];
  attn_linear L;
  attn_status st = prepare_self(prob, mask, ctx, d_model, p, off, L);
  if (st != ATTN_OK) return st;
  if (L.rows == 0) {  // no rows: G_W is an empty sum
    if (G_W && !aligned16(G_W)) return ATTN_ERR_INVALID_ARG;
    return linear_bwd(ctx, L, X, W_qkv, nullptr, nullptr, G_W, false, stream);
  }
  if (!X || !W_qkv || !QKV || !aligned16(X) || !aligned16(W_qkv) || !aligned16(QKV)) return ATTN_ERR_INVALID_ARG;
  if (!O || !lse || !dO || !aligned16(O) || !aligned16(lse) || !aligned16(dO)) return ATTN_ERR_INVALID_ARG;
  if ((G_X && !aligned16(G_X)) || (G_W && !aligned16(G_W))) return ATTN_ERR_INVALID_ARG;
  const size_t need = attn_self_attention_bwd_workspace_size(prob), ws_attn = attn_bwd_workspace_size(prob);
  if (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace % 256) != 0) return ATTN_ERR_WORKSPACE;
  const size_t es = es_of(p.dtype);
  void* G = (char*)workspace + ws_attn;  // G_QKV: [rows][C], the layout of QKV
  // G_Q, G_K, G_V into the column blocks of G_QKV (every row written: the
  // inactive rows and padded keys as zeros)
  st = attn_bwd(&p, mask, cat(QKV, off[0], es), cat(QKV, off[1], es), cat(QKV, off[2], es), O, lse, dO,
                mat(G, off[0], es), mat(G, off[1], es), mat(G, off[2], es), workspace, ws_attn, stream);
  if (st != ATTN_OK) return st;
  // G_W = X^T G_QKV; G_X = G_QKV W^T sums the Q, K and V branches
  return linear_bwd(ctx, L, X, W_qkv, G, G_X, G_W, false, stream);
}

}  // extern "C"
