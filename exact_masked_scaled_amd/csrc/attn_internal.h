// Internal (non-ABI) declarations shared by the host dispatcher and the HIP
// kernels of libattn_mi355x.so.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "attn.h"

namespace attn {

// Sequences per launch when per-sequence data are given: lengths, offsets
// and packed row starts travel by value in the kernel arguments (5 x 512 B),
// so longer batches are split into several launches on the same stream.
constexpr int kMaxBatchChunk = 128;

// Everything a kernel needs, passed by value (__grid_constant__).
struct KernelParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;      // forward output (backward input)
  const void* dout;   // G_O
  void* o_out;        // forward: O
  float* lse;         // [B][H_q][n_q]
  float* delta;       // workspace: -D = -rowsum(G_O o O), indexed like lse (written by the dQ pass)
  float* lse2;        // workspace: lse * log2(e), indexed like lse (written by the dQ pass)
  void* dq;
  void* dk;
  void* dv;
  int64_t q_sb, q_sh, q_sr;
  int64_t k_sb, k_sh, k_sr;
  int64_t v_sb, v_sh, v_sr;
  int64_t o_sb, o_sh, o_sr;
  int64_t dq_sb, dq_sh, dq_sr;  // G_Q (the strides of Q unless Q is a rotated copy)
  int64_t dk_sb, dk_sh, dk_sr;  // G_K (likewise for K)
  int32_t B, H_q, H_kv, n_q, n_k;
  int32_t group;        // H_q / H_kv
  int32_t causal;       // 0/1
  int32_t offset;       // causal offset, clamped to [0, n_k]
  float scale;          // 1/sqrt(d_h)
  float scale_log2;     // log2(e)/sqrt(d_h)
  int32_t has_lens;     // 0: every row active, every key valid
  int32_t has_offs;     // 1: per-sequence causal offsets in offs[]
  int32_t varlen;       // 1: packed layout, sequence b starts at rows row0_q/k[b]
  int32_t groups;       // (b, kv-head) units of work
  int32_t per_group;    // work items per unit
  int32_t xcd_map;      // 1: unit u runs on XCD u % 8 (groups % 8 == 0)
  int32_t pack;         // forward: a workgroup's rows are (position, head) pairs of the unit's heads
  int64_t lse_sb, lse_sh;  // element strides of lse and D: sequence, head (rows: 1)
  // forward split over the keys: `splits` parts per row block, each writing
  // its normalised float32 partial output and partial lse at split s of
  // part_o [s][rows][d_v] / part_lse [s][rows] (rows indexed like lse; the
  // split stride is part_rows rows); a combine kernel merges them
  int32_t splits;
  float* part_o;
  float* part_lse;
  int64_t part_rows;
  // dK/dV pass split over the query heads of a group (hsplits > 1): part h
  // of the heads writes float32 partial G_K / G_V of its keys at
  // part_dk [h][krows][d_h] / part_dv [h][krows][d_v], key row index
  // b * krow_sb + g * krow_sh + (first row of the sequence) + j
  int32_t hsplits;
  float* part_dk;
  float* part_dv;
  int64_t krow_sb, krow_sh, part_krows;
  // rotary positions: table [n_pos][d_h/2][2] of (cos, sin); rope flags say
  // which operand a kernel turns (kRopeQ: Q rows as loaded, forward;
  // kRopeDQ / kRopeDK: G_Q / G_K turned back in the stores); query row i of
  // sequence b sits at position i + rope_pos[b], key j at j
  const float* rope_cs;
  int32_t rope;
  // dQ pass with rotary positions: where the rotated query rows are written
  // (the dK/dV pass's copy of q~), with its element strides
  void* qt;
  int64_t qt_sb, qt_sh, qt_sr;
  // backward keeping G_S (bf16): the dK/dV pass writes each step's G_S as
  // 4 KB blocks, block (((b * H_kv + g) * 2 gs_nkb + t) * gs_nqb + qb) * group
  // + rr for 64-key tile t (half t % 2 of 128-key block t / 2), 32-row block
  // qb and query head rr of the group (tile-major, so the blocks the G_Q
  // product reads together, and the ones the dK/dV pass writes in a row, lie
  // side by side); the G_Q product then reads them instead of recomputing S
  // and dP.  Null when not used.
  void* gs;
  int32_t gs_nqb, gs_nkb;
  int32_t lens_q[kMaxBatchChunk];
  int32_t lens_k[kMaxBatchChunk];
  int32_t offs[kMaxBatchChunk];    // causal offsets, clamped to [0, n_k]
  int32_t row0_q[kMaxBatchChunk];  // packed layout: first row of each sequence
  int32_t row0_k[kMaxBatchChunk];
  int32_t rope_pos[kMaxBatchChunk];
};

// kernel arguments are limited to 4 KiB
static_assert(sizeof(KernelParams) <= 4096, "kernel arguments too large");

enum : int32_t { kRopeQ = 1, kRopeDQ = 2, kRopeDK = 4 };

// The standalone rotation: rows i < len[b] of sequence b (first row row0[b]
// in the packed layout) at positions i + pos0[b], all heads; 8 columns per
// thread.
struct RopeParams {
  const void* x;
  void* y;
  const float* cs;
  int64_t x_sb, x_sh, x_sr;
  int64_t y_sb, y_sh, y_sr;
  int32_t B, H, n;   // sequences of this launch, heads, row bound
  int32_t inverse;
  int32_t len[kMaxBatchChunk];
  int32_t row0[kMaxBatchChunk];
  int32_t pos0[kMaxBatchChunk];
};

// Host-only validation; pure C++ (no HIP), shared by attn_validate/fwd/bwd.
attn_status validate_problem(const attn_problem* prob, const attn_mask* mask);

// Dense products of the projections (vendor GEMM); arguments checked.
attn_status validate_linear(const attn_linear* L);
attn_status linear_fwd(attn_gemm ctx, const attn_linear& L, const void* X, const void* W, void* Y, void* stream);
attn_status linear_bwd(attn_gemm ctx, const attn_linear& L, const void* X, const void* W, const void* G_Y, void* G_X,
                       void* G_W, bool accumulate, void* stream);

// Launchers (defined in the .hip translation units).  Return hipSuccess or
// the launch error, as an int to keep this header free of HIP types.
int launch_fwd(const KernelParams& p, int dtype, int d_h, int d_v, void* stream);
int launch_bwd_dq(const KernelParams& p, int dtype, int d_h, int d_v, void* stream);
int launch_bwd_dkdv(const KernelParams& p, int dtype, int d_h, int d_v, void* stream);
// bf16 dK/dV pass by the four-role kernel (attn_bwd_quad.hip)
int launch_bwd_dkdv_quad(const KernelParams& p, int d_h, int d_v, void* stream);
// backward with G_S kept (bf16): the per-row pass (-D, lse log2 e) and G_Q
// from the kept blocks; both use the dQ pass's grid (bwd_gs_block_rows rows
// per workgroup)
int launch_bwd_rows(const KernelParams& p, int d_v, void* stream);
int launch_bwd_dq_gs(const KernelParams& p, int d_h, void* stream);
int bwd_gs_block_rows();
// workgroups of the G_Q product per (sequence, KV head)
int64_t bwd_dq_gs_items(int n_q, int group);
int launch_dkdv_combine(const KernelParams& p, int dtype, int d_h, int d_v, void* stream);
// forward split over the keys (p.splits > 1): partial pass, then the merge
int launch_fwd_split(const KernelParams& p, int dtype, int d_h, int d_v, void* stream);
int launch_fwd_combine(const KernelParams& p, int dtype, int d_v, void* stream);
int launch_rope(const RopeParams& p, int dtype, int d_h, void* stream);

// Tile sizes the dispatcher needs to size grids.
int fwd_block_rows(int dtype);
int bwd_dq_block_rows(int dtype);
int bwd_dkdv_block_keys(int dtype);

}  // namespace attn
