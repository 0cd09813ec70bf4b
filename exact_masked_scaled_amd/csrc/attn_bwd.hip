// Backward kernels ("Appendix A.10 - Attention matrices and backpropagation",
// glenzli.com, eqs. A.10.5-A.10.9, and sec. A.10.5 for grouped heads).
//
// The backward runs as two passes over the visible (query, key) pairs, each
// recomputing P = exp(S - lse) from the forward's logsumexp (no n_q x n_k
// state is ever stored):
//
//   bwd_dq    query-stationary, shaped like the forward: one workgroup owns
//             128 query rows of one query head, a wave 32 rows (lane = row).
//             It first forms D_i = sum_l G_O[i,l] O[i,l] for its rows (equal to
//             the row scalar c_i of eq. A.10.7, since
//             c_i = sum_j A_ij sum_l G_O[i,l] V[j,l]) and stores it for the
//             second pass.  Then per key tile, with K/V staged in LDS:
//               S^T  = K Q^T, P^T = exp(S^T - lse)          (eqs. A.10.1-2)
//               dP^T = V G_O^T                                (eq. A.10.6)
//               G_S^T = P^T o (dP^T - D)                      (eq. A.10.7)
//               G_Q^T += K^T G_S^T / sqrt(d_h)                (eq. A.10.8)
//             G_S^T has one query per lane, which is exactly the B-operand
//             layout of the last product: no transpose through LDS and no
//             atomics; each G_Q element is written once.
//   bwd_dkdv  key-stationary: one workgroup owns 128 * KT keys of one
//             (sequence, KV head), a wave 32 * KT keys (lane = key), and keeps
//             those keys' K and V rows in registers and their G_K, G_V
//             accumulators.  It walks every query head sharing the KV head
//             (sec. A.10.5: their contributions add up) and every block of 32
//             query rows that sees its keys, with Q / G_O double-buffered in
//             LDS:
//               S = Q K^T, P = exp(S - lse), dP = G_O V^T, G_S = P o (dP - D)
//               G_V += P^T G_O                                (eq. A.10.5)
//               G_K += G_S^T Q / sqrt(d_h)                    (eq. A.10.9)
// Keys at or beyond L_k[b] and rows at or beyond L_q[b] get P = 0 and G_S = 0,
// so padded keys receive exactly zero G_K / G_V and inactive rows zero G_Q.
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {



__device__ __forceinline__ int key_limit_b(int i, int Lk, int causal, int off) {
  return causal ? min(Lk, i + off + 1) : Lk;
}

// ============================================================== dQ pass
template <typename T, int DH, int DV>
struct DqCfg {
  static constexpr int NW = 4;
  static constexpr int BM = 32 * NW;
  static constexpr int BN = 64;
  static constexpr int KS = Tile<T, DH>::STRIDE;
  static constexpr int VS = Tile<T, DV>::STRIDE;
};

// SPLIT: the workgroup covers part s of its row block's key tiles and writes
// its float32 partial G_Q (dq_combine_kernel sums the parts in order).
// ROPE: rotary positions: Q is turned as it is loaded (and written through
// to the rotated copy at p.qt for the dK/dV pass) and G_Q is turned back in
// the stores; its own instance.
template <typename T, int DH, int DV, bool SPLIT, bool ROPE>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void bwd_dq_kernel(const KernelParams p) {
  using C = DqCfg<T, DH, DV>;
  using op_t = typename Op<T>::type;
  // one array per buffer, so the compiler sees that the copy into one buffer
  // never aliases reads of the other and leaves the copy in flight
  __shared__ __attribute__((aligned(16))) T k_lds0[C::BN * C::KS];
  __shared__ __attribute__((aligned(16))) T k_lds1[C::BN * C::KS];
  __shared__ __attribute__((aligned(16))) T v_lds0[C::BN * C::VS];
  __shared__ __attribute__((aligned(16))) T v_lds1[C::BN * C::VS];

  const int nqblk = (p.n_q + C::BM - 1) / C::BM;
  int unit, item;
  if (!map_work(blockIdx.x, p.groups, p.per_group, p.xcd_map, unit, item)) return;
  const int b = unit / p.H_kv, g = unit - (unit / p.H_kv) * p.H_kv;
  int sidx = 0;  // key part of this workgroup (SPLIT)
  if constexpr (SPLIT) {
    sidx = item % p.splits;
    item /= p.splits;
  }
  const int qb = nqblk - 1 - item / p.group;
  const int r = g * p.group + item % p.group;

  // the wave index is the same in every lane: held in a scalar register, so
  // row-range branches are scalar branches
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, kg = lane >> 5;
  const SeqView sv = seq_view(p, b);
  const int Lq = sv.Lq, Lk = sv.Lk, off = sv.off;
  const int q_lo = qb * C::BM;
  const int qi = q_lo + 32 * w + (lane & 31);
  const bool row_exists = qi < sv.nq_lim;
  const bool row_active = qi < Lq;

  const T* Qb = (const T*)p.q + b * p.q_sb + sv.q_row0 * p.q_sr + r * p.q_sh;
  const T* Kb = (const T*)p.k + b * p.k_sb + sv.k_row0 * p.k_sr + g * p.k_sh;
  const T* Vb = (const T*)p.v + b * p.v_sb + sv.k_row0 * p.v_sr + g * p.v_sh;
  const T* Ob = (const T*)p.o + b * p.o_sb + sv.q_row0 * p.o_sr + r * p.o_sh;
  const T* dOb = (const T*)p.dout + b * p.o_sb + sv.q_row0 * p.o_sr + r * p.o_sh;
  T* dQb = (T*)p.dq + b * p.dq_sb + sv.q_row0 * p.dq_sr + r * p.dq_sh;
  const int64_t rowbase = b * p.lse_sb + r * p.lse_sh + sv.q_row0;

  // this lane's G_O row (B operand of dP^T = V G_O^T) and D_i = G_O . O
  op_t doreg[DV / 16];
  float dpart = 0.f;
#pragma unroll
  for (int ks = 0; ks < DV / 16; ++ks) {
    if (row_active) {
      doreg[ks] = ld8<T>(dOb + (int64_t)qi * p.o_sr + 16 * ks + 8 * kg);
      const op_t o8 = ld8<T>(Ob + (int64_t)qi * p.o_sr + 16 * ks + 8 * kg);
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart += (float)doreg[ks][e] * (float)o8[e];
    } else {
      doreg[ks] = zero_op<T>();
    }
  }
  const float Di = row_active ? dpart + partner32(dpart) : 0.f;
  if (row_exists && kg == 0 && sidx == 0) p.delta[rowbase + qi] = Di;
  const float lse2 = row_active ? p.lse[rowbase + qi] * 1.4426950408889634f : 0.f;

  const int act_hi = min(q_lo + C::BM, Lq);
  int ntiles = 0, nfull = 0;
  if (act_hi > q_lo) {
    ntiles = (key_limit_b(act_hi - 1, Lk, p.causal, off) + C::BN - 1) / C::BN;
    nfull = key_limit_b(q_lo, Lk, p.causal, off) / C::BN;
  }
  const int w_lo = q_lo + 32 * w, w_hi = min(w_lo + 32, Lq);
  const int wtiles = w_hi > w_lo ? (key_limit_b(w_hi - 1, Lk, p.causal, off) + C::BN - 1) / C::BN : 0;
  const int kmax_lane = key_limit_b(qi, Lk, p.causal, off);
  // key tiles [t_lo, t_hi) of this workgroup: all, or part sidx of `splits`
  int t_lo = 0, t_hi = ntiles;
  if constexpr (SPLIT) {
    t_lo = (int)((int64_t)sidx * ntiles / p.splits);
    t_hi = (int)((int64_t)(sidx + 1) * ntiles / p.splits);
  }

  f32x16 acc[DH / 32];
#pragma unroll
  for (int i = 0; i < DH / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;

  if (t_hi > t_lo) {
    op_t qreg[DH / 16];
#pragma unroll
    for (int ks = 0; ks < DH / 16; ++ks)
      qreg[ks] = row_active ? ld8<T>(Qb + (int64_t)qi * p.q_sr + 16 * ks + 8 * kg) : zero_op<T>();
    if constexpr (ROPE) {
      // rotary positions: the lane's query row turned as it is loaded (the
      // row at position qi + rope_pos[b]), and the turned row written through
      // to the copy the dK/dV pass reads (each active row once: one
      // workgroup per row block and head)
      const float* cs = p.rope_cs + (int64_t)(max(min(qi, Lq - 1), 0) + p.rope_pos[b]) * DH + 8 * kg;
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) qreg[ks] = rope8<T>(qreg[ks], cs + 16 * ks, false);
      if (row_active) {
        T* qt = (T*)p.qt + b * p.qt_sb + sv.q_row0 * p.qt_sr + r * p.qt_sh + (int64_t)qi * p.qt_sr;
#pragma unroll
        for (int ks = 0; ks < DH / 16; ++ks) st8<T>(qt + 16 * ks + 8 * kg, qreg[ks]);
      }
    }

    // per-lane LDS offsets (K and V tiles share them when d_h == d_v)
    RowOffsets<T, DH> kro;
    RowOffsets<T, DV> vro_own;
    TrOffsets<T, DH> kto;
    kro.init(lane);
    kto.init(lane);
    if constexpr (DH != DV) vro_own.init(lane);
    const RowOffsets<T, DV>& vro = [&]() -> const RowOffsets<T, DV>& {
      if constexpr (DH == DV) return kro; else return vro_own;
    }();

    // The dP^T chain starts from -D_i (one query per lane: every element of
    // the lane's block has the same D_i), so it ends at dP - D_i.
    f32x16 negd;
#pragma unroll
    for (int e = 0; e < 16; ++e) negd[e] = -Di;

    // one key tile, 32 keys at a time: S^T, dP^T - D, G_S^T, then
    // G_Q^T += K^T G_S^T (only one 32-key slice of S^T / dP^T is live at once)
    auto tile = [&](const int t, const T* Ks, const T* Vs) __attribute__((always_inline)) {
      const bool masked = t >= nfull;  // tile straddles the causal diagonal or the key length
#pragma unroll
      for (int mt = 0; mt < C::BN / 32; ++mt) {
        f32x16 s, dp = negd;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.f;
        if constexpr (sizeof(T) == 2 && DH == DV) {
          // the S and dP chains side by side, each operand read PF k-steps
          // ahead of its product (the order pinned through scheduling)
          constexpr int KS = DH / 16, PF = 2;
          op_t ka[PF + 1], va[PF + 1];
#pragma unroll
          for (int j = 0; j < PF; ++j) {
            ka[j] = kro.read(Ks, 32 * mt, j);
            va[j] = vro.read(Vs, 32 * mt, j);
          }
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            if (ks + PF < KS) {
              ka[(ks + PF) % (PF + 1)] = kro.read(Ks, 32 * mt, ks + PF);
              va[(ks + PF) % (PF + 1)] = vro.read(Vs, 32 * mt, ks + PF);
            }
            mma(s, ka[ks % (PF + 1)], qreg[ks]);
            mma(dp, va[ks % (PF + 1)], doreg[ks]);
          }
#pragma unroll
          for (int j = 0; j < PF; ++j) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            if (ks + PF < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < DH / 16; ++ks) mma(s, kro.read(Ks, 32 * mt, ks), qreg[ks]);
#pragma unroll
          for (int ks = 0; ks < DV / 16; ++ks) mma(dp, vro.read(Vs, 32 * mt, ks), doreg[ks]);
        }
        if (masked) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = t * C::BN + 32 * mt + 8 * (e >> 2) + 4 * kg + (e & 3);
            float pv = __builtin_amdgcn_exp2f(fmaf(s[e], p.scale_log2, -lse2));
            pv = key < kmax_lane ? pv : 0.f;
            dp[e] = pv * dp[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(s[e], p.scale_log2, -lse2));
            dp[e] = pv * dp[e];
          }
        }
        // G_Q^T += K^T G_S^T: A = K^T (lane = d) by transposed read, B = G_S^T
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          float tmp[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) tmp[e] = dp[8 * st + e];
          const op_t bop = to_op<T>(tmp);
#pragma unroll
          for (int dt = 0; dt < DH / 32; ++dt) mma(acc[dt], kto.read(Ks, 32 * mt + 16 * st, dt), bop);
        }
      }
    };

    using KL = TileLoad<T, C::BN, DH, 64 * C::NW>;
    using VL = TileLoad<T, C::BN, DV, 64 * C::NW>;
    // buffer copies with 32-bit offsets from row 0 of this (sequence, KV
    // head) when its rows fit, else one resource per row
    const int rows_k = max(sv.nk_lim, C::BN);
    const bool fast = fits_u32<T>(rows_k, p.k_sr, DH) && fits_u32<T>(rows_k, p.v_sr, DV);
    const uint32_t k_srb = (uint32_t)(p.k_sr * (int64_t)sizeof(T)), v_srb = (uint32_t)(p.v_sr * (int64_t)sizeof(T));
    const __amdgpu_buffer_rsrc_t k_rs = buf_rsrc(Kb, 0xffffffffu), v_rs = buf_rsrc(Vb, 0xffffffffu);
    // per-lane copy offsets, fixed for the loop (tiles wholly below L_k take
    // them with the tile's row offset as the scalar offset; the last,
    // partial tile clamps its rows)
    uint32_t k_off[KL::N], v_off[VL::N];
    KL::lane_offsets(p.k_sr, tid, k_off);
    VL::lane_offsets(p.v_sr, tid, v_off);
    auto copy_tile = [&](int t, T* kl, T* vl) __attribute__((always_inline)) {
      if (fast) {
        if ((t + 1) * C::BN <= Lk) {
          KL::issue_buf_full(k_rs, (uint32_t)(t * C::BN) * k_srb, k_off, kl, tid);
          VL::issue_buf_full(v_rs, (uint32_t)(t * C::BN) * v_srb, v_off, vl, tid);
        } else {
          KL::issue_buf(k_rs, k_srb, t * C::BN, Lk, kl, tid);
          VL::issue_buf(v_rs, v_srb, t * C::BN, Lk, vl, tid);
        }
      } else {
        KL::issue_rows(Kb, p.k_sr, t * C::BN, Lk, kl, tid);
        VL::issue_rows(Vb, p.v_sr, t * C::BN, Lk, vl, tid);
      }
    };
    copy_tile(t_lo, k_lds0, v_lds0);
    wait_tile_loads();
    __syncthreads();
    // two tiles per trip so each LDS buffer address is a compile-time constant
    for (int t = t_lo; t < t_hi; t += 2) {
      if (t + 1 < t_hi) copy_tile(t + 1, k_lds1, v_lds1);
      if (t < wtiles) tile(t, k_lds0, v_lds0);
      wait_tile_loads();
      __syncthreads();
      if (t + 1 >= t_hi) break;
      if (t + 2 < t_hi) copy_tile(t + 2, k_lds0, v_lds0);
      if (t + 1 < wtiles) tile(t + 1, k_lds1, v_lds1);
      wait_tile_loads();
      __syncthreads();
    }
  }

  if constexpr (SPLIT) {
    // float32 partial of part sidx (inactive rows: zeros); no rotation (the
    // split is not combined with rotary positions)
    if (row_exists) {
      const float sc = row_active ? p.scale : 0.f;
      float* pq = p.part_o + ((int64_t)sidx * p.part_rows + rowbase + qi) * DH;
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 32 * dt + 8 * j + 4 * kg;
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = acc[dt][4 * j + e] * sc;
          *reinterpret_cast<f32x4*>(pq + d) = v4;
        }
    }
    return;
  }
  if (row_exists) {
    const float sc = row_active ? p.scale : 0.f;
    // rotary positions: G_Q = R^T G_Q~ (the lane's four columns are two
    // pairs); inactive rows (zeros) read an active row's table entries
    constexpr bool turn = ROPE;
    f32x4 tab[DH / 32][4];
    if (turn) {
      // all of the row's table entries in flight at once (pinned so the
      // compiler keeps the loads together)
      const float* cs = p.rope_cs + (int64_t)(max(min(qi, Lq - 1), 0) + p.rope_pos[b]) * DH;
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) tab[dt][j] = *reinterpret_cast<const f32x4*>(cs + 32 * dt + 8 * j + 4 * kg);
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(tab[dt][j]));
    }
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * dt + 8 * j + 4 * kg;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[dt][4 * j + e] * sc;
        if (turn) {
          const f32x4 t = tab[dt][j];
          rope_pair(t[0], -t[1], v[0], v[1]);
          rope_pair(t[2], -t[3], v[2], v[3]);
          if (!row_active) v[0] = v[1] = v[2] = v[3] = 0.f;
        }
        st4<T>(dQb + (int64_t)qi * p.dq_sr + d, v[0], v[1], v[2], v[3]);
      }
  }
}

// ============================================================== dK/dV pass
template <typename T, int DH, int DV>
struct DkvCfg {
  static constexpr int NW = 4;
  static constexpr int KT = 1;                        // 32-key tiles per wave
  static constexpr int BN = 32 * KT * NW;             // keys per workgroup
  static constexpr int BM = 32;                       // query rows per step
  static constexpr int NS = 4;                        // pipeline stages (steps in flight)
  static constexpr int QS = Tile<T, DH>::STRIDE;
  static constexpr int OS = Tile<T, DV>::STRIDE;
};

template <typename T, int DH, int DV>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(const KernelParams p) {
  using C = DkvCfg<T, DH, DV>;
  using op_t = typename Op<T>::type;
  constexpr int KT = C::KT;
  // A ring of NS stages for the Q / G_O tiles of consecutive steps (one array
  // per stage, see bwd_dq_kernel), and per stage and wave its own copy of the
  // 32 rows' lse (natural log) followed by their D.
  constexpr int NS = C::NS;
  __shared__ __attribute__((aligned(16))) T q_st0[C::BM * C::QS];
  __shared__ __attribute__((aligned(16))) T q_st1[C::BM * C::QS];
  __shared__ __attribute__((aligned(16))) T q_st2[C::BM * C::QS];
  __shared__ __attribute__((aligned(16))) T q_st3[C::BM * C::QS];
  __shared__ __attribute__((aligned(16))) T o_st0[C::BM * C::OS];
  __shared__ __attribute__((aligned(16))) T o_st1[C::BM * C::OS];
  __shared__ __attribute__((aligned(16))) T o_st2[C::BM * C::OS];
  __shared__ __attribute__((aligned(16))) T o_st3[C::BM * C::OS];
  __shared__ __attribute__((aligned(16))) float r_st0[C::NW * 2 * C::BM];
  __shared__ __attribute__((aligned(16))) float r_st1[C::NW * 2 * C::BM];
  __shared__ __attribute__((aligned(16))) float r_st2[C::NW * 2 * C::BM];
  __shared__ __attribute__((aligned(16))) float r_st3[C::NW * 2 * C::BM];
  // stage -> arrays (folds to one array when the stage is a constant)
  auto q_st = [&](int st) -> T* { return st == 0 ? q_st0 : st == 1 ? q_st1 : st == 2 ? q_st2 : q_st3; };
  auto o_st = [&](int st) -> T* { return st == 0 ? o_st0 : st == 1 ? o_st1 : st == 2 ? o_st2 : o_st3; };
  auto r_st = [&](int st) -> float* { return st == 0 ? r_st0 : st == 1 ? r_st1 : st == 2 ? r_st2 : r_st3; };

  int unit, kb;
  if (!map_work(blockIdx.x, p.groups, p.per_group, p.xcd_map, unit, kb)) return;
  const int b = unit / p.H_kv, g = unit - (unit / p.H_kv) * p.H_kv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, kg = lane >> 5;
  const SeqView sv = seq_view(p, b);
  const int Lq = sv.Lq, Lk = sv.Lk, off = sv.off, nk_lim = sv.nk_lim;
  const int k_lo = kb * C::BN;
  const int kw0 = k_lo + 32 * KT * w;                 // first key of this wave

  const T* Kb = (const T*)p.k + b * p.k_sb + sv.k_row0 * p.k_sr + g * p.k_sh;
  const T* Vb = (const T*)p.v + b * p.v_sb + sv.k_row0 * p.v_sr + g * p.v_sh;
  T* dKb = (T*)p.dk + b * p.dk_sb + sv.k_row0 * p.dk_sr + g * p.dk_sh;
  T* dVb = (T*)p.dv + b * p.v_sb + sv.k_row0 * p.v_sr + g * p.v_sh;

  f32x16 dk[KT][DH / 32], dv[KT][DV / 32];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
    for (int i = 0; i < DH / 32; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) dk[kt][i][e] = 0.f;
#pragma unroll
    for (int i = 0; i < DV / 32; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) dv[kt][i][e] = 0.f;
  }

  // rows that see any key of this block: causal j <= i + off  =>  i >= k_lo - off
  const int q_first = p.causal ? max(0, k_lo - off) : 0;
  const int qb_first = q_first / C::BM;
  const int qb_end = (Lq + C::BM - 1) / C::BM;
  const int nq = k_lo < Lk && qb_first < qb_end ? qb_end - qb_first : 0;
  const int nsteps = nq * p.group;

  if (nsteps > 0) {
    // K and V rows of this lane's keys as B operands of S = Q K^T and dP = G_O V^T
    op_t kreg[KT][DH / 16], vreg[KT][DV / 16];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int key = kw0 + 32 * kt + (lane & 31);
      const bool ok = key < Lk;
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks)
        kreg[kt][ks] = ok ? ld8<T>(Kb + (int64_t)key * p.k_sr + 16 * ks + 8 * kg) : zero_op<T>();
#pragma unroll
      for (int ks = 0; ks < DV / 16; ++ks)
        vreg[kt][ks] = ok ? ld8<T>(Vb + (int64_t)key * p.v_sr + 16 * ks + 8 * kg) : zero_op<T>();
    }
    // the wave's key range decides whether a step needs the element mask
    const int wk_hi = kw0 + 32 * KT;  // exclusive

    using QL = TileLoad<T, C::BM, DH, 64 * C::NW>;
    using OL = TileLoad<T, C::BM, DV, 64 * C::NW>;
    // vector-memory instructions one wave issues per step (all waves alike)
    constexpr int CPS = QL::N + OL::N + 1;
    // Copies of step s: Q and G_O rows into stage `st`; every wave also copies
    // the 32 rows' lse and D (lanes 0-31 and 32-63) into its own slot, so all
    // waves issue the same number of copies and each reads only its own slot.
    // (everything the copies need is read from the kernel arguments once,
    // here, so no argument load sits behind the copies in the memory queue)
    const T* const q_base = (const T*)p.q + b * p.q_sb + sv.q_row0 * p.q_sr;
    const T* const o_base = (const T*)p.dout + b * p.o_sb + sv.q_row0 * p.o_sr;
    const float* const rows_base = (lane < 32 ? p.lse : p.delta) + b * p.lse_sb + sv.q_row0;
    const int64_t q_sh = p.q_sh, o_sh = p.o_sh, q_sr = p.q_sr, o_sr = p.o_sr, r_sh = p.lse_sh;
    // copies of rows past the last active one repeat it (finite data only)
    const int n_q = Lq, group = p.group;
    auto issue = [&](int s, int st) {
      const int rr = s / nq, qb = qb_first + s % nq;
      const int r = g * group + rr;
      const int q0 = qb * C::BM;
      QL::issue(q_base + r * q_sh, q_sr, q0, n_q, q_st(st), tid);
      OL::issue(o_base + r * o_sh, o_sr, q0, n_q, o_st(st), tid);
      const int qq = min(q0 + (lane & 31), n_q - 1);
      load_lane_floats(rows_base + (int64_t)r * r_sh + qq, r_st(st) + w * 2 * C::BM);
    };

    // per-lane LDS offsets (Q and G_O tiles share them when d_h == d_v)
    RowOffsets<T, DH> qro;
    RowOffsets<T, DV> oro_own;
    TrOffsets<T, DH> qto;
    TrOffsets<T, DV> oto_own;
    qro.init(lane);
    qto.init(lane);
    if constexpr (DH != DV) {
      oro_own.init(lane);
      oto_own.init(lane);
    }
    const RowOffsets<T, DV>& oro = [&]() -> const RowOffsets<T, DV>& {
      if constexpr (DH == DV) return qro; else return oro_own;
    }();
    const TrOffsets<T, DV>& oto = [&]() -> const TrOffsets<T, DV>& {
      if constexpr (DH == DV) return qto; else return oto_own;
    }();

    // one step: 32 query rows of one query head against the wave's keys
    auto step = [&](const int s, const T* Qs, const T* Os, const float* lse_s, const float* dlt_s) {
      const int q0 = (qb_first + s % nq) * C::BM;

      // With bf16 operands every LDS operand of the step is read up front, so
      // the products below run back to back instead of each waiting on its
      // own read (there are registers for it at one wave per SIMD; the float32
      // operands are twice as large and are read where they are used):
      // A operands of S = Q K^T and dP = G_O V^T (row order, lane = query)...
      constexpr bool PRELOAD = sizeof(T) == 2;
      op_t qa[DH / 16], oa[DV / 16];
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) qa[ks] = qro.read(Qs, 0, ks);
#pragma unroll
      for (int ks = 0; ks < DV / 16; ++ks) oa[ks] = oro.read(Os, 0, ks);
      // ...and B operands of G_V += P^T G_O and G_K += G_S^T Q (C order, lane = d)
      op_t ob[2][DV / 32], qb[2][DH / 32];
      auto read_b = [&](int st) {
#pragma unroll
        for (int nt = 0; nt < DV / 32; ++nt) ob[st][nt] = oto.read(Os, 16 * st, nt);
#pragma unroll
        for (int nt = 0; nt < DH / 32; ++nt) qb[st][nt] = qto.read(Qs, 16 * st, nt);
      };
      if constexpr (PRELOAD) read_b(0);
      f32x4 l4[4], d4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        l4[j] = *reinterpret_cast<const f32x4*>(&lse_s[8 * j + 4 * kg]) * 1.4426950408889634f;
        d4[j] = *reinterpret_cast<const f32x4*>(&dlt_s[8 * j + 4 * kg]);
      }

      // S and dP for the wave's keys (lane = key, registers = queries)
      f32x16 sv[KT], dp[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) { sv[kt][e] = 0.f; dp[kt][e] = 0.f; }
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) mma(sv[kt], qa[ks], kreg[kt][ks]);
#pragma unroll
      for (int ks = 0; ks < DV / 16; ++ks)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) mma(dp[kt], oa[ks], vreg[kt][ks]);

      // P = exp(S/sqrt(d) - lse) on the visible set and G_S = P o (dP - D);
      // register e holds query q0 + 8*(e/4) + 4*kg + e%4
      const bool full = (q0 + C::BM <= Lq) && (wk_hi <= Lk) && (!p.causal || wk_hi - 1 <= q0 + off);
      if (full) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float pv = __builtin_amdgcn_exp2f(sv[kt][e] * p.scale_log2 - l4[e >> 2][e & 3]);
            sv[kt][e] = pv;
            dp[kt][e] = pv * (dp[kt][e] - d4[e >> 2][e & 3]);
          }
      } else {
        const int off_eff = p.causal ? off : p.n_k;  // j <= i + n_k always holds
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const int key = kw0 + 32 * kt + (lane & 31);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int q = q0 + 8 * (e >> 2) + 4 * kg + (e & 3);
            const bool vis = (key < Lk) & (q < Lq) & (key <= q + off_eff);
            float pv = __builtin_amdgcn_exp2f(sv[kt][e] * p.scale_log2 - l4[e >> 2][e & 3]);
            pv = vis ? pv : 0.f;
            sv[kt][e] = pv;
            dp[kt][e] = pv * (dp[kt][e] - d4[e >> 2][e & 3]);
          }
        }
      }
      // G_V += P^T G_O, G_K += G_S^T Q (A = this lane's key row, C order over queries)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (!PRELOAD || st == 1) read_b(st);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          float tmp[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) tmp[e] = sv[kt][8 * st + e];
          const op_t pa = to_op<T>(tmp);
#pragma unroll
          for (int e = 0; e < 8; ++e) tmp[e] = dp[kt][8 * st + e];
          const op_t da = to_op<T>(tmp);
#pragma unroll
          for (int nt = 0; nt < DV / 32; ++nt) mma(dv[kt][nt], pa, ob[st][nt]);
#pragma unroll
          for (int nt = 0; nt < DH / 32; ++nt) mma(dk[kt][nt], da, qb[st][nt]);
        }
      }
    };

    // Step s waits for its own copies only (those of the next NS - 2 steps
    // stay in flight), passes a workgroup barrier, issues the copies of step
    // s + NS - 1 into the stage step s - 1 used (every wave is past it), and
    // computes.
    static_assert(NS == 4, "wait_for assumes at most two later steps in flight");
    auto wait_for = [&](int s) {
      const int ahead = min(nsteps - 1, s + NS - 2) - s;  // later steps already issued
      if (ahead >= 2) stage_barrier<2 * CPS>();
      else if (ahead == 1) stage_barrier<CPS>();
      else stage_barrier<0>();
    };
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      if (s < nsteps) issue(s, s);
    if constexpr (sizeof(T) == 4) {  // float32: stage chosen at run time (register budget)
      for (int s = 0; s < nsteps; ++s) {
        const int st = s % NS;
        wait_for(s);
        if (s + NS - 1 < nsteps) issue(s + NS - 1, (s + NS - 1) % NS);
        const float* rw = r_st(st) + w * 2 * C::BM;
        step(s, q_st(st), o_st(st), rw, rw + C::BM);
      }
    } else {
      // NS steps per trip so every stage is a distinct, compile-time LDS object
      for (int s0 = 0; s0 < nsteps; s0 += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
          const int s = s0 + u;
          if (s >= nsteps) break;
          wait_for(s);
          if (s + NS - 1 < nsteps) issue(s + NS - 1, (u + NS - 1) % NS);
          const float* rw = r_st(u) + w * 2 * C::BM;
          step(s, q_st(u), o_st(u), rw, rw + C::BM);
        }
      }
    }
  }

  // store G_K (scaled) and G_V; lane = d, registers = keys
  const bool turn = (p.rope & kRopeDK) != 0, odd = (lane & 1) != 0;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int kbase = kw0 + 32 * kt;
#pragma unroll
    for (int nt = 0; nt < DH / 32; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kbase + 8 * (e >> 2) + 4 * kg + (e & 3);
        float val = dk[kt][nt][e] * p.scale;
        if (turn) {  // rotary positions: G_K = R^T G_K~, key at position key
          const int kc = max(min(key, Lk - 1), 0);
          float2 t = *reinterpret_cast<const float2*>(p.rope_cs + (int64_t)kc * DH +
                                                      ((32 * nt + (lane & 31)) & ~1));
          asm volatile("" : "+v"(t.x), "+v"(t.y));
          const float turned = rope_back_lanes(val, t.x, t.y, odd);
          val = key < Lk ? turned : val;
        }
        if (key < nk_lim) dKb[(int64_t)key * p.dk_sr + 32 * nt + (lane & 31)] = (T)val;
      }
#pragma unroll
    for (int nt = 0; nt < DV / 32; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kbase + 8 * (e >> 2) + 4 * kg + (e & 3);
        if (key < nk_lim) dVb[(int64_t)key * p.v_sr + 32 * nt + (lane & 31)] = (T)dv[kt][nt][e];
      }
  }
}

// ============================================================== dK/dV pass, four roles (bf16)
// Same work unit as bwd_dkdv_kernel (128 keys of one sequence and KV head,
// every query head of the group, 32-row query steps).  Each of the four
// products of a step has its own wave per 64-key half, so every wave keeps a
// 64-key operand or accumulator in registers and each LDS operand read feeds
// two matrix products (half the LDS reads of 32-key waves):
//   XS (waves 0, 1): holds K; S = Q K^T, then P = exp(S - lse) on the visible
//       set, handed on as bf16 MFMA operands;
//   XD (waves 2, 3): holds V; dP = G_O V^T, then G_S = P o (dP - D), handed on;
//   YV (waves 4, 5): G_V += P^T G_O;     YK (waves 6, 7): G_K += G_S^T Q.
// In iteration s, XS forms S of step s and the exponentials of step s - 1; XD
// forms dP of step s - 1 and G_S of step s - 2; YV and YK accumulate step
// s - 3.  Products and element-wise work of one wave are interleaved
// so the exponentials run while the matrix core works; a SIMD holds one X and
// one Y wave.  Q / G_O tiles (and the step's lse and D rows) come through an
// NS-stage ring of direct global-to-LDS copies, issued by the Y waves two
// steps ahead right after the barrier (a wave stalls while its copies queue,
// and its X partner keeps the SIMD busy meanwhile).
template <typename T, int DH, int DV>
struct DkvQuadCfg {
  static constexpr int NW = 8;
  static constexpr int KH = 64;           // keys per half (per wave of a role)
  static constexpr int BN = 2 * KH;       // keys per workgroup
  static constexpr int BM = 32;           // query rows per step
  static constexpr int NS = 6;            // ring stages: steps s - 3 .. s + 2
  static constexpr int PD = NS - 4;       // copy distance in steps
  static constexpr int QCH = BM * Tile<T, DH>::CH;
  static constexpr int OCH = BM * Tile<T, DV>::CH;
  static constexpr int JOBS = (QCH + OCH) / 64;      // wave-instructions of tile copies per step
  static constexpr int JPW = JOBS / 4;               // per Y wave
  static constexpr int CPS = JPW + 1;                // + the lse/D row copy
  static constexpr int KB_S = 2 * DH / 64;           // register blocks of XS's K rows
  static constexpr int KB_D = 2 * DV / 64;           // ... of XD's V rows
  static constexpr int NB_X = (KB_S > KB_D ? KB_S : KB_D) + 4;   // + two S / dP buffers
  static constexpr int NB_Y = 2 * (DH > DV ? DH : DV) / 32;      // accumulators
  static constexpr int NB = NB_X > NB_Y ? NB_X : NB_Y;
  static_assert(QCH % 64 == 0 && OCH % 64 == 0 && JOBS % 4 == 0, "tiles must be whole wave copies");
  static_assert(NS % 2 == 0, "exchange parity follows the stage");
};

// HSPLIT: the workgroup covers part of the group's query heads and writes
// float32 partial G_K / G_V (dkdv_combine_kernel sums the parts in order).
// ROPE: G_K is turned back in the stores (rotary positions).  Separate
// instances keep the other paths' registers out of the plain kernel.
template <typename T, int DH, int DV, bool HSPLIT, bool ROPE>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_quad_kernel(const KernelParams p) {
  static_assert(sizeof(T) == 2, "four-role dK/dV pass is the bf16 path");
  using C = DkvQuadCfg<T, DH, DV>;
  using op_t = typename Op<T>::type;
  constexpr int NS = C::NS, PD = C::PD;
  // one __shared__ array per ring stage (Q tile, G_O tile, lse/D rows),
  // selected at compile time so reads need not wait for unrelated copies
  constexpr int QB = C::BM * DH * (int)sizeof(T), OB = C::BM * DV * (int)sizeof(T);
  constexpr int SB = QB + OB + 2 * C::BM * (int)sizeof(float);
  __shared__ __attribute__((aligned(16))) char st0[SB];
  __shared__ __attribute__((aligned(16))) char st1[SB];
  __shared__ __attribute__((aligned(16))) char st2[SB];
  __shared__ __attribute__((aligned(16))) char st3[SB];
  __shared__ __attribute__((aligned(16))) char st4[SB];
  __shared__ __attribute__((aligned(16))) char st5[SB];
  // P (from XS, three slots: step t in slot t % 3) and G_S (from XD, two
  // slots: step t in slot 3 + t % 2), in one array: per half, per 32-key
  // block and per 16-row k-step one operand per lane, at
  // slot * XSLOT + ((h * 2 + kb) * 2 + ks) * 64 + lane.  The Y waves select
  // their operands and tiles by offsets within one array (never by choosing
  // between arrays), so every LDS read keeps the identity of the object it
  // reads and waits only for copies into that object.
  constexpr int XSLOT = 2 * 2 * 2 * 64;
  __shared__ op_t xch[5 * XSLOT];
  auto stage = [&](auto K) __attribute__((always_inline)) -> char* {
    constexpr int k = decltype(K)::value % NS;
    if constexpr (k == 0) return st0; else if constexpr (k == 1) return st1;
    else if constexpr (k == 2) return st2; else if constexpr (k == 3) return st3;
    else if constexpr (k == 4) return st4; else return st5;
  };
  auto q_st = [&](auto K) __attribute__((always_inline)) -> T* { return reinterpret_cast<T*>(stage(K)); };
  auto o_st = [&](auto K) __attribute__((always_inline)) -> T* { return reinterpret_cast<T*>(stage(K) + QB); };
  auto r_st = [&](auto K) __attribute__((always_inline)) -> float* { return reinterpret_cast<float*>(stage(K) + QB + OB); };

  int unit, kb;
  if (!map_work(blockIdx.x, p.groups, p.per_group, p.xcd_map, unit, kb)) return;
  const int b = unit / p.H_kv, g = unit - (unit / p.H_kv) * p.H_kv;
  // split over the query heads: part hs covers heads [rr_lo, rr_hi) of the group
  int hs = 0, rr_lo = 0, rr_hi = p.group;
  if constexpr (HSPLIT) {
    hs = kb % p.hsplits;
    kb /= p.hsplits;
    rr_lo = (int)((int64_t)hs * p.group / p.hsplits);
    rr_hi = (int)((int64_t)(hs + 1) * p.group / p.hsplits);
  }
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, kg = lane >> 5;
  const int h = w & 1;                                   // key half
  const bool is_x = w < 4, is_s = (w & 2) == 0;          // XS / YV use P, XD / YK use G_S
  const SeqView sv = seq_view(p, b);
  const int Lq = sv.Lq, Lk = sv.Lk, off = sv.off, nk_lim = sv.nk_lim;
  const int k_lo = kb * C::BN;
  const int kh0 = k_lo + C::KH * h;                      // first key of the half
  const int kh_hi = kh0 + C::KH;

  const T* Kb = (const T*)p.k + b * p.k_sb + sv.k_row0 * p.k_sr + g * p.k_sh;
  const T* Vb = (const T*)p.v + b * p.v_sb + sv.k_row0 * p.v_sr + g * p.v_sh;
  T* dKb = (T*)p.dk + b * p.dk_sb + sv.k_row0 * p.dk_sr + g * p.dk_sh;
  T* dVb = (T*)p.dv + b * p.v_sb + sv.k_row0 * p.v_sr + g * p.v_sh;

  // XS: R[0, KB_S) this lane's K rows of both 32-key blocks (operand
  //     kb2 * DH/16 + ks), R[NB_X - 4 + 2j + kb2] the S tile of parity j;
  // XD: the same with V rows and dP tiles;
  // YV / YK: R[kb2 * D/32 + nt] accumulate G_V / G_K.
  f32x16 R[C::NB];
#pragma unroll
  for (int i = 0; i < C::NB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) R[i][e] = 0.f;
  constexpr int XB = C::NB_X - 4;  // first S / dP buffer block

  const int q_first = p.causal ? max(0, k_lo - off) : 0;
  const int qb_first = q_first / C::BM;
  const int qb_end = (Lq + C::BM - 1) / C::BM;
  const int nq = k_lo < Lk && qb_first < qb_end ? qb_end - qb_first : 0;
  const int nsteps = nq * (rr_hi - rr_lo);

  if (nsteps > 0) {
    if (is_x) {
      const T* src = is_s ? Kb : Vb;
      const int64_t sr = is_s ? p.k_sr : p.v_sr;
      const int nks = is_s ? DH / 16 : DV / 16;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const int key = kh0 + 32 * kb2 + (lane & 31);
        const bool ok = key < Lk;
        const T* row = src + (int64_t)key * sr + 8 * kg;
        constexpr int NK = (DH > DV ? DH : DV) / 16;
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          if (ks >= nks) continue;
          const op_t v = ok ? ld8<T>(row + 16 * ks) : zero_op<T>();
          // operand kb2 * nks + ks: the block index is a constant in each role's branch
          if (is_s) {
            if (ks < DH / 16) set_op_part(R[(kb2 * (DH / 16) + ks) / 4], (kb2 * (DH / 16) + ks) % 4, v);
          } else {
            if (ks < DV / 16) set_op_part(R[(kb2 * (DV / 16) + ks) / 4], (kb2 * (DV / 16) + ks) % 4, v);
          }
        }
      }
    }

    // copies (Y waves): per-lane address parts fixed for the loop
    const T* const q_base = (const T*)p.q + b * p.q_sb + sv.q_row0 * p.q_sr;
    const T* const o_base = (const T*)p.dout + b * p.o_sb + sv.q_row0 * p.o_sr;
    const int64_t q_sh = p.q_sh, o_sh = p.o_sh, q_sr = p.q_sr, o_sr = p.o_sr, r_sh = p.lse_sh;
    // copies of rows past the last active one repeat it (finite data only)
    const int n_q = Lq, group = p.group;
    const float* const rows_lane = (lane < 32 ? p.lse : p.delta) + b * p.lse_sb + sv.q_row0 + (lane & 31);
    const int yw = w & 3;  // copy slot of a Y wave
    // per-lane source offset (elements) of each copy instruction within a
    // 32-row block
    int64_t c_off[C::JPW];
#pragma unroll
    for (int i = 0; i < C::JPW; ++i) {
      const int job = yw + 4 * i;
      if (i < C::QCH / 256) {
        using L = Tile<T, DH>;
        const int pc = job * 64 + lane, row = pc / L::CH;
        c_off[i] = row * q_sr + ((pc % L::CH) ^ L::f(row)) * L::EPC;
      } else {
        using L = Tile<T, DV>;
        const int pc = (job - C::QCH / 64) * 64 + lane, row = pc / L::CH;
        c_off[i] = row * o_sr + ((pc % L::CH) ^ L::f(row)) * L::EPC;
      }
    }
    // Exactly CPS copies on every path.
    static_assert(C::QCH % 256 == 0 && C::OCH % 256 == 0, "each Y wave copies whole Q and G_O wave rows");
    auto issue = [&](int rr, int qb, auto ST) __attribute__((always_inline)) {
      const int r = g * group + rr;
      const int q0 = qb * C::BM;
      const T* qt = q_base + r * q_sh + (int64_t)q0 * q_sr;
      const T* ot = o_base + r * o_sh + (int64_t)q0 * o_sr;
      // rows past the last active one repeat it (finite data only): a lane
      // whose row lies past it reads that row's chunk instead
      const int last = n_q - 1 - q0;  // last active row of the block (>= 31: all rows active)
      const int64_t last_q = (int64_t)last * q_sr, last_o = (int64_t)last * o_sr;
      int64_t off[C::JPW];
#pragma unroll
      for (int i = 0; i < C::JPW; ++i) {
        const int job = yw + 4 * i;
        if (i < C::QCH / 256) {
          using L = Tile<T, DH>;
          const int pc = job * 64 + lane, row = pc / L::CH;
          off[i] = row <= last ? c_off[i] : last_q + ((pc % L::CH) ^ L::f(row)) * L::EPC;
        } else {
          using L = Tile<T, DV>;
          const int pc = (job - C::QCH / 64) * 64 + lane, row = pc / L::CH;
          off[i] = row <= last ? c_off[i] : last_o + ((pc % L::CH) ^ L::f(row)) * L::EPC;
        }
      }
      const int qq = q0 + min(lane & 31, last) - (lane & 31);
#pragma unroll
      for (int i = 0; i < C::JPW; ++i) {
        const int job = yw + 4 * i;  // i < QCH / 256: a Q chunk (yw < 4)
        const T* src;
        T* dst;
        if (i < C::QCH / 256) {
          src = qt + off[i];
          dst = q_st(ST) + job * 64 * Tile<T, DH>::EPC;
        } else {
          src = ot + off[i];
          dst = o_st(ST) + (job - C::QCH / 64) * 64 * Tile<T, DV>::EPC;
        }
        __builtin_amdgcn_global_load_lds((const void*)src, (ATTN_LDS void*)dst, 16, 0, 0);
      }
      // every Y wave copies the same lse / D rows (keeps the per-wave count equal)
      load_lane_floats(rows_lane + (int64_t)r * r_sh + qq, r_st(ST));
    };

    // LDS operand offsets, one table for all roles:
    //   XS: Q row operands; XD: G_O row operands;
    //   YV: G_O^T halves ofs[hh * DV/32 + nt]; YK: Q^T halves ofs[hh * DH/32 + nt]
    constexpr int NOFS = (DH > DV ? DH : DV) / 16;
    int ofs[NOFS];
    if (is_x) {
#pragma unroll
      for (int ks = 0; ks < NOFS; ++ks) ofs[ks] = is_s ? RowOffsets<T, DH>::at(lane, ks) : RowOffsets<T, DV>::at(lane, ks);
    } else {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int nt = 0; nt < NOFS / 2; ++nt)
          ofs[hh * (NOFS / 2) + nt] = is_s ? TrOffsets<T, DV>::at(lane, hh, nt) : TrOffsets<T, DH>::at(lane, hh, nt);
    }
    auto row_op = [&](const T* tile, int off) __attribute__((always_inline)) -> op_t {
      return *reinterpret_cast<const op_t*>(reinterpret_cast<const char*>(tile) + off);
    };

    const int off_eff = p.causal ? off : p.n_k;  // j <= i + n_k always holds
    auto full_tile = [&](int q0) __attribute__((always_inline)) {
      return (q0 + C::BM <= Lq) && (kh_hi <= Lk) && (!p.causal || kh_hi - 1 <= q0 + off);
    };

    // ---- XS: S of one step (both key blocks share each Q operand read)
    // interleaved with the exponentials of the previous step
    auto xs_iter = [&](auto MF, auto EX, auto FULL, auto J, const T* Qs, int q0_old, const float* rows,
                       op_t* xb) __attribute__((always_inline)) {
      constexpr bool mf = decltype(MF)::value, ex = decltype(EX)::value;
      constexpr int jn = decltype(J)::value, jo = jn ^ 1;
      f32x16& s0 = R[XB + 2 * jn];
      f32x16& s1 = R[XB + 2 * jn + 1];
      f32x16& o0 = R[XB + 2 * jo];
      f32x16& o1 = R[XB + 2 * jo + 1];
      if constexpr (mf) {
#pragma unroll
        for (int e = 0; e < 16; ++e) { s0[e] = 0.f; s1[e] = 0.f; }
      }
      constexpr int KS = DH / 16;
      constexpr int EPK = 16 / KS;  // elements of each block finished per k-step
      // operands are read one k-step ahead of their products, the rows up front
      f32x4 l4v[4];
      if constexpr (ex) {
#pragma unroll
        for (int j = 0; j < 4; ++j) l4v[j] = *reinterpret_cast<const f32x4*>(&rows[8 * j + 4 * kg]);
      }
      op_t a_nxt;
      if constexpr (mf) a_nxt = row_op(Qs, ofs[0]);
      op_t* xo = xb + (h * 2) * 2 * 64;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (mf) {
          const op_t a = a_nxt;
          if (ks + 1 < KS) a_nxt = row_op(Qs, ofs[ks + 1]);
          mma(s0, a, op_part(R[ks / 4], ks % 4));
          mma(s1, a, op_part(R[(DH / 16 + ks) / 4], (DH / 16 + ks) % 4));
        }
        if constexpr (ex) {
#pragma unroll
          for (int e = EPK * ks; e < EPK * (ks + 1); ++e) {
            const float lse2 = l4v[e >> 2][e & 3] * 1.4426950408889634f;
            const int q = q0_old + 8 * (e >> 2) + 4 * kg + (e & 3);
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
              f32x16& so = kb2 ? o1 : o0;
              const float pv = __builtin_amdgcn_exp2f(fmaf(so[e], p.scale_log2, -lse2));
              if constexpr (decltype(FULL)::value) {
                so[e] = pv;
              } else {
                const int key = kh0 + 32 * kb2 + (lane & 31);
                so[e] = ((key < Lk) & (q < Lq) & (key <= q + off_eff)) ? pv : 0.f;
              }
            }
          }
          if (EPK * (ks + 1) % 8 == 0) {
            const int st = EPK * (ks + 1) / 8 - 1;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
              f32x16& so = kb2 ? o1 : o0;
              float pt[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) pt[e] = so[8 * st + e];
              xo[(kb2 * 2 + st) * 64 + lane] = to_op<T>(pt);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // ---- XD: dP of one step (both key blocks share each G_O operand read)
    // interleaved with G_S of an earlier step (P from XS)
    auto xd_iter = [&](auto MF, auto EX, auto J, const T* Os, const float* rows, const op_t* xpb, op_t* xb) __attribute__((always_inline)) {
      constexpr bool mf = decltype(MF)::value, ex = decltype(EX)::value;
      constexpr int jn = decltype(J)::value, jo = jn ^ 1;
      f32x16& d0 = R[XB + 2 * jn];
      f32x16& d1 = R[XB + 2 * jn + 1];
      f32x16& o0 = R[XB + 2 * jo];
      f32x16& o1 = R[XB + 2 * jo + 1];
      if constexpr (mf) {
#pragma unroll
        for (int e = 0; e < 16; ++e) { d0[e] = 0.f; d1[e] = 0.f; }
      }
      constexpr int KS = DV / 16;
      constexpr int EPK = 16 / KS;
      const op_t* pin = xpb + (h * 2) * 2 * 64;
      op_t* xo = xb + (h * 2) * 2 * 64;
      // operands are read one k-step ahead of their products; D and P up front
      f32x4 d4v[4];
      op_t pp[2][2];
      if constexpr (ex) {
#pragma unroll
        for (int j = 0; j < 4; ++j) d4v[j] = *reinterpret_cast<const f32x4*>(&rows[C::BM + 8 * j + 4 * kg]);
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int st = 0; st < 2; ++st) pp[kb2][st] = pin[(kb2 * 2 + st) * 64 + lane];
      }
      op_t a_nxt;
      if constexpr (mf) a_nxt = row_op(Os, ofs[0]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (mf) {
          const op_t a = a_nxt;
          if (ks + 1 < KS) a_nxt = row_op(Os, ofs[ks + 1]);
          mma(d0, a, op_part(R[ks / 4], ks % 4));
          mma(d1, a, op_part(R[(DV / 16 + ks) / 4], (DV / 16 + ks) % 4));
        }
        if constexpr (ex) {
#pragma unroll
          for (int e = EPK * ks; e < EPK * (ks + 1); ++e) {
            const float dd = d4v[e >> 2][e & 3];
            o0[e] = (float)pp[0][e >> 3][e & 7] * (o0[e] - dd);
            o1[e] = (float)pp[1][e >> 3][e & 7] * (o1[e] - dd);
          }
          if (EPK * (ks + 1) % 8 == 0) {
            const int st = EPK * (ks + 1) / 8 - 1;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
              f32x16& so = kb2 ? o1 : o0;
              float dt[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) dt[e] = so[8 * st + e];
              xo[(kb2 * 2 + st) * 64 + lane] = to_op<T>(dt);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // ---- YV / YK: accumulate step s - 3 (each transposed read feeds both key
    // blocks).  Both roles read that step's ring stage (G_O for YV, Q for YK)
    // and its exchange slot (P for YV, G_S for YK), each chosen by an offset
    // within one array.
    auto y_iter = [&](auto U) __attribute__((always_inline)) {
      constexpr int u = decltype(U)::value;
      const char* stg = stage(IC<u + NS - 3>());
      const T* tile = reinterpret_cast<const T*>(stg + (is_s ? QB : 0));
      const op_t* in = xch + (is_s ? u % 3 : 3 + ((u + 1) & 1)) * XSLOT + (h * 2) * 2 * 64;
      op_t a[2][2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int st = 0; st < 2; ++st) a[kb2][st] = in[(kb2 * 2 + st) * 64 + lane];
      auto products = [&](auto DC) __attribute__((always_inline)) {
        constexpr int D = decltype(DC)::value, NT = D / 32;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const op_t bt = TrOffsets<T, D>::read_at(tile, 16 * st, ofs[nt], ofs[NOFS / 2 + nt]);
            mma(R[nt], a[0][st], bt);
            mma(R[NT + nt], a[1][st], bt);
          }
      };
      // YV: G_V += P^T G_O; YK: G_K += G_S^T Q.  With d_h = d_v one path, so
      // the two roles' accumulators share one register assignment.
      if constexpr (DH == DV) products(IC<DV>());
      else if (is_s) products(IC<DV>());
      else products(IC<DH>());
    };
    // With d_h = d_v the steady loop reads each step's transposed tile
    // operands one step early (its stage has been complete since two barriers
    // before): after the barrier only the exchange-slot reads stand between
    // a Y wave and its products.
    op_t ybt[2][DV / 32];
    auto y_load = [&](auto U) __attribute__((always_inline)) {  // operands of step u - 3
      constexpr int u = decltype(U)::value;
      const char* stg = stage(IC<u + NS - 3>());
      const T* tile = reinterpret_cast<const T*>(stg + (is_s ? QB : 0));
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int nt = 0; nt < DV / 32; ++nt)
          ybt[st][nt] = TrOffsets<T, DV>::read_at(tile, 16 * st, ofs[nt], ofs[NOFS / 2 + nt]);
    };
    auto y_iter_pre = [&](auto U) __attribute__((always_inline)) {
      constexpr int u = decltype(U)::value;
      const op_t* in = xch + (is_s ? u % 3 : 3 + ((u + 1) & 1)) * XSLOT + (h * 2) * 2 * 64;
      op_t a[2][2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int st = 0; st < 2; ++st) a[kb2][st] = in[(kb2 * 2 + st) * 64 + lane];
      constexpr int NT = DV / 32;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          mma(R[nt], a[0][st], ybt[st][nt]);
          mma(R[NT + nt], a[1][st], ybt[st][nt]);
        }
      y_load(IC<u + 1>());
    };

    int i_rr = rr_lo, i_qb = qb_first;   // next step to copy
    int xs_qb = qb_first;            // query block of the step XS exponentiates next
    // after a copy: move on to the next step while one is left (past the last
    // step the copies repeat it, into stages no later step reads)
    auto next = [&](int s_copied, int& rr, int& qb) __attribute__((always_inline)) {
      if (s_copied + 1 < nsteps) {
        if (++qb == qb_end) { qb = qb_first; ++rr; }
      }
    };
    using F = IC<0>;
    using TR = IC<1>;
    // One step of one role (XS = 0, XD = 1, Y = 2).  Every role runs its own
    // loop over the same steps with one barrier each, so a role's loop holds
    // only its own work: the Y loop copies in every step (the same number of
    // copies on every path), which lets the compiler's wait for an LDS read
    // count only the copies into that read's stage instead of every copy in
    // flight, and the X loops hold no copies at all.
    //   RAMP: the step may lie in the ramp-up (0 .. 2) or ramp-down (the last
    //   steps), where roles skip parts; the steady range 3 .. nsteps - 1 has
    //   no such branches, so its loop keeps every register block in place.
    auto step = [&](int s, auto U, auto ROLE, auto RAMP) __attribute__((always_inline)) {
      constexpr int u = decltype(U)::value, role = decltype(ROLE)::value;
      constexpr bool ramp = decltype(RAMP)::value;
      constexpr int jn = u & 1;  // parity of step s (NS even)
      if constexpr (role == 2) {
        // copies of step s + PD are in flight: wait for all but them
        stage_barrier<C::CPS>();
        issue(i_rr, i_qb, IC<u + PD>());
        next(s + PD, i_rr, i_qb);
        // YV / YK: step s - 3 (P or G_S of that step)
        if constexpr (!ramp && DH == DV) y_iter_pre(U);
        else if (!ramp || s >= 3) y_iter(IC<u>());
      } else if constexpr (role == 0) {
        stage_barrier<0>();
        // XS: S(s) and P(s - 1) -> P slot (s - 1) % 3
        op_t* xw = xch + ((u + 2) % 3) * XSLOT;
        const float* rows = r_st(IC<u + NS - 1>());
        const int q0 = xs_qb * C::BM;
        const bool mf = !ramp || s < nsteps, ex = !ramp || (s >= 1 && s <= nsteps);
        if (mf && ex) {
          if (full_tile(q0)) xs_iter(TR(), TR(), TR(), IC<jn>(), q_st(U), q0, rows, xw);
          else xs_iter(TR(), TR(), F(), IC<jn>(), q_st(U), q0, rows, xw);
        } else if constexpr (ramp) {
          if (ex) {
            if (full_tile(q0)) xs_iter(F(), TR(), TR(), IC<jn>(), q_st(U), q0, rows, xw);
            else xs_iter(F(), TR(), F(), IC<jn>(), q_st(U), q0, rows, xw);
          } else if (mf) {
            xs_iter(TR(), F(), TR(), IC<jn>(), q_st(U), q0, rows, xw);
          }
        }
        if (ex) { if (++xs_qb == qb_end) xs_qb = qb_first; }
      } else {
        stage_barrier<0>();
        // XD: dP(s - 1) into parity (s - 1) & 1, G_S(s - 2) -> G_S slot 3 + (s - 2) % 2
        constexpr int jd = (u + 1) & 1;
        const T* Os = o_st(IC<u + NS - 1>());
        const float* rows = r_st(IC<u + NS - 2>());
        const op_t* pin = xch + ((u + 1) % 3) * XSLOT;  // P(s - 2)
        op_t* xw = xch + (3 + (u & 1)) * XSLOT;         // G_S(s - 2)
        const bool mf = !ramp || (s >= 1 && s <= nsteps), ex = !ramp || (s >= 2 && s <= nsteps + 1);
        if (mf && ex) xd_iter(TR(), TR(), IC<jd>(), Os, rows, pin, xw);
        else if constexpr (ramp) {
          if (ex) xd_iter(F(), TR(), IC<jd>(), Os, rows, pin, xw);
          else if (mf) xd_iter(TR(), F(), IC<jd>(), Os, rows, pin, xw);
        }
      }
    };
    static_assert(NS == 6, "the steady loop below is written for six ring stages");
    auto run = [&](auto ROLE) __attribute__((always_inline)) {
      // steps 0 .. nsteps + 2: the ramp-up, the steady loop, the ramp-down
      auto ramp_step = [&](int s, auto U) __attribute__((always_inline)) -> bool {
        if (s > nsteps + 2) return false;
        step(s, U, ROLE, TR());
        return true;
      };
      if (ramp_step(0, IC<0>()) && ramp_step(1, IC<1>()) && ramp_step(2, IC<2>())) {
        int s = 3;
        if constexpr (decltype(ROLE)::value == 2 && DH == DV) {
          if (s + NS <= nsteps) y_load(IC<3>());
        }
        for (; s + NS <= nsteps; s += NS) {
          step(s, IC<3>(), ROLE, F());
          step(s + 1, IC<4>(), ROLE, F());
          step(s + 2, IC<5>(), ROLE, F());
          step(s + 3, IC<0>(), ROLE, F());
          step(s + 4, IC<1>(), ROLE, F());
          step(s + 5, IC<2>(), ROLE, F());
        }
        // the remaining steps s .. nsteps + 2 (at most 8; s % NS == 3)
        if (ramp_step(s, IC<3>()) && ramp_step(s + 1, IC<4>()) && ramp_step(s + 2, IC<5>()) &&
            ramp_step(s + 3, IC<0>()) && ramp_step(s + 4, IC<1>()) && ramp_step(s + 5, IC<2>()) &&
            ramp_step(s + 6, IC<3>()))
          ramp_step(s + 7, IC<4>());
      }
    };
    if (is_x && is_s) {
      run(IC<0>());
    } else if (is_x) {
      run(IC<1>());
    } else {
      // the first two steps' copies; then each step copies the step PD ahead
      issue(i_rr, i_qb, IC<0>());
      next(0, i_rr, i_qb);
      issue(i_rr, i_qb, IC<1>());
      next(1, i_rr, i_qb);
      run(IC<2>());
      // no copy may still be writing LDS when the workgroup ends
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  }

  // store: YV holds G_V, YK G_K (scaled) of both key blocks; lane = column, registers = keys
  auto store = [&](auto NTC, auto TURN, T* dst, int64_t sr, float sc) __attribute__((always_inline)) {
    constexpr int NT = decltype(NTC)::value;
    constexpr bool turn = decltype(TURN)::value;
    const bool odd = (lane & 1) != 0;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int eh = 0; eh < 16; eh += 8) {
          float2 t[8];
          if constexpr (turn) {
            // rotary positions: G_K = R^T G_K~, key kk at position kk.  Eight
            // table entries are read up front, clamped into the valid keys
            // (whose rows exist), and pinned by an empty asm so the compiler
            // cannot sink each load into its guarded store and wait for them
            // one at a time; keys past L_k keep their exact zeros.
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int kk = kh0 + 32 * kb2 + 8 * ((eh + e) >> 2) + 4 * kg + ((eh + e) & 3);
              const int kc = max(min(kk, Lk - 1), 0);
              t[e] = *reinterpret_cast<const float2*>(p.rope_cs + (int64_t)kc * DH + ((32 * nt + (lane & 31)) & ~1));
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(t[e].x), "+v"(t[e].y));
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int kk = kh0 + 32 * kb2 + 8 * ((eh + e) >> 2) + 4 * kg + ((eh + e) & 3);
            float val = R[kb2 * NT + nt][eh + e] * sc;
            if constexpr (turn) {
              const float turned = rope_back_lanes(val, t[e].x, t[e].y, odd);
              val = kk < Lk ? turned : val;
            }
            if (kk < nk_lim) dst[(int64_t)kk * sr + 32 * nt + (lane & 31)] = (T)val;
          }
        }
  };
  if constexpr (HSPLIT) {
    // float32 partials of this part of the heads (no rotation: the split is
    // not combined with rotary positions)
    if (!is_x) {
      const int64_t krow = b * p.krow_sb + g * p.krow_sh + sv.k_row0;
      auto store_part = [&](auto NTC, float* base, int D, float sc) __attribute__((always_inline)) {
        constexpr int NT = decltype(NTC)::value;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int kk = kh0 + 32 * kb2 + 8 * (e >> 2) + 4 * kg + (e & 3);
              if (kk < nk_lim)
                base[((int64_t)hs * p.part_krows + krow + kk) * D + 32 * nt + (lane & 31)] = R[kb2 * NT + nt][e] * sc;
            }
      };
      if (is_s) store_part(IC<DV / 32>(), p.part_dv, DV, 1.f);
      else store_part(IC<DH / 32>(), p.part_dk, DH, p.scale);
    }
    return;
  }
  if (!is_x) {
    if (is_s) store(IC<DV / 32>(), IC<0>(), dVb, p.v_sr, 1.f);
    else if constexpr (ROPE) store(IC<DH / 32>(), IC<1>(), dKb, p.dk_sr, p.scale);
    else store(IC<DH / 32>(), IC<0>(), dKb, p.dk_sr, p.scale);
  }
}

// ============================================================== split sums
// G_Q of a dQ pass split over the keys: the float32 parts summed in order
// (G_Q is a plain sum over the keys, eq. A.10.8), one wave per row.
template <typename T, int DH>
__global__ __launch_bounds__(256) void dq_combine_kernel(const KernelParams p) {
  constexpr int CPL = DH / 64;  // columns per lane
  const int b = blockIdx.z, r = blockIdx.y, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const SeqView sv = seq_view(p, b);
  if (i >= sv.nq_lim) return;
  const int64_t row = b * p.lse_sb + r * p.lse_sh + sv.q_row0 + i;
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  for (int s = 0; s < p.splits; ++s) {
    const float* pq = p.part_o + (s * p.part_rows + row) * DH + CPL * lane;
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] += pq[c];
  }
  T* q = (T*)p.dq + b * p.dq_sb + (sv.q_row0 + i) * p.dq_sr + r * p.dq_sh + CPL * lane;
#pragma unroll
  for (int c = 0; c < CPL; ++c) q[c] = (T)acc[c];
}

// G_K and G_V of a dK/dV pass split over the query heads: the float32 parts
// summed in order (the sums over the group's heads of [A.10 sec. A.10.5]),
// one wave per key row.
template <typename T, int DH, int DV>
__global__ __launch_bounds__(256) void dkdv_combine_kernel(const KernelParams p) {
  const int b = blockIdx.z, g = blockIdx.y, lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const SeqView sv = seq_view(p, b);
  if (j >= sv.nk_lim) return;
  const int64_t krow = b * p.krow_sb + g * p.krow_sh + sv.k_row0 + j;
  {
    constexpr int CPL = DH / 64;
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
    for (int s = 0; s < p.hsplits; ++s) {
      const float* pk = p.part_dk + (s * p.part_krows + krow) * DH + CPL * lane;
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] += pk[c];
    }
    T* dk = (T*)p.dk + b * p.dk_sb + (sv.k_row0 + j) * p.dk_sr + g * p.dk_sh + CPL * lane;
#pragma unroll
    for (int c = 0; c < CPL; ++c) dk[c] = (T)acc[c];
  }
  {
    constexpr int CPL = DV / 64;
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
    for (int s = 0; s < p.hsplits; ++s) {
      const float* pv = p.part_dv + (s * p.part_krows + krow) * DV + CPL * lane;
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] += pv[c];
    }
    T* dv = (T*)p.dv + b * p.v_sb + (sv.k_row0 + j) * p.v_sr + g * p.v_sh + CPL * lane;
#pragma unroll
    for (int c = 0; c < CPL; ++c) dv[c] = (T)acc[c];
  }
}

// ============================================================== launchers
template <typename T, int DH, int DV>
static int launch_dq_t(const KernelParams& p, void* stream) {
  const int64_t units = p.xcd_map ? ((p.groups + 7) / 8) * 8 : p.groups;
  const int64_t grid = units * p.per_group;
  if (grid <= 0) return (int)hipSuccess;
  if (p.splits > 1) {
    hipLaunchKernelGGL((bwd_dq_kernel<T, DH, DV, true, false>), dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL((dq_combine_kernel<T, DH>), dim3((unsigned)((p.n_q + 3) / 4), (unsigned)p.H_q, (unsigned)p.B),
                       dim3(256), 0, (hipStream_t)stream, p);
    return (int)hipGetLastError();
  }
  if (p.rope & kRopeDQ)
    hipLaunchKernelGGL((bwd_dq_kernel<T, DH, DV, false, true>), dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<T, DH, DV, false, false>), dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

template <typename T, int DH, int DV>
static int launch_dkdv_t(const KernelParams& p, void* stream) {
  const int64_t units = p.xcd_map ? ((p.groups + 7) / 8) * 8 : p.groups;
  const int64_t grid = units * p.per_group;
  if (grid <= 0) return (int)hipSuccess;
  if constexpr (sizeof(T) == 2) {
    if (p.hsplits > 1)
      hipLaunchKernelGGL((bwd_dkdv_quad_kernel<T, DH, DV, true, false>), dim3((unsigned)grid), dim3(512), 0,
                         (hipStream_t)stream, p);
    else if (p.rope & kRopeDK)
      hipLaunchKernelGGL((bwd_dkdv_quad_kernel<T, DH, DV, false, true>), dim3((unsigned)grid), dim3(512), 0,
                         (hipStream_t)stream, p);
    else
      hipLaunchKernelGGL((bwd_dkdv_quad_kernel<T, DH, DV, false, false>), dim3((unsigned)grid), dim3(512), 0,
                         (hipStream_t)stream, p);
  } else {
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, DH, DV>), dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, p);
  }
  return (int)hipGetLastError();
}

int bwd_dq_block_rows(int /*dtype*/) { return 128; }
int bwd_dkdv_block_keys(int /*dtype*/) { return 128; }

#define ATTN_DISPATCH(FN)                                                       \
  if (dtype == ATTN_BF16) {                                                     \
    if (d_h == 128 && d_v == 128) return FN<__bf16, 128, 128>(p, stream);       \
    if (d_h == 128 && d_v == 64) return FN<__bf16, 128, 64>(p, stream);         \
    if (d_h == 64 && d_v == 64) return FN<__bf16, 64, 64>(p, stream);           \
    if (d_h == 64 && d_v == 128) return FN<__bf16, 64, 128>(p, stream);         \
  } else {                                                                      \
    if (d_h == 128 && d_v == 128) return FN<float, 128, 128>(p, stream);        \
    if (d_h == 128 && d_v == 64) return FN<float, 128, 64>(p, stream);          \
    if (d_h == 64 && d_v == 64) return FN<float, 64, 64>(p, stream);            \
    if (d_h == 64 && d_v == 128) return FN<float, 64, 128>(p, stream);          \
  }                                                                             \
  return (int)hipErrorInvalidValue;

int launch_bwd_dq(const KernelParams& p, int dtype, int d_h, int d_v, void* stream) {
  ATTN_DISPATCH(launch_dq_t)
}

int launch_bwd_dkdv(const KernelParams& p, int dtype, int d_h, int d_v, void* stream) {
  ATTN_DISPATCH(launch_dkdv_t)
}

template <typename T, int DH, int DV>
static int launch_dkdv_combine_t(const KernelParams& p, void* stream) {
  if (p.B <= 0 || p.n_k <= 0) return (int)hipSuccess;
  hipLaunchKernelGGL((dkdv_combine_kernel<T, DH, DV>), dim3((unsigned)((p.n_k + 3) / 4), (unsigned)p.H_kv, (unsigned)p.B),
                     dim3(256), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

int launch_dkdv_combine(const KernelParams& p, int dtype, int d_h, int d_v, void* stream) {
  ATTN_DISPATCH(launch_dkdv_combine_t)
}

}  // namespace attn
