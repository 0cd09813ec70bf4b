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
//   bwd_dkdv  (float32; the bf16 pass is the four-role kernel of
//             attn_bwd_quad.hip, same work unit and products)
//             key-stationary: one workgroup owns 128 * KT keys of one
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

  // this lane's G_O row (B operand of dP^T = V G_O^T) and D_i = G_O . O; the
  // row's loads (and its lse) are issued together under one branch, so they
  // are in flight at once and waited for once
  op_t doreg[DV / 16], oreg[DV / 16];
  float lse_i = 0.f;
  if (row_active) {
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks) {
      doreg[ks] = ld8<T>(dOb + (int64_t)qi * p.o_sr + 16 * ks + 8 * kg);
      oreg[ks] = ld8<T>(Ob + (int64_t)qi * p.o_sr + 16 * ks + 8 * kg);
    }
    lse_i = p.lse[rowbase + qi];
  } else {
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks) doreg[ks] = oreg[ks] = zero_op<T>();
  }
  float dpart = 0.f;
#pragma unroll
  for (int ks = 0; ks < DV / 16; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart += (float)doreg[ks][e] * (float)oreg[ks][e];
  const float Di = row_active ? dpart + partner32(dpart) : 0.f;
  const float lse2 = row_active ? lse_i * 1.4426950408889634f : 0.f;
  // Stores that nothing in this kernel reads back go last: a store's address
  // and data registers stay claimed until it completes, so an early store
  // makes the next reuse of those registers wait for its write to finish.
  // For the dK/dV pass: -D_i (its dP chains start from it) and lse_i log2 e.
  auto row_stores = [&]() __attribute__((always_inline)) {
    if (row_exists && kg == 0 && sidx == 0) {
      p.delta[rowbase + qi] = -Di;
      p.lse2[rowbase + qi] = lse2;
    }
  };

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
    // this lane's Q row (the loads under one branch, so they are all in
    // flight at once)
    op_t qreg[DH / 16];
    if (row_active) {
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) qreg[ks] = ld8<T>(Qb + (int64_t)qi * p.q_sr + 16 * ks + 8 * kg);
    } else {
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) qreg[ks] = zero_op<T>();
    }
    // rotary positions: the lane's query row is turned (the row at position
    // qi + rope_pos[b]) once the first key tile's copies are in flight; its
    // table entries are loaded with the row, so that wait overlaps the copies
    f32x4 qtab[ROPE ? DH / 16 : 1][2];
    if constexpr (ROPE) {
      const float* cs = p.rope_cs + (int64_t)(max(min(qi, Lq - 1), 0) + p.rope_pos[b]) * DH + 8 * kg;
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) {
        qtab[ks][0] = *reinterpret_cast<const f32x4*>(cs + 16 * ks);
        qtab[ks][1] = *reinterpret_cast<const f32x4*>(cs + 16 * ks + 4);
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
        // each slice's chains scheduled on their own (their read-ahead order
        // below is pinned per slice)
        __builtin_amdgcn_sched_barrier(0);
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
    if constexpr (ROPE) {
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) qreg[ks] = rope8_tab<T>(qreg[ks], qtab[ks][0], qtab[ks][1], false);
    }
    wait_tile_loads();
    __syncthreads();
    // two tiles per trip so each LDS buffer address is a compile-time constant
    for (int t = t_lo; t < t_hi; t += 2) {
      if (t + 1 < t_hi) copy_tile(t + 1, k_lds1, v_lds1);
      if constexpr (ROPE) {
        // the turned row written through to the copy the dK/dV pass reads
        // (each active row once: one workgroup per row block and head),
        // before the first tile's products, so they cover its latency before
        // the tile's wait
        if (t == t_lo && row_active) {
          T* qt = (T*)p.qt + b * p.qt_sb + sv.q_row0 * p.qt_sr + r * p.qt_sh + (int64_t)qi * p.qt_sr;
#pragma unroll
          for (int ks = 0; ks < DH / 16; ++ks) st8<T>(qt + 16 * ks + 8 * kg, qreg[ks]);
        }
      }
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
    row_stores();
    return;
  }
  // rotary positions: G_Q = R^T G_Q~ (the lane's four columns are two
  // pairs); inactive rows (zeros) read an active row's table entries
  constexpr bool turn = ROPE;
  f32x4 tab[DH / 32][4];
  if constexpr (turn) {
    // Each lane needs 16-byte pieces of its own row's table entries, so
    // reading them directly touches a different table row in every lane.
    // Where each wave's K / V buffer (free after the loop's last barrier)
    // holds the wave's 32 table rows, the wave instead copies those rows in
    // whole 1 KB pieces into it (the 16-byte chunk c of row r at position
    // c ^ (r % 16), so the lanes' reads below hit distinct banks) and reads
    // its entries from there.
    constexpr bool staged = sizeof(v_lds0) >= 32 * DH * sizeof(float);
    if constexpr (staged) {
      constexpr int CH = DH / 4, RPI = 64 / CH;  // chunks per row, rows per copy
      static_assert(CH >= 16 && 64 % CH == 0, "table staging needs 16 to 64 chunks per row");
      float* tl = w == 0 ? (float*)k_lds0 : w == 1 ? (float*)k_lds1 : w == 2 ? (float*)v_lds0 : (float*)v_lds1;
      const int r_lo = q_lo + 32 * w;
      const int base_pos = max(min(r_lo, Lq - 1), 0) + p.rope_pos[b];
      const __amdgpu_buffer_rsrc_t trs = buf_rsrc(p.rope_cs + (int64_t)base_pos * DH, 32u * DH * 4u);
#pragma unroll
      for (int i = 0; i < 32 / RPI; ++i) {
        const int r = i * RPI + lane / CH, pos = lane % CH;
        const int rel = max(min(r_lo + r, Lq - 1), 0) + p.rope_pos[b] - base_pos;
        buf_copy16(trs, tl + i * 256, (uint32_t)(rel * DH * 4 + ((pos ^ (r & 15)) * 16)), 0u);
      }
      wait_tile_loads();
      const int r = lane & 31;
      const f32x4* row = reinterpret_cast<const f32x4*>(tl + r * DH);
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) tab[dt][j] = row[(8 * dt + 2 * j + kg) ^ (r & 15)];
    } else {
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
  }
  if (row_exists) {
    const float sc = row_active ? p.scale : 0.f;
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
  row_stores();
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
    const float* const rows_base = (lane < 32 ? p.lse2 : p.delta) + b * p.lse_sb + sv.q_row0;
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
        l4[j] = *reinterpret_cast<const f32x4*>(&lse_s[8 * j + 4 * kg]);  // lse log2 e
        d4[j] = *reinterpret_cast<const f32x4*>(&dlt_s[8 * j + 4 * kg]);  // -D
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
            dp[kt][e] = pv * (dp[kt][e] + d4[e >> 2][e & 3]);
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
            dp[kt][e] = pv * (dp[kt][e] + d4[e >> 2][e & 3]);
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
    return launch_bwd_dkdv_quad(p, DH, DV, stream);  // the four-role kernel (attn_bwd_quad.hip)
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
