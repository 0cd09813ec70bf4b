// Forward kernel: O = softmax_V(Q K^T / sqrt(d_h)) V and the per-row
// logsumexp ("Appendix A.10 - Attention matrices and backpropagation",
// glenzli.com, eqs. A.10.1-A.10.3; the visible sets of secs. A.10.1/A.10.6).
//
// One workgroup = 4 waves = 128 query rows of one (sequence, query head); a
// wave owns 32 rows.  Keys stream through LDS in tiles of 64 (double
// buffered).  Per tile a wave computes the TRANSPOSED score tile
// S^T = K Q^T on MFMA, so that a lane owns one query row (lane % 32) and its
// row statistics need one cross-lane exchange (with lane ^ 32).  The
// probabilities then feed O^T += V^T P^T directly as the B operand (their
// C-layout order is the operand's k order); V^T comes from LDS through the
// transpose read.  The softmax is the shifted one of eq. A.10.2, evaluated
// online: per row a shift m and a running sum l of exp(S - m); the shift
// follows the running maximum (lazily, see below) and the accumulator is
// rescaled whenever it moves.  Because O and l always share one shift, the
// quotient O / l is exactly the softmax-weighted sum in real arithmetic
// (the shift only keeps the exponentials in range).  Whole key tiles beyond a
// row block's visible range are skipped; tiles that straddle the causal
// diagonal or the key length get an element mask.
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {

template <typename T, int DH, int DV>
struct FwdCfg {
  static constexpr int NW = 4;            // waves per workgroup
  static constexpr int BM = 32 * NW;      // query rows per workgroup
  static constexpr int BN = 64;           // keys per tile
  static constexpr int KS = Tile<T, DH>::STRIDE;  // LDS row stride of K tiles (elements)
  static constexpr int VS = Tile<T, DV>::STRIDE;  // LDS row stride of V tiles
};

// Row i sees keys j < kmax(i).
__device__ __forceinline__ int key_limit(int i, int Lk, int causal, int off) {
  return causal ? min(Lk, i + off + 1) : Lk;
}

// SPLIT: the workgroup covers only part s of its row block's key tiles and
// writes a normalised float32 partial output and partial lse (merged by
// fwd_combine_kernel); otherwise it covers all of them and writes O and lse.
// ROPE: the query rows are turned as they are loaded (rotary positions); its
// own instance.
template <typename T, int DH, int DV, bool SPLIT, bool ROPE>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void fwd_kernel(const KernelParams p) {
  using C = FwdCfg<T, DH, DV>;
  using op_t = typename Op<T>::type;
  // separate arrays per buffer: the compiler can then see that the copy into
  // one buffer never aliases reads of the other and keeps the copy in flight
  __shared__ __attribute__((aligned(16))) T k_lds0[C::BN * C::KS];
  __shared__ __attribute__((aligned(16))) T k_lds1[C::BN * C::KS];
  __shared__ __attribute__((aligned(16))) T v_lds0[C::BN * C::VS];
  __shared__ __attribute__((aligned(16))) T v_lds1[C::BN * C::VS];

  int unit, item;
  if (!map_work(blockIdx.x, p.groups, p.per_group, p.xcd_map, unit, item)) return;
  const int b = unit / p.H_kv, g = unit - (unit / p.H_kv) * p.H_kv;
  int sidx = 0;  // key part of this workgroup (SPLIT)
  if constexpr (SPLIT) {
    sidx = item % p.splits;
    item /= p.splits;
  }
  // The rows of a workgroup: 128 query rows of one head (the unit's heads
  // interleaved), or with p.pack 128 consecutive rows rho of the unit's
  // (position, head) pairs, rho -> position rho / group, head g group +
  // rho % group: the heads that share the K/V tiles share the workgroup, so
  // a few positions per head (decoding) still fill it.  Heavy (late) blocks
  // first.
  const bool pack = p.pack != 0;
  int qb, r;
  if (pack) {
    qb = (p.group * p.n_q + C::BM - 1) / C::BM - 1 - item;
    r = 0;  // per lane below
  } else {
    qb = (p.n_q + C::BM - 1) / C::BM - 1 - item / p.group;
    r = g * p.group + item % p.group;
  }

  // the wave index is the same in every lane: held in a scalar register, so
  // row-range branches are scalar branches
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const SeqView sv = seq_view(p, b);
  const int Lq = sv.Lq, Lk = sv.Lk, off = sv.off;
  const int q_lo = qb * C::BM;                          // first row of the block
  const int rho = q_lo + 32 * w + (lane & 31);          // this lane's row
  if (pack) r = g * p.group + rho % p.group;
  auto pos_of = [&](int row) { return pack ? row / p.group : row; };
  const int rows_active = pack ? p.group * Lq : Lq;     // rows before it are active

  const T* Qb = (const T*)p.q + b * p.q_sb + sv.q_row0 * p.q_sr + r * p.q_sh;
  const T* Kb = (const T*)p.k + b * p.k_sb + sv.k_row0 * p.k_sr + g * p.k_sh;
  const T* Vb = (const T*)p.v + b * p.v_sb + sv.k_row0 * p.v_sr + g * p.v_sh;
  T* Ob = (T*)p.o_out + b * p.o_sb + sv.q_row0 * p.o_sr + r * p.o_sh;
  float* lse_b = p.lse + b * p.lse_sb + r * p.lse_sh + sv.q_row0;

  const int qi = pos_of(rho);                           // this lane's query position
  const int kg = lane >> 5;                             // k-group of the lane
  const bool row_exists = qi < sv.nq_lim;
  const bool row_active = qi < Lq;

  // rows of the block that are active, and their positions
  const int act_hi = min(q_lo + C::BM, rows_active);    // exclusive
  int ntiles = 0, nfull = 0;
  if (act_hi > q_lo) {
    const int kend = key_limit(pos_of(act_hi - 1), Lk, p.causal, off);
    const int kfull = key_limit(pos_of(q_lo), Lk, p.causal, off);
    ntiles = (kend + C::BN - 1) / C::BN;
    nfull = kfull / C::BN;
  }
  // this wave's rows
  const int w_lo = q_lo + 32 * w;
  const int w_hi = min(w_lo + 32, rows_active);
  int wtiles = 0;
  if (w_hi > w_lo) wtiles = (key_limit(pos_of(w_hi - 1), Lk, p.causal, off) + C::BN - 1) / C::BN;
  const int kmax_lane = key_limit(qi, Lk, p.causal, off);
  // key tiles [t_lo, t_hi) of this workgroup: all of them, or part sidx of
  // `splits` nearly equal parts
  int t_lo = 0, t_hi = ntiles;
  if constexpr (SPLIT) {
    t_lo = (int)((int64_t)sidx * ntiles / p.splits);
    t_hi = (int)((int64_t)(sidx + 1) * ntiles / p.splits);
  }

  f32x16 oacc[DV / 32];
#pragma unroll
  for (int i = 0; i < DV / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  if (t_hi > t_lo) {
    // Q of this lane's row as the B operand of S^T = K Q^T (row k order)
    op_t qreg[DH / 16];
    // (the row's loads under one branch, so they are all in flight at once)
    if (row_active) {
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) qreg[ks] = ld8<T>(Qb + (int64_t)qi * p.q_sr + 16 * ks + 8 * kg);
    } else {
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) qreg[ks] = zero_op<T>();
    }
    // rotary positions: the table entries of the lane's row (at position
    // qi + rope_pos[b]; inactive rows hold zeros and read an active row's
    // entries) are loaded with the row, so the turn below, made once the
    // first tiles are in flight, does not wait for them one by one
    f32x4 qtab[ROPE ? DH / 16 : 1][2];
    if constexpr (ROPE) {
      const float* cs = p.rope_cs + (int64_t)(max(min(qi, Lq - 1), 0) + p.rope_pos[b]) * DH + 8 * kg;
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) {
        qtab[ks][0] = *reinterpret_cast<const f32x4*>(cs + 16 * ks);
        qtab[ks][1] = *reinterpret_cast<const f32x4*>(cs + 16 * ks + 4);
      }
    }

    RowOffsets<T, DH> kro;
    TrOffsets<T, DV> vto;
    kro.init(lane);
    vto.init(lane);
    const float tau_raw = 8.f / p.scale_log2;
    // K/V tiles stream through two LDS buffers, copied from memory into LDS
    // by buffer loads (no staging registers)
    using KL = TileLoad<T, C::BN, DH, 64 * C::NW>;
    using VL = TileLoad<T, C::BN, DV, 64 * C::NW>;
    // per-lane copy offsets, fixed for the loop (tiles wholly below L_k take
    // them with the tile's row offset as the scalar offset; the last,
    // partial tile clamps its rows)
    uint32_t k_off[KL::N], v_off[VL::N];
    // buffer copies with 32-bit offsets from row 0 of this (sequence, KV
    // head) when its rows fit, else one resource per row
    const int rows_k = max(sv.nk_lim, C::BN);
    const bool fast = fits_u32<T>(rows_k, p.k_sr, DH) && fits_u32<T>(rows_k, p.v_sr, DV);
    const uint32_t k_srb = (uint32_t)(p.k_sr * (int64_t)sizeof(T)), v_srb = (uint32_t)(p.v_sr * (int64_t)sizeof(T));
    const __amdgpu_buffer_rsrc_t k_rs = buf_rsrc(Kb, 0xffffffffu), v_rs = buf_rsrc(Vb, 0xffffffffu);
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
      // the lane's row turned while the first tiles are in flight
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) qreg[ks] = rope8_tab<T>(qreg[ks], qtab[ks][0], qtab[ks][1], false);
    }
    wait_tile_loads();
    __syncthreads();

    auto tile = [&](const int t, const T* Ks, const T* Vs) __attribute__((always_inline)) {
        // S^T tile: keys (rows) x this wave's 32 queries (columns), raw scores
        // the key blocks' product chains side by side, each K operand read
        // PF k-steps ahead of its product
        f32x16 s[C::BN / 32];
#pragma unroll
        for (int mt = 0; mt < C::BN / 32; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) s[mt][e] = 0.f;
        constexpr int KS = DH / 16, PF = 2;
        op_t ka[PF + 1][C::BN / 32];
#pragma unroll
        for (int j = 0; j < PF; ++j)
#pragma unroll
          for (int mt = 0; mt < C::BN / 32; ++mt) ka[j][mt] = kro.read(Ks, 32 * mt, j);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + PF < KS) {
#pragma unroll
            for (int mt = 0; mt < C::BN / 32; ++mt) ka[(ks + PF) % (PF + 1)][mt] = kro.read(Ks, 32 * mt, ks + PF);
          }
#pragma unroll
          for (int mt = 0; mt < C::BN / 32; ++mt) mma(s[mt], ka[ks % (PF + 1)][mt], qreg[ks]);
        }
        // keep that order through scheduling: PF groups of reads, then per
        // k-step the reads PF steps ahead before that step's products
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int j = 0; j < PF; ++j) __builtin_amdgcn_sched_group_barrier(0x100, C::BN / 32, 0);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            if (ks + PF < KS) __builtin_amdgcn_sched_group_barrier(0x100, C::BN / 32, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, C::BN / 32, 0);
          }
        }
        if (t >= nfull) {  // tile straddles the causal diagonal or the key length
#pragma unroll
          for (int mt = 0; mt < C::BN / 32; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int key = t * C::BN + 32 * mt + 8 * (e >> 2) + 4 * kg + (e & 3);
              s[mt][e] = key < kmax_lane ? s[mt][e] : -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < C::BN / 32; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mt][e]);
        mx = fmaxf(mx, partner32(mx));
        // The shift m (raw-score units) follows the running max lazily: it only
        // moves when the max exceeds it by more than 8 in log2 units, so the
        // probabilities stay below 2^8 and the accumulator is rescaled rarely.
        // O and l always share the same shift, so the quotient is unchanged.
        const bool grow = mx > m_run + tau_raw;
        if (__any(grow)) {
          const float m_new = grow ? mx : m_run;
          const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * p.scale_log2);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int i = 0; i < DV / 32; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
        }
        const float mc = m_run == -INFINITY ? 0.f : m_run * p.scale_log2;
        float psum = 0.f;
#pragma unroll
        for (int mt = 0; mt < C::BN / 32; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float pe = __builtin_amdgcn_exp2f(fmaf(s[mt][e], p.scale_log2, -mc));
            s[mt][e] = pe;
            psum += pe;
          }
        l_run += psum;
        // O^T += V^T P^T, contracting over the tile's keys in C order
#pragma unroll
        for (int mt = 0; mt < C::BN / 32; ++mt)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pv[e] = s[mt][8 * st + e];
            const op_t bop = to_op<T>(pv);
#pragma unroll
            for (int dt = 0; dt < DV / 32; ++dt) mma(oacc[dt], vto.read(Vs, 32 * mt + 16 * st, dt), bop);
          }
    };

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

  // epilogue: O = acc / l, lse = ln2 * (m + log2 l); inactive rows get zeros
  const float l_tot = l_run + partner32(l_run);
  const float inv = (row_active && l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if constexpr (SPLIT) {
    // partial of split sidx: a row that saw no key of this part gets lse = -inf
    if (row_exists) {
      const int64_t prow = (int64_t)sidx * p.part_rows + b * p.lse_sb + r * p.lse_sh + sv.q_row0 + qi;
      float* po = p.part_o + prow * DV;
#pragma unroll
      for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 32 * dt + 8 * j + 4 * kg;
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = oacc[dt][4 * j + e] * inv;
          *reinterpret_cast<f32x4*>(po + d) = v4;
        }
      if (kg == 0)
        p.part_lse[prow] = (row_active && l_tot > 0.f)
                               ? (m_run * p.scale_log2 + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994530942f
                               : -INFINITY;
    }
    return;
  }
  if (row_exists) {
#pragma unroll
    for (int dt = 0; dt < DV / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * dt + 8 * j + 4 * kg;
        st4<T>(Ob + (int64_t)qi * p.o_sr + d, oacc[dt][4 * j] * inv, oacc[dt][4 * j + 1] * inv,
               oacc[dt][4 * j + 2] * inv, oacc[dt][4 * j + 3] * inv);
      }
    if (kg == 0)
      lse_b[qi] = row_active ? (m_run * p.scale_log2 + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994530942f
                             : 0.f;
  }
}

// Merge of the key parts of a split forward, one wave per row: with the
// partial logsumexps l_s and outputs O_s (each normalised over its part),
//   lse = log sum_s exp(l_s),  O = sum_s exp(l_s - lse) O_s,
// which is the softmax-weighted sum over the union of the parts (the parts
// partition the visible set; a part the row does not see has l_s = -inf).
// Inactive rows get O = 0 and lse = 0 as in the unsplit forward.
template <typename T, int DV>
__global__ __launch_bounds__(256) void fwd_combine_kernel(const KernelParams p) {
  constexpr int CPL = DV / 64;  // columns per lane
  const int b = blockIdx.z, r = blockIdx.y, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const SeqView sv = seq_view(p, b);
  if (i >= sv.nq_lim) return;
  const int64_t row = b * p.lse_sb + r * p.lse_sh + sv.q_row0 + i;
  T* orow = (T*)p.o_out + b * p.o_sb + (sv.q_row0 + i) * p.o_sr + r * p.o_sh + CPL * lane;
  if (i >= sv.Lq) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) orow[c] = (T)0.f;
    if (lane == 0) p.lse[row] = 0.f;
    return;
  }
  constexpr float kLog2e = 1.4426950408889634f;
  float mx = -INFINITY;
  for (int s = 0; s < p.splits; ++s) mx = fmaxf(mx, p.part_lse[s * p.part_rows + row]);
  float sum = 0.f;
  for (int s = 0; s < p.splits; ++s) sum += __builtin_amdgcn_exp2f((p.part_lse[s * p.part_rows + row] - mx) * kLog2e);
  const float lse = mx + __builtin_amdgcn_logf(sum) * 0.69314718055994530942f;
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  for (int s = 0; s < p.splits; ++s) {
    const float wgt = __builtin_amdgcn_exp2f((p.part_lse[s * p.part_rows + row] - lse) * kLog2e);
    const float* po = p.part_o + (s * p.part_rows + row) * DV + CPL * lane;
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = fmaf(wgt, po[c], acc[c]);
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) orow[c] = (T)acc[c];
  if (lane == 0) p.lse[row] = lse;
}

template <typename T, int DH, int DV, bool SPLIT>
static int launch_fwd_t(const KernelParams& p, void* stream) {
  using C = FwdCfg<T, DH, DV>;
  const int64_t units = p.xcd_map ? ((p.groups + 7) / 8) * 8 : p.groups;
  const int64_t grid = units * p.per_group;
  if (grid <= 0) return (int)hipSuccess;
  if constexpr (!SPLIT) {
    if (p.rope & kRopeQ) {
      hipLaunchKernelGGL((fwd_kernel<T, DH, DV, false, true>), dim3((unsigned)grid), dim3(64 * C::NW), 0,
                         (hipStream_t)stream, p);
      return (int)hipGetLastError();
    }
  }
  hipLaunchKernelGGL((fwd_kernel<T, DH, DV, SPLIT, false>), dim3((unsigned)grid), dim3(64 * C::NW), 0,
                     (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

int fwd_block_rows(int /*dtype*/) { return 128; }

template <bool SPLIT>
static int launch_fwd_any(const KernelParams& p, int dtype, int d_h, int d_v, void* stream) {
  if (dtype == ATTN_BF16) {
    if (d_h == 128 && d_v == 128) return launch_fwd_t<__bf16, 128, 128, SPLIT>(p, stream);
    if (d_h == 128 && d_v == 64) return launch_fwd_t<__bf16, 128, 64, SPLIT>(p, stream);
    if (d_h == 64 && d_v == 64) return launch_fwd_t<__bf16, 64, 64, SPLIT>(p, stream);
    if (d_h == 64 && d_v == 128) return launch_fwd_t<__bf16, 64, 128, SPLIT>(p, stream);
  } else {
    if (d_h == 128 && d_v == 128) return launch_fwd_t<float, 128, 128, SPLIT>(p, stream);
    if (d_h == 128 && d_v == 64) return launch_fwd_t<float, 128, 64, SPLIT>(p, stream);
    if (d_h == 64 && d_v == 64) return launch_fwd_t<float, 64, 64, SPLIT>(p, stream);
    if (d_h == 64 && d_v == 128) return launch_fwd_t<float, 64, 128, SPLIT>(p, stream);
  }
  return (int)hipErrorInvalidValue;
}

int launch_fwd(const KernelParams& p, int dtype, int d_h, int d_v, void* stream) {
  return launch_fwd_any<false>(p, dtype, d_h, d_v, stream);
}

int launch_fwd_split(const KernelParams& p, int dtype, int d_h, int d_v, void* stream) {
  return launch_fwd_any<true>(p, dtype, d_h, d_v, stream);
}

int launch_fwd_combine(const KernelParams& p, int dtype, int d_v, void* stream) {
  const dim3 grid((unsigned)((p.n_q + 3) / 4), (unsigned)p.H_q, (unsigned)p.B);
  if (p.n_q <= 0 || p.B <= 0) return (int)hipSuccess;
  if (dtype == ATTN_BF16) {
    if (d_v == 128) hipLaunchKernelGGL((fwd_combine_kernel<__bf16, 128>), grid, dim3(256), 0, (hipStream_t)stream, p);
    else if (d_v == 64) hipLaunchKernelGGL((fwd_combine_kernel<__bf16, 64>), grid, dim3(256), 0, (hipStream_t)stream, p);
    else return (int)hipErrorInvalidValue;
  } else {
    if (d_v == 128) hipLaunchKernelGGL((fwd_combine_kernel<float, 128>), grid, dim3(256), 0, (hipStream_t)stream, p);
    else if (d_v == 64) hipLaunchKernelGGL((fwd_combine_kernel<float, 64>), grid, dim3(256), 0, (hipStream_t)stream, p);
    else return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // namespace attn
