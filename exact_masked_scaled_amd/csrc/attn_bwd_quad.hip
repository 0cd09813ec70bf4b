// dK/dV pass, bf16: the four-role kernel ("Appendix A.10 - Attention
// matrices and backpropagation", glenzli.com, eqs. A.10.5, A.10.6, A.10.7 and
// A.10.9, and sec. A.10.5 for grouped heads).
//
// Key-stationary like the float32 dK/dV kernel: one workgroup owns 128 keys of
// one (sequence, KV head), keeps their K and V rows in registers and their
// G_K, G_V accumulators, and walks every query head of the group and every
// block of 32 query rows that sees its keys:
//   S = Q K^T, P = exp(S - lse), dP = G_O V^T, G_S = P o (dP - D)
//   G_V += P^T G_O                                (eq. A.10.5)
//   G_K += G_S^T Q / sqrt(d_h)                    (eq. A.10.9)
// Keys at or beyond L_k[b] and rows at or beyond L_q[b] get P = 0 and G_S = 0,
// so padded keys receive exactly zero G_K / G_V.  D (from the dQ pass) is the
// row scalar of eq. A.10.7.
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {

// ============================================================== dK/dV pass, four roles (bf16)
// Same work unit as bwd_dkdv_kernel (128 keys of one sequence and KV head,
// every query head of the group, 32-row query steps).  Each of the four
// products of a step has its own wave per 64-key half, so every wave keeps a
// 64-key operand or accumulator in registers and each LDS operand read feeds
// two matrix products (half the LDS reads of 32-key waves):
//   XS (waves 0, 1): holds K; S = Q K^T, then P = exp(S - lse) on the visible
//       set, handed on as bf16 MFMA operands;
//   XD (waves 2, 3): holds V; dP = G_O V^T, then G_S = P o (dP - D), handed on;
//   YV (waves 4, 5): G_V += P^T G_O;     YK (waves 6, 7): G_K += G_S^T Q,
//       both accumulated as their transposes (a lane holds one key's columns).
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
// ROPE: G_K is turned back in the stores (rotary positions).
// BUF: Q / G_O blocks of 32 rows span less than 4 GiB, so the ring copies are
// buffer loads from one resource per block (below).  Separate instances keep
// the other paths' registers out of each kernel.
template <typename T, int DH, int DV, bool HSPLIT, bool ROPE, bool BUF, bool GS>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_quad_kernel(const KernelParams p) {
  static_assert(sizeof(T) == 2, "four-role dK/dV pass is the bf16 path");
  using C = DkvQuadCfg<T, DH, DV>;
  using op_t = typename Op<T>::type;
  using gop_t = __attribute__((address_space(1))) op_t;
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
        // keys past L_k read the last key's row (L_k > 0 here) and take
        // zeros: the loads need no branch, so they are all in flight at once
        const int key = kh0 + 32 * kb2 + (lane & 31);
        const bool ok = key < Lk;
        const T* row = src + (int64_t)min(key, Lk - 1) * sr + 8 * kg;
        constexpr int NK = (DH > DV ? DH : DV) / 16;
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          if (ks >= nks) continue;
          op_t v = ld8<T>(row + 16 * ks);
          if (!ok) v = zero_op<T>();
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
    // the step's rows: lse log2 e (lanes 0-31) and -D (lanes 32-63), from the dQ pass
    const float* const rows_lane = (lane < 32 ? p.lse2 : p.delta) + b * p.lse_sb + sv.q_row0 + (lane & 31);
    const int yw = w & 3;  // copy slot of a Y wave
    // Copy instruction i of a Y wave moves job yw + 4 i of the step's 64-lane
    // jobs (Q chunks first, then G_O; i < QCH / 256 a Q chunk since yw < 4).
    //   BUF: one buffer resource per block, from its first row to the end of
    //   its last active row (rows past it read as zeros), and a lane byte
    //   offset fixed for the kernel;
    //   otherwise 64-bit addresses: a lane offset (elements) fixed for the
    //   kernel, and rows past the last active one repeating it by selecting
    //   a precomputed chunk of that row.
    // Either way exactly CPS copies per step on every path.
    static_assert(C::QCH % 256 == 0 && C::OCH % 256 == 0, "each Y wave copies whole Q and G_O wave rows");
    auto job_row = [&](int i) __attribute__((always_inline)) -> int {
      const int job = yw + 4 * i;
      return i < C::QCH / 256 ? (job * 64 + lane) / Tile<T, DH>::CH
                              : ((job - C::QCH / 64) * 64 + lane) / Tile<T, DV>::CH;
    };
    auto job_col = [&](int i) __attribute__((always_inline)) -> int {  // swizzled element column
      const int job = yw + 4 * i;
      if (i < C::QCH / 256) {
        using L = Tile<T, DH>;
        const int pc = job * 64 + lane;
        return ((pc % L::CH) ^ L::f(pc / L::CH)) * L::EPC;
      } else {
        using L = Tile<T, DV>;
        const int pc = (job - C::QCH / 64) * 64 + lane;
        return ((pc % L::CH) ^ L::f(pc / L::CH)) * L::EPC;
      }
    };
    auto job_dst = [&](int i, auto ST) __attribute__((always_inline)) -> T* {
      const int job = yw + 4 * i;
      return i < C::QCH / 256 ? q_st(ST) + job * 64 * Tile<T, DH>::EPC
                              : o_st(ST) + (job - C::QCH / 64) * 64 * Tile<T, DV>::EPC;
    };
    const uint32_t q_srb = (uint32_t)(q_sr * (int64_t)sizeof(T)), o_srb = (uint32_t)(o_sr * (int64_t)sizeof(T));
    uint32_t c_voff[C::JPW];   // BUF
    int64_t c_off[C::JPW];     // otherwise
#pragma unroll
    for (int i = 0; i < C::JPW; ++i) {
      if constexpr (BUF)
        c_voff[i] = (uint32_t)job_row(i) * (i < C::QCH / 256 ? q_srb : o_srb) + (uint32_t)(job_col(i) * (int)sizeof(T));
      else
        c_off[i] = job_row(i) * (i < C::QCH / 256 ? q_sr : o_sr) + job_col(i);
    }
    auto issue = [&](int rr, int qb, auto ST) __attribute__((always_inline)) {
      const int r = g * group + rr;
      const int q0 = qb * C::BM;
      const T* qt = q_base + r * q_sh + (int64_t)q0 * q_sr;
      const T* ot = o_base + r * o_sh + (int64_t)q0 * o_sr;
      const int last = min(n_q - q0, C::BM) - 1;  // last active row of the block
      if constexpr (BUF) {
        const auto rq = buf_rsrc(qt, (uint32_t)(last + 1) * q_srb);
        const auto ro = buf_rsrc(ot, (uint32_t)(last + 1) * o_srb);
#pragma unroll
        for (int i = 0; i < C::JPW; ++i) buf_copy16(i < C::QCH / 256 ? rq : ro, job_dst(i, ST), c_voff[i], 0u);
      } else {
        const int64_t last_q = (int64_t)last * q_sr, last_o = (int64_t)last * o_sr;
#pragma unroll
        for (int i = 0; i < C::JPW; ++i) {
          const bool isq = i < C::QCH / 256;
          const int64_t off = job_row(i) <= last ? c_off[i] : (isq ? last_q : last_o) + job_col(i);
          __builtin_amdgcn_global_load_lds((const void*)((isq ? qt : ot) + off), (ATTN_LDS void*)job_dst(i, ST), 16, 0,
                                           0);
        }
      }
      // every Y wave copies the same lse / D rows (keeps the per-wave count
      // equal); rows past the last active one repeat it
      const int qq = q0 + min(lane & 31, last) - (lane & 31);
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
      // the rows up front
      f32x4 l4v[4];
      if constexpr (ex) {
#pragma unroll
        for (int j = 0; j < 4; ++j) l4v[j] = *reinterpret_cast<const f32x4*>(&rows[8 * j + 4 * kg]);
      }
      constexpr int PF = 2;  // operand reads run PF k-steps ahead of their products
      op_t qa[PF + 1];
      if constexpr (mf) {
#pragma unroll
        for (int j = 0; j < PF; ++j) qa[j] = row_op(Qs, ofs[j]);
      }
      op_t* xo = xb + (h * 2) * 2 * 64;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (mf) {
          const op_t a = qa[ks % (PF + 1)];
          if (ks + PF < KS) qa[(ks + PF) % (PF + 1)] = row_op(Qs, ofs[ks + PF]);
          mma(s0, a, op_part(R[ks / 4], ks % 4));
          mma(s1, a, op_part(R[(DH / 16 + ks) / 4], (DH / 16 + ks) % 4));
        }
        if constexpr (ex) {
#pragma unroll
          for (int e = EPK * ks; e < EPK * (ks + 1); ++e) {
            const float lse2 = l4v[e >> 2][e & 3];
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
    auto xd_iter = [&](auto MF, auto EX, auto J, const T* Os, const float* rows, const op_t* xpb, op_t* xb, gop_t* gsb) __attribute__((always_inline)) {
      constexpr bool mf = decltype(MF)::value, ex = decltype(EX)::value;
      constexpr int jn = decltype(J)::value, jo = jn ^ 1;
      f32x16& d0 = R[XB + 2 * jn];
      f32x16& d1 = R[XB + 2 * jn + 1];
      f32x16& o0 = R[XB + 2 * jo];
      f32x16& o1 = R[XB + 2 * jo + 1];
      if constexpr (mf) {
        // the dP chains start from -D of their rows (rows: the dP step's), so
        // they end at dP - D
        f32x16 nd;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(&rows[C::BM + 8 * j + 4 * kg]);
#pragma unroll
          for (int e = 0; e < 4; ++e) nd[4 * j + e] = v[e];
        }
        d0 = nd;
        d1 = nd;
      }
      constexpr int KS = DV / 16;
      constexpr int EPK = 16 / KS;
      const op_t* pin = xpb + (h * 2) * 2 * 64;
      op_t* xo = xb + (h * 2) * 2 * 64;
      // P up front
      op_t pp[2][2];
      if constexpr (ex) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int st = 0; st < 2; ++st) pp[kb2][st] = pin[(kb2 * 2 + st) * 64 + lane];
      }
      constexpr int PF = 2;  // operand reads run PF k-steps ahead of their products
      op_t oa[PF + 1];
      if constexpr (mf) {
#pragma unroll
        for (int j = 0; j < PF; ++j) oa[j] = row_op(Os, ofs[j]);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (mf) {
          const op_t a = oa[ks % (PF + 1)];
          if (ks + PF < KS) oa[(ks + PF) % (PF + 1)] = row_op(Os, ofs[ks + PF]);
          mma(d0, a, op_part(R[ks / 4], ks % 4));
          mma(d1, a, op_part(R[(DV / 16 + ks) / 4], (DV / 16 + ks) % 4));
        }
        if constexpr (ex) {
#pragma unroll
          for (int e = EPK * ks; e < EPK * (ks + 1); ++e) {
            o0[e] = (float)pp[0][e >> 3][e & 7] * o0[e];
            o1[e] = (float)pp[1][e >> 3][e & 7] * o1[e];
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
      if constexpr (GS && ex) {
        // G_S kept for the dQ product: the block just handed on, read back
        // transposed (lane = query row, eight keys per operand) and written
        // as the product's four B operands, 16 bytes per lane each, with
        // non-temporal stores (written once, read once by the next kernel:
        // the pass 1.377 -> 1.344 ms, same box)
        const __bf16* blk = reinterpret_cast<const __bf16*>(xo);
        const int goff = gs_lane_offset(lane);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int st = 0; st < 2; ++st)
            __builtin_nontemporal_store(gs_read(blk, mt * 2048 + st * 256 + goff), &gsb[(mt * 2 + st) * 64 + lane]);
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
            mma(R[nt], bt, a[0][st]);
            mma(R[NT + nt], bt, a[1][st]);
          }
      };
      // YV: G_V^T += G_O^T P; YK: G_K^T += Q^T G_S (the transposed tile
      // operand as A, the exchanged one as B, so a lane accumulates one key's
      // columns and stores them four at a time).  With d_h = d_v one path, so
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
          mma(R[nt], ybt[st][nt], a[0][st]);
          mma(R[NT + nt], ybt[st][nt], a[1][st]);
        }
      y_load(IC<u + 1>());
    };

    int i_rr = rr_lo, i_qb = qb_first;   // next step to copy
    int xs_qb = qb_first;            // query block of the step XS exponentiates next
    // G_S kept: the step XD forms G_S of next, and this (sequence, KV head,
    // key block, half)'s blocks (one per query head and 32-row block)
    int xd_rr = rr_lo, xd_qb = qb_first;
    gop_t* const gs_kh =
        GS ? (gop_t*)p.gs + ((size_t)(b * p.H_kv + g) * 2 * p.gs_nkb + 2 * kb + h) * p.gs_nqb * p.group * 256
           : nullptr;
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
        // with G_S kept, XD's barrier leaves its block stores in flight (it
        // issues no other memory access in the loop)
        stage_barrier<GS ? 63 : 0>();
        // XD: dP(s - 1) into parity (s - 1) & 1, G_S(s - 2) -> G_S slot 3 + (s - 2) % 2
        constexpr int jd = (u + 1) & 1;
        const T* Os = o_st(IC<u + NS - 1>());
        const float* rows = r_st(IC<u + NS - 1>());  // -D of step s - 1
        const op_t* pin = xch + ((u + 1) % 3) * XSLOT;  // P(s - 2)
        op_t* xw = xch + (3 + (u & 1)) * XSLOT;         // G_S(s - 2)
        const bool mf = !ramp || (s >= 1 && s <= nsteps), ex = !ramp || (s >= 2 && s <= nsteps + 1);
        gop_t* gsb = nullptr;
        if constexpr (GS) gsb = gs_kh + ((size_t)xd_qb * p.group + xd_rr) * 256;
        if (mf && ex) xd_iter(TR(), TR(), IC<jd>(), Os, rows, pin, xw, gsb);
        else if constexpr (ramp) {
          if (ex) xd_iter(F(), TR(), IC<jd>(), Os, rows, pin, xw, gsb);
          else if (mf) xd_iter(TR(), F(), IC<jd>(), Os, rows, pin, xw, gsb);
        }
        if constexpr (GS) {
          if (ex) { if (++xd_qb == qb_end) { xd_qb = qb_first; ++xd_rr; } }
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

  // store: YV holds G_V, YK G_K (scaled) of both key blocks, transposed:
  // block kb2 * NT + nt of a lane holds key kh0 + 32 kb2 + lane % 32, element
  // e column 32 nt + 8 (e / 4) + 4 kg + e % 4, so four consecutive columns go
  // out in one store
  auto store = [&](auto NTC, auto TURN, T* dst, int64_t sr, float sc) __attribute__((always_inline)) {
    constexpr int NT = decltype(NTC)::value;
    constexpr bool turn = decltype(TURN)::value;
    constexpr int NBLK = 2 * NT;  // blocks i = (kb2, nt)
    // rotary positions: G_K = R^T G_K~, key kk at position kk; a lane's four
    // columns are two pairs, whose (cos, sin) entries are one 16-byte read.
    // A block's entries are read TD blocks ahead of its stores, clamped into
    // the valid keys (whose rows exist), and pinned by an empty asm where they
    // are used, so the compiler cannot sink the loads into the guarded stores;
    // keys past L_k keep their exact zeros.
    constexpr int TD = 2;
    f32x4 t[TD + 1][4];
    auto load = [&](int i) __attribute__((always_inline)) {
      const int kc = max(min(kh0 + 32 * (i / NT) + (lane & 31), Lk - 1), 0);
      const float* row = p.rope_cs + (int64_t)kc * DH + 32 * (i % NT) + 4 * kg;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) t[i % (TD + 1)][q4] = *reinterpret_cast<const f32x4*>(row + 8 * q4);
    };
    if constexpr (turn) {
#pragma unroll
      for (int i = 0; i < TD; ++i) load(i);
    }
#pragma unroll
    for (int i = 0; i < NBLK; ++i) {
      const int kb2 = i / NT, nt = i % NT;
      const int kk = kh0 + 32 * kb2 + (lane & 31);
      if constexpr (turn) {
        if (i + TD < NBLK) load(i + TD);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) asm volatile("" : "+v"(t[i % (TD + 1)][q4]));
      }
      if (kk < nk_lim) {
        T* out = dst + (int64_t)kk * sr + 32 * nt + 4 * kg;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = R[kb2 * NT + nt][4 * q4 + e] * sc;
          if constexpr (turn) {
            if (kk < Lk) {
              const f32x4 c = t[i % (TD + 1)][q4];
              rope_pair(c[0], -c[1], v[0], v[1]);
              rope_pair(c[2], -c[3], v[2], v[3]);
            }
          }
          ::attn::st4<T>(out + 8 * q4, v[0], v[1], v[2], v[3]);
        }
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
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const int kk = kh0 + 32 * kb2 + (lane & 31);
          if (kk < nk_lim) {
            float* out = base + ((int64_t)hs * p.part_krows + krow + kk) * D + 4 * kg;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4) {
                const f32x16& r = R[kb2 * NT + nt];
                ::attn::st4<float>(out + 32 * nt + 8 * q4, r[4 * q4] * sc, r[4 * q4 + 1] * sc, r[4 * q4 + 2] * sc,
                           r[4 * q4 + 3] * sc);
              }
          }
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

template <typename T, int DH, int DV, bool BUF>
static void launch_quad(const KernelParams& p, int64_t grid, void* stream) {
  if (p.hsplits > 1)
    hipLaunchKernelGGL((bwd_dkdv_quad_kernel<T, DH, DV, true, false, BUF, false>), dim3((unsigned)grid), dim3(512), 0,
                       (hipStream_t)stream, p);
  else if (p.rope & kRopeDK)
    hipLaunchKernelGGL((bwd_dkdv_quad_kernel<T, DH, DV, false, true, BUF, false>), dim3((unsigned)grid), dim3(512), 0,
                       (hipStream_t)stream, p);
  else if (p.gs != nullptr)
    hipLaunchKernelGGL((bwd_dkdv_quad_kernel<T, DH, DV, false, false, BUF, true>), dim3((unsigned)grid), dim3(512), 0,
                       (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL((bwd_dkdv_quad_kernel<T, DH, DV, false, false, BUF, false>), dim3((unsigned)grid), dim3(512), 0,
                       (hipStream_t)stream, p);
}

template <typename T, int DH, int DV>
static int launch_quad_t(const KernelParams& p, void* stream) {
  const int64_t units = p.xcd_map ? ((p.groups + 7) / 8) * 8 : p.groups;
  const int64_t grid = units * p.per_group;
  if (grid <= 0) return (int)hipSuccess;
  // buffer copies when a 32-row block of Q and of G_O spans less than 4 GiB
  constexpr int64_t kBlock = 32 * (int64_t)sizeof(T);
  if (p.q_sr >= 0 && p.o_sr >= 0 && p.q_sr * kBlock <= 0xffffffffLL && p.o_sr * kBlock <= 0xffffffffLL)
    launch_quad<T, DH, DV, true>(p, grid, stream);
  else
    launch_quad<T, DH, DV, false>(p, grid, stream);
  return (int)hipGetLastError();
}

int launch_bwd_dkdv_quad(const KernelParams& p, int d_h, int d_v, void* stream) {
  if (d_h == 128 && d_v == 128) return launch_quad_t<__bf16, 128, 128>(p, stream);
  if (d_h == 128 && d_v == 64) return launch_quad_t<__bf16, 128, 64>(p, stream);
  if (d_h == 64 && d_v == 64) return launch_quad_t<__bf16, 64, 64>(p, stream);
  if (d_h == 64 && d_v == 128) return launch_quad_t<__bf16, 64, 128>(p, stream);
  return (int)hipErrorInvalidValue;
}

}  // namespace attn
