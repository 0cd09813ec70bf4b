// Backward with G_S kept (bf16): a per-row pass, then the dK/dV pass writing
// each step's G_S, then G_Q as one product over the kept G_S ("Appendix A.10 -
// Attention matrices and backpropagation", glenzli.com, eqs. A.10.7 and
// A.10.8: G_Q = G_S K / sqrt(d_h)).
//
// The two-pass backward forms G_S twice: the dK/dV pass for G_K and G_V, and
// the dQ pass again from S and dP for G_Q.  Here the dK/dV pass's XD waves
// also write the G_S they hand to YK, one 4 KB block per wave and step
// (2 bytes per (row, key) of each 32-row block against a 128-key block), and
// the dQ product reads each block once instead of recomputing S and dP.  -D
// and lse log2 e, which the dK/dV pass needs before it runs, come from the
// per-row pass first.
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {

constexpr int kRowsBM = 128;  // query rows per workgroup (4 waves of 32), as the dQ pass

// -D_i = -rowsum(G_O o O) and lse_i log2 e for every existing row, in the
// dQ pass's arithmetic (the lane's half of the row, then the other half's
// partial), indexed like lse.
template <typename T, int DV>
__global__ __launch_bounds__(256) void bwd_rows_kernel(const KernelParams p) {
  using op_t = typename Op<T>::type;
  const int nqblk = (p.n_q + kRowsBM - 1) / kRowsBM;
  int unit, item;
  if (!map_work(blockIdx.x, p.groups, p.per_group, p.xcd_map, unit, item)) return;
  const int b = unit / p.H_kv, g = unit - (unit / p.H_kv) * p.H_kv;
  const int qb = nqblk - 1 - item / p.group;
  const int r = g * p.group + item % p.group;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, kg = lane >> 5;
  const SeqView sv = seq_view(p, b);
  const int qi = qb * kRowsBM + 32 * w + (lane & 31);
  const bool row_exists = qi < sv.nq_lim, row_active = qi < sv.Lq;
  const T* Ob = (const T*)p.o + b * p.o_sb + sv.q_row0 * p.o_sr + r * p.o_sh;
  const T* dOb = (const T*)p.dout + b * p.o_sb + sv.q_row0 * p.o_sr + r * p.o_sh;
  const int64_t rowbase = b * p.lse_sb + r * p.lse_sh + sv.q_row0;
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
  if (row_exists && kg == 0) {
    p.delta[rowbase + qi] = -Di;
    p.lse2[rowbase + qi] = lse2;
  }
}

// G_Q^T += K^T G_S^T over 64-key tiles, one 32-row block per wave: the dQ
// pass's key-tile loop and G_Q products without S, dP and the exponentials.
// The dK/dV pass wrote each block of G_S as this product's four B operands
// (lane = query row, eight keys each; 1 KB per operand), so a wave loads
// them straight into registers.  Reading G_S from HBM bounds this pass
// (2 bytes per visible pair), so the K tile (through LDS) serves eight
// waves: the heads of the KV group side by side (hw = min(group, 8) of them,
// 32 * (8 / hw) positions each), which also gives the waves nearly the same
// key range.  K tiles and G_S operands run two tiles ahead.  A wave uses only tiles its rows see; the dK/dV pass
// wrote each such block (its key block's query range starts at or before
// the wave's rows), and invisible pairs inside them hold exact zeros.
template <int DH>
__global__ __launch_bounds__(512, 1) void bwd_dq_gs_kernel(const KernelParams p) {
  using T = __bf16;
  using op_t = bf16x8;
  constexpr int BN = 64, PF = 3;  // keys per tile; tile stages
  __shared__ __attribute__((aligned(16))) T k_lds0[BN * DH];
  __shared__ __attribute__((aligned(16))) T k_lds1[BN * DH];
  __shared__ __attribute__((aligned(16))) T k_lds2[BN * DH];

  // hw heads side by side, spw 32-row position blocks each (waves past
  // hw * spw idle when hw does not divide 8)
  const int hw = min(p.group, 8), spw = 8 / hw, pb = 32 * spw;
  const int npblk = (p.n_q + pb - 1) / pb;
  int unit, item;
  if (!map_work(blockIdx.x, p.groups, p.per_group, p.xcd_map, unit, item)) return;
  const int b = unit / p.H_kv, g = unit - (unit / p.H_kv) * p.H_kv;
  const int pblk = npblk - 1 - item % npblk, hblk = item / npblk;  // the heaviest position blocks first
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, kg = lane >> 5;
  const int rr = hblk * hw + w % hw, r = g * p.group + rr;
  const bool head_ok = w < hw * spw && rr < p.group;
  const SeqView sv = seq_view(p, b);
  const int Lq = sv.Lq, Lk = sv.Lk, off = sv.off;
  const int p_lo = pblk * pb;
  const int w_lo = p_lo + 32 * (w / hw);
  const int qi = w_lo + (lane & 31);
  const bool row_exists = head_ok && qi < sv.nq_lim, row_active = head_ok && qi < Lq;
  const T* Kb = (const T*)p.k + b * p.k_sb + sv.k_row0 * p.k_sr + g * p.k_sh;
  T* dQb = (T*)p.dq + b * p.dq_sb + sv.q_row0 * p.dq_sr + (head_ok ? r : 0) * p.dq_sh;

  const int act_hi = min(p_lo + pb, Lq);
  const int ntiles = act_hi > p_lo ? (key_limit_b(act_hi - 1, Lk, p.causal, off) + BN - 1) / BN : 0;
  const int w_hi = min(w_lo + 32, Lq);
  const int wtiles = head_ok && w_hi > w_lo ? (key_limit_b(w_hi - 1, Lk, p.causal, off) + BN - 1) / BN : 0;

  f32x16 acc[DH / 32];
#pragma unroll
  for (int i = 0; i < DH / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;

  if (ntiles > 0) {
    TrOffsets<T, DH> kto;
    kto.init(lane);
    // this wave's blocks (tile-major, 4 KB each): tile t's lies g_step
    // bytes after tile t - 1's, and the workgroup's waves read adjacent ones
    const size_t g_step = (size_t)p.gs_nqb * p.group * 4096;
    const char* gsw = reinterpret_cast<const char*>(p.gs) +
                      ((size_t)(b * p.H_kv + g) * 2 * p.gs_nkb * p.gs_nqb + (size_t)(w_lo / 32)) * p.group * 4096 +
                      (size_t)(head_ok ? rr : 0) * 4096;
    // Every tile of the loop issues the same loads (the K-tile copies and
    // four G_S operand loads per lane), so each wait below is a fixed count: K rows
    // at or past L_k lie outside the K resource and read as zeros, and a G_S
    // block past the wave's tiles has an empty resource (zeros, no memory
    // access).  K row offsets fit 32 bits (checked on the host).
    using KL = TileLoad<T, BN, DH, 512>;
    const uint32_t k_srb = (uint32_t)(p.k_sr * (int64_t)sizeof(T));
    const __amdgpu_buffer_rsrc_t k_rs =
        buf_rsrc(Kb, Lk > 0 ? (uint32_t)(Lk - 1) * k_srb + (uint32_t)(DH * sizeof(T)) : 0u);
    uint32_t k_off[KL::N];
    KL::lane_offsets(p.k_sr, tid, k_off);
    auto kbuf = [&](auto I) __attribute__((always_inline)) -> T* {
      if constexpr (decltype(I)::value == 0) return k_lds0;
      else if constexpr (decltype(I)::value == 1) return k_lds1;
      else return k_lds2;
    };
    // G_S is read once: non-temporal loads (cache-policy bit 1, "nt" on
    // gfx950) keep it from displacing the K tiles the next items reuse
    // (measured: the pass 0.574 -> 0.533 ms, same box)
    constexpr int kNonTemporal = 2;
    op_t gr[PF][4];
    auto issue = [&](int t, auto I, auto LOADG) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      KL::issue_buf_full(k_rs, (uint32_t)(t * BN) * k_srb, k_off, kbuf(I), tid);
      if constexpr (decltype(LOADG)::value) {
        const __amdgpu_buffer_rsrc_t g_rs = buf_rsrc(gsw + (size_t)t * g_step, t < wtiles ? 4096u : 0u);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          gr[i][e] = __builtin_bit_cast(op_t, __builtin_amdgcn_raw_buffer_load_b128(g_rs, lane * 16 + e * 1024, 0, kNonTemporal));
      }
    };
    // Tile t issues tile t + 2's loads into the stage tile t - 1 used (free
    // since the last barrier), multiplies tile t, then waits for everything
    // but tile t + 2's loads.  The last round's steps load no G_S (nothing
    // would read it: the compiler would drop such loads and the fixed count
    // would then no longer cover tile t + 1), so they wait for all but the
    // K copies of tile t + 2.
    auto step = [&](int t, auto I, auto TAIL) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      constexpr bool tail = decltype(TAIL)::value;
      issue(t + 2, IC<(i + 2) % PF>(), IC<!tail>());
      if (t < wtiles) {
#pragma unroll
        for (int mt = 0; mt < BN / 32; ++mt)
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int dt = 0; dt < DH / 32; ++dt) mma(acc[dt], kto.read(kbuf(I), 32 * mt + 16 * st, dt), gr[i][mt * 2 + st]);
      }
      stage_barrier<tail ? KL::N : KL::N + 4>();
    };
    issue(0, IC<0>(), IC<1>());
    issue(1, IC<1>(), IC<1>());
    stage_barrier<KL::N + 4>();
    // Whole rounds of three tiles in the loop and the rest after it: an exit
    // from inside the loop body would reach the loop head on the compiler's
    // paths with the latest G_S stage still in flight, and it would then wait
    // for that stage at the head.
    int t = 0;
    for (; t + 3 <= ntiles; t += 3) {
      step(t, IC<0>(), IC<0>());
      step(t + 1, IC<1>(), IC<0>());
      step(t + 2, IC<2>(), IC<0>());
    }
    if (t < ntiles) {
      step(t, IC<0>(), IC<1>());
      if (t + 1 < ntiles) step(t + 1, IC<1>(), IC<1>());
    }
    // no copy may still be writing LDS when the workgroup ends
    wait_tile_loads();
  }
  if (row_exists) {
    const float sc = row_active ? p.scale : 0.f;
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * dt + 8 * j + 4 * kg;
        st4<T>(dQb + (int64_t)qi * p.dq_sr + d, acc[dt][4 * j] * sc, acc[dt][4 * j + 1] * sc,
               acc[dt][4 * j + 2] * sc, acc[dt][4 * j + 3] * sc);
      }
  }
}

int bwd_gs_block_rows() { return kRowsBM; }

int64_t bwd_dq_gs_items(int n_q, int group) {
  const int hw = group < 8 ? group : 8, pb = 32 * (8 / hw);
  return (int64_t)((n_q + pb - 1) / pb) * ((group + hw - 1) / hw);
}

int launch_bwd_rows(const KernelParams& p, int d_v, void* stream) {
  const int64_t units = p.xcd_map ? ((p.groups + 7) / 8) * 8 : p.groups;
  const int64_t grid = units * p.per_group;
  if (grid <= 0) return (int)hipSuccess;
  if (d_v == 128)
    hipLaunchKernelGGL((bwd_rows_kernel<__bf16, 128>), dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, p);
  else if (d_v == 64)
    hipLaunchKernelGGL((bwd_rows_kernel<__bf16, 64>), dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, p);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int launch_bwd_dq_gs(const KernelParams& p, int d_h, void* stream) {
  const int64_t units = p.xcd_map ? ((p.groups + 7) / 8) * 8 : p.groups;
  const int64_t grid = units * p.per_group;
  if (grid <= 0) return (int)hipSuccess;
  if (d_h == 128)
    hipLaunchKernelGGL((bwd_dq_gs_kernel<128>), dim3((unsigned)grid), dim3(512), 0, (hipStream_t)stream, p);
  else if (d_h == 64)
    hipLaunchKernelGGL((bwd_dq_gs_kernel<64>), dim3((unsigned)grid), dim3(512), 0, (hipStream_t)stream, p);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // namespace attn
