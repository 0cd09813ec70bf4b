// Backward kernels ("Appendix A.10 - Attention matrices and backpropagation",
// glenzli.com, eqs. A.10.5-A.10.9 and sec. A.10.5 for grouped heads):
//
//   bwd_pre   D_i = sum_l G_O[i,l] O[i,l]  (equals the row scalar c_i of
//             eq. A.10.7, because c_i = sum_j A_ij sum_l G_O[i,l] V[j,l]);
//             also clears the float32 G_Q accumulator.
//   bwd_main  one workgroup per (sequence, KV head, block of 128 keys); a wave
//             owns 32 keys and keeps K, V of its keys in registers and
//             G_K, G_V accumulators for them.  It walks every query head that
//             shares the KV head and every block of query rows that can see
//             its keys, recomputing P = exp(S - lse) from the forward's
//             logsumexp (no n_q x n_k state is ever stored), then
//               G_V += P^T G_O                               (eq. A.10.5)
//               dP   = G_O V^T                               (eq. A.10.6)
//               G_S  = P o (dP - D)                          (eq. A.10.7)
//               G_K += G_S^T Q / sqrt(d_h)                   (eq. A.10.9)
//               G_Q += G_S K / sqrt(d_h)  (float32 atomics)  (eq. A.10.8)
//             The score tile is computed as S = Q K^T so that a lane owns one
//             key: P and G_S are then directly the A operands of the G_V and
//             G_K products.  G_Q needs G_S with a lane per query, so G_S goes
//             through LDS once and is read back transposed.
//   bwd_dq    converts the G_Q accumulator to the I/O dtype.
// Keys at or beyond L_k[b] and rows at or beyond L_q[b] get P = 0 and G_S = 0,
// so padded keys receive exactly zero G_K / G_V.
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {

// ============================================================== preprocess
// 16 threads per row, 16 rows per 256-thread block.
template <typename T, int DH, int DV>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const KernelParams p) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const int64_t rows = (int64_t)p.B * p.H_q * p.n_q;
  if (row >= rows) return;
  const int i = (int)(row % p.n_q);
  const int64_t bh = row / p.n_q;
  const int r = (int)(bh % p.H_q);
  const int b = (int)(bh / p.H_q);
  const int Lq = p.has_lens ? p.lens_q[b] : p.n_q;
  constexpr int EV = DV / 16;  // elements per thread
  const T* o = (const T*)p.o + b * p.o_sb + r * p.o_sh + (int64_t)i * p.o_sr + sub * EV;
  const T* go = (const T*)p.dout + b * p.o_sb + r * p.o_sh + (int64_t)i * p.o_sr + sub * EV;
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < EV; ++e) acc += (float)o[e] * (float)go[e];
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (sub == 0) p.delta[row] = i < Lq ? acc : 0.f;
  // clear this row of the G_Q accumulator
  float* dq = p.dq_acc + row * DH + sub * (DH / 16);
#pragma unroll
  for (int e = 0; e < DH / 16; e += 4) *reinterpret_cast<f32x4*>(dq + e) = f32x4{0.f, 0.f, 0.f, 0.f};
}

// ============================================================== main
template <typename T, int DH, int DV>
struct BwdCfg {
  static constexpr int NW = 4;                          // waves per workgroup
  static constexpr int BN = 32 * NW;                    // keys per workgroup
  static constexpr int BM = sizeof(T) == 2 ? 64 : 32;   // query rows per step
  static constexpr int PAD = 32 / (int)sizeof(T);
  static constexpr int KS = DH + PAD;                   // LDS stride of K and Q rows
  static constexpr int OS = DV + PAD;                   // LDS stride of G_O rows
  static constexpr int SS = BM + PAD;                   // LDS stride of G_S^T rows
  static constexpr int CH_H = DH * (int)sizeof(T) / 16;
  static constexpr int CH_V = DV * (int)sizeof(T) / 16;
};

template <typename T, int DH, int DV>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(const KernelParams p) {
  using C = BwdCfg<T, DH, DV>;
  using op_t = typename Op<T>::type;
  __shared__ __attribute__((aligned(16))) T k_lds[C::BN * C::KS];
  __shared__ __attribute__((aligned(16))) T q_lds[C::BM * C::KS];
  __shared__ __attribute__((aligned(16))) T do_lds[C::BM * C::OS];
  __shared__ __attribute__((aligned(16))) T ds_lds[C::BN * C::SS];
  __shared__ float lse_lds[C::BM];
  __shared__ float dlt_lds[C::BM];

  int unit, kb;
  if (!map_work(blockIdx.x, p.groups, p.per_group, p.xcd_map, unit, kb)) return;
  const int b = unit / p.H_kv, g = unit - (unit / p.H_kv) * p.H_kv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, kg = lane >> 5;
  const int Lq = p.has_lens ? p.lens_q[b] : p.n_q;
  const int Lk = p.has_lens ? p.lens_k[b] : p.n_k;
  const int k_lo = kb * C::BN;
  const int kw = k_lo + 32 * w + (lane & 31);          // this lane's key (S layout)

  const T* Kb = (const T*)p.k + b * p.k_sb + g * p.k_sh;
  const T* Vb = (const T*)p.v + b * p.v_sb + g * p.v_sh;
  T* dKb = (T*)p.dk + b * p.k_sb + g * p.k_sh;
  T* dVb = (T*)p.dv + b * p.v_sb + g * p.v_sh;

  f32x16 dk_acc[DH / 32], dv_acc[DV / 32];
#pragma unroll
  for (int i = 0; i < DH / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk_acc[i][e] = 0.f;
#pragma unroll
  for (int i = 0; i < DV / 32; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dv_acc[i][e] = 0.f;

  // first query row that sees any key of this block (causal: j <= i + off)
  const int q_first = p.causal ? max(0, k_lo - p.offset) : 0;
  const bool any_work = k_lo < Lk && q_first < Lq;

  if (any_work) {
    // K tile of the workgroup's keys -> LDS (operand of the G_Q product)
    for (int c = tid; c < C::BN * C::CH_H; c += 64 * C::NW) {
      const int row = c / C::CH_H, col = c % C::CH_H;
      const int key = k_lo + row;
      u32x4 v = key < p.n_k ? *reinterpret_cast<const u32x4*>(
                                  (const char*)(Kb + (int64_t)key * p.k_sr) + 16 * col)
                            : u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>((char*)(&k_lds[row * C::KS]) + 16 * col) = v;
    }
    // K and V of this lane's key as B operands of S = Q K^T and dP = G_O V^T
    op_t kreg[DH / 16], vreg[DV / 16];
    const bool key_exists = kw < p.n_k;
#pragma unroll
    for (int ks = 0; ks < DH / 16; ++ks)
      kreg[ks] = key_exists ? ld8<T>(Kb + (int64_t)kw * p.k_sr + 16 * ks + 8 * kg) : zero_op<T>();
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
      vreg[ks] = key_exists ? ld8<T>(Vb + (int64_t)kw * p.v_sr + 16 * ks + 8 * kg) : zero_op<T>();

    const int qb_first = q_first / C::BM;
    const int qb_end = (Lq + C::BM - 1) / C::BM;
    for (int rr = 0; rr < p.group; ++rr) {
      const int r = g * p.group + rr;
      const T* Qb = (const T*)p.q + b * p.q_sb + r * p.q_sh;
      const T* dOb = (const T*)p.dout + b * p.o_sb + r * p.o_sh;
      const float* lse_b = p.lse + ((int64_t)b * p.H_q + r) * p.n_q;
      const float* dlt_b = p.delta + ((int64_t)b * p.H_q + r) * p.n_q;
      float* dq_b = p.dq_acc + ((int64_t)b * p.H_q + r) * p.n_q * DH;

      for (int qb = qb_first; qb < qb_end; ++qb) {
        const int q0 = qb * C::BM;
        __syncthreads();  // previous step is done with q_lds / do_lds / ds_lds
        for (int c = tid; c < C::BM * C::CH_H; c += 64 * C::NW) {
          const int row = c / C::CH_H, col = c % C::CH_H;
          const int q = q0 + row;
          u32x4 v = q < p.n_q ? *reinterpret_cast<const u32x4*>(
                                    (const char*)(Qb + (int64_t)q * p.q_sr) + 16 * col)
                              : u32x4{0, 0, 0, 0};
          *reinterpret_cast<u32x4*>((char*)(&q_lds[row * C::KS]) + 16 * col) = v;
        }
        for (int c = tid; c < C::BM * C::CH_V; c += 64 * C::NW) {
          const int row = c / C::CH_V, col = c % C::CH_V;
          const int q = q0 + row;
          u32x4 v = q < p.n_q ? *reinterpret_cast<const u32x4*>(
                                    (const char*)(dOb + (int64_t)q * p.o_sr) + 16 * col)
                              : u32x4{0, 0, 0, 0};
          *reinterpret_cast<u32x4*>((char*)(&do_lds[row * C::OS]) + 16 * col) = v;
        }
        if (tid < C::BM) {
          const int q = q0 + tid;
          lse_lds[tid] = q < p.n_q ? lse_b[q] * 1.4426950408889634f : 0.f;
          dlt_lds[tid] = q < p.n_q ? dlt_b[q] : 0.f;
        }
        __syncthreads();

        // S = Q K^T and dP = G_O V^T for this wave's 32 keys (lane = key)
        f32x16 s[C::BM / 32], dp[C::BM / 32];
#pragma unroll
        for (int mt = 0; mt < C::BM / 32; ++mt) {
#pragma unroll
          for (int e = 0; e < 16; ++e) { s[mt][e] = 0.f; dp[mt][e] = 0.f; }
#pragma unroll
          for (int ks = 0; ks < DH / 16; ++ks)
            mma(s[mt], ld8<T>(q_lds + (32 * mt + (lane & 31)) * C::KS + 16 * ks + 8 * kg), kreg[ks]);
#pragma unroll
          for (int ks = 0; ks < DV / 16; ++ks)
            mma(dp[mt], ld8<T>(do_lds + (32 * mt + (lane & 31)) * C::OS + 16 * ks + 8 * kg), vreg[ks]);
        }
        // P = exp(S/sqrt(d) - lse) on the visible set, G_S = P o (dP - D)
        const bool full = (q0 + C::BM <= Lq) && (k_lo + C::BN <= Lk) &&
                          (!p.causal || k_lo + C::BN - 1 <= q0 + p.offset);
#pragma unroll
        for (int mt = 0; mt < C::BM / 32; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int ql = 32 * mt + 8 * (e >> 2) + 4 * kg + (e & 3);
            float pv = __builtin_amdgcn_exp2f(s[mt][e] * p.scale_log2 - lse_lds[ql]);
            if (!full) {
              const int q = q0 + ql;
              const bool vis = (kw < Lk) && (q < Lq) && (!p.causal || kw <= q + p.offset);
              pv = vis ? pv : 0.f;
            }
            s[mt][e] = pv;
            dp[mt][e] = pv * (dp[mt][e] - dlt_lds[ql]);
          }
        // G_V += P^T G_O and G_K += G_S^T Q (A = this lane's key row, C order over queries)
#pragma unroll
        for (int mt = 0; mt < C::BM / 32; ++mt)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            float tmp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) tmp[e] = s[mt][8 * st + e];
            const op_t pa = to_op<T>(tmp);
#pragma unroll
            for (int e = 0; e < 8; ++e) tmp[e] = dp[mt][8 * st + e];
            const op_t da = to_op<T>(tmp);
#pragma unroll
            for (int nt = 0; nt < DV / 32; ++nt)
              mma(dv_acc[nt], pa, ld_tr<T>(do_lds, C::OS, 32 * mt + 16 * st, 32 * nt));
#pragma unroll
            for (int nt = 0; nt < DH / 32; ++nt)
              mma(dk_acc[nt], da, ld_tr<T>(q_lds, C::KS, 32 * mt + 16 * st, 32 * nt));
          }
        // G_S^T -> LDS as [key][query] (4 consecutive queries per store)
#pragma unroll
        for (int mt = 0; mt < C::BM / 32; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            st4<T>(ds_lds + (32 * w + (lane & 31)) * C::SS + 32 * mt + 8 * j + 4 * kg,
                   dp[mt][4 * j], dp[mt][4 * j + 1], dp[mt][4 * j + 2], dp[mt][4 * j + 3]);
        __syncthreads();
        // G_Q tile(s) = G_S K over the workgroup's keys: A = G_S (lane = query),
        // B = K (lane = d), both transposed reads in C order over keys
        constexpr int QT = C::BM / 32, DT = DH / 32;
        for (int tile = w; tile < QT * DT; tile += C::NW) {
          const int qt = tile / DT, nt = tile % DT;
          f32x16 acc;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
          for (int ks = 0; ks < C::BN / 16; ++ks)
            mma(acc, ld_tr<T>(ds_lds, C::SS, 16 * ks, 32 * qt), ld_tr<T>(k_lds, C::KS, 16 * ks, 32 * nt));
          const int d = 32 * nt + (lane & 31);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int q = q0 + 32 * qt + 8 * (e >> 2) + 4 * kg + (e & 3);
            if (q < Lq) unsafeAtomicAdd(dq_b + (int64_t)q * DH + d, acc[e] * p.scale);
          }
        }
      }
    }
  }

  // store G_K (scaled) and G_V for this wave's keys; lane = d, registers = keys
  const int kbase = k_lo + 32 * w;
#pragma unroll
  for (int nt = 0; nt < DH / 32; ++nt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kbase + 8 * (e >> 2) + 4 * kg + (e & 3);
      if (key < p.n_k) dKb[(int64_t)key * p.k_sr + 32 * nt + (lane & 31)] = (T)(dk_acc[nt][e] * p.scale);
    }
#pragma unroll
  for (int nt = 0; nt < DV / 32; ++nt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kbase + 8 * (e >> 2) + 4 * kg + (e & 3);
      if (key < p.n_k) dVb[(int64_t)key * p.v_sr + 32 * nt + (lane & 31)] = (T)dv_acc[nt][e];
    }
}

// ============================================================== dQ convert
// 8 elements per thread.
template <typename T, int DH>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const KernelParams p) {
  constexpr int TPR = DH / 8;  // threads per row
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / TPR;
  const int sub = (int)(idx % TPR);
  const int64_t rows = (int64_t)p.B * p.H_q * p.n_q;
  if (row >= rows) return;
  const int i = (int)(row % p.n_q);
  const int64_t bh = row / p.n_q;
  const int r = (int)(bh % p.H_q);
  const int b = (int)(bh / p.H_q);
  const float* src = p.dq_acc + row * DH + sub * 8;
  T* dst = (T*)p.dq + b * p.q_sb + r * p.q_sh + (int64_t)i * p.q_sr + sub * 8;
  const f32x4 a = *reinterpret_cast<const f32x4*>(src);
  const f32x4 c = *reinterpret_cast<const f32x4*>(src + 4);
  st4<T>(dst, a[0], a[1], a[2], a[3]);
  st4<T>(dst + 4, c[0], c[1], c[2], c[3]);
}

// ============================================================== launchers
template <typename T, int DH, int DV>
static int launch_pre_t(const KernelParams& p, void* stream) {
  const int64_t rows = (int64_t)p.B * p.H_q * p.n_q;
  if (rows <= 0) return (int)hipSuccess;
  hipLaunchKernelGGL((bwd_pre_kernel<T, DH, DV>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0,
                     (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

template <typename T, int DH, int DV>
static int launch_main_t(const KernelParams& p, void* stream) {
  const int64_t units = p.xcd_map ? ((p.groups + 7) / 8) * 8 : p.groups;
  const int64_t grid = units * p.per_group;
  if (grid <= 0) return (int)hipSuccess;
  hipLaunchKernelGGL((bwd_main_kernel<T, DH, DV>), dim3((unsigned)grid), dim3(256), 0,
                     (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

template <typename T, int DH>
static int launch_dq_t(const KernelParams& p, void* stream) {
  const int64_t threads = (int64_t)p.B * p.H_q * p.n_q * (DH / 8);
  if (threads <= 0) return (int)hipSuccess;
  hipLaunchKernelGGL((bwd_dq_kernel<T, DH>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

int bwd_block_keys(int /*dtype*/) { return 128; }

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

int launch_bwd_pre(const KernelParams& p, int dtype, int d_h, int d_v, void* stream) {
  ATTN_DISPATCH(launch_pre_t)
}

int launch_bwd_main(const KernelParams& p, int dtype, int d_h, int d_v, void* stream) {
  ATTN_DISPATCH(launch_main_t)
}

int launch_bwd_dq(const KernelParams& p, int dtype, int d_h, void* stream) {
  if (dtype == ATTN_BF16) {
    if (d_h == 128) return launch_dq_t<__bf16, 128>(p, stream);
    if (d_h == 64) return launch_dq_t<__bf16, 64>(p, stream);
  } else {
    if (d_h == 128) return launch_dq_t<float, 128>(p, stream);
    if (d_h == 64) return launch_dq_t<float, 64>(p, stream);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace attn
