// Standalone rotary-position rotation of Q- or K-shaped tensors (gfx950).
//
// Row t of a sequence turns each column pair (2k, 2k+1) by the angle of its
// position ("Chapter 15: matrix formulas to look up", math.zhuph.uk,
// sec. 15.6); the inverse turns by minus that angle ("Chapter 31: attention
// backpropagation", eonloom handbook, sec. 5).  A pure streaming pass: every
// element is read once and written once, so HBM bandwidth bounds it.  One
// thread owns 8 consecutive columns of a row (16 bytes of bf16, 32 of
// float32); a workgroup of 256 threads covers 256 * 8 / d_h rows per trip and
// makes kTrips trips, with consecutive lanes on consecutive 16-byte chunks of
// a row so every wave reads whole rows.
#include <hip/hip_runtime.h>

#include "attn_device.h"

namespace attn {

namespace {

constexpr int kThreads = 256;
constexpr int kTrips = 4;

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void rope_kernel(const RopeParams p) {
  constexpr int TPR = D / 8;                 // threads per row
  constexpr int RPT = kThreads / TPR;        // rows per trip
  const int b = blockIdx.z, h = blockIdx.y;
  const int L = p.len[b];
  const int tid = threadIdx.x;
  const int c0 = 8 * (tid % TPR);
  const int row_in = tid / TPR;
  const T* X = (const T*)p.x + b * p.x_sb + (int64_t)p.row0[b] * p.x_sr + h * p.x_sh;
  T* Y = (T*)p.y + b * p.y_sb + (int64_t)p.row0[b] * p.y_sr + h * p.y_sh;
  const bool inv = p.inverse != 0;
  const int64_t first = (int64_t)blockIdx.x * RPT * kTrips;
  if (first + (int64_t)kTrips * RPT <= L) {
    // every trip's row exists: all loads issued before the first turn, so
    // the trips' memory latencies overlap
    typename Op<T>::type x[kTrips];
    f32x4 c[kTrips][2];
#pragma unroll
    for (int t = 0; t < kTrips; ++t) {
      const int64_t i = first + t * RPT + row_in;
      x[t] = ld8<T>(X + i * p.x_sr + c0);
      const float* cs = p.cs + (i + p.pos0[b]) * D + c0;
      c[t][0] = *reinterpret_cast<const f32x4*>(cs);
      c[t][1] = *reinterpret_cast<const f32x4*>(cs + 4);
    }
#pragma unroll
    for (int t = 0; t < kTrips; ++t) {
      const int64_t i = first + t * RPT + row_in;
      st8<T>(Y + i * p.y_sr + c0, rope8_tab<T>(x[t], c[t][0], c[t][1], inv));
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < kTrips; ++t) {
    const int64_t i = first + t * RPT + row_in;
    if (i >= L) break;
    const typename Op<T>::type x = ld8<T>(X + i * p.x_sr + c0);
    const float* cs = p.cs + (i + p.pos0[b]) * D + c0;
    st8<T>(Y + i * p.y_sr + c0, rope8<T>(x, cs, inv));
  }
}

template <typename T, int D>
int launch_rope_t(const RopeParams& p, void* stream) {
  constexpr int RPT = kThreads / (D / 8);
  const int64_t blocks = ((int64_t)p.n + RPT * kTrips - 1) / (RPT * kTrips);
  if (blocks <= 0 || p.B <= 0 || p.H <= 0) return (int)hipSuccess;
  hipLaunchKernelGGL((rope_kernel<T, D>), dim3((unsigned)blocks, (unsigned)p.H, (unsigned)p.B), dim3(kThreads), 0,
                     (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

}  // namespace

int launch_rope(const RopeParams& p, int dtype, int d_h, void* stream) {
  if (dtype == ATTN_BF16) {
    if (d_h == 128) return launch_rope_t<__bf16, 128>(p, stream);
    if (d_h == 64) return launch_rope_t<__bf16, 64>(p, stream);
  } else {
    if (d_h == 128) return launch_rope_t<float, 128>(p, stream);
    if (d_h == 64) return launch_rope_t<float, 64>(p, stream);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace attn
