// Device-side building blocks for the gfx950 attention kernels.
//
// MFMA shapes used (CDNA4):
//   bf16: v_mfma_f32_32x32x16_bf16   A 32x16, B 16x32, C 32x32 float32
//   fp32: v_mfma_f32_32x32x2_f32     issued 8 times per 16-wide k chunk
// Lane layouts (verified on the device):
//   A operand:  lane l holds A[m = l % 32][k in chunk(l / 32)]
//   B operand:  lane l holds B[k in chunk(l / 32)][n = l % 32]
//   C result:   lane l holds C[m][n = l % 32] for m = 8*(e/4) + 4*(l/32) + e%4,
//               e = 0..15 (the "C-layout" k order).
// A 16-wide k chunk of an operand is 8 values per lane.  Two k orders are used:
//   row order:  k = 8*(l/32) + e          (contiguous 16-byte row reads)
//   C order:    k = 8*(e/4) + 4*(l/32) + e%4
// Both operands of one product always use the same order, so any order is a
// valid split of the sum over k; the C order is the one a C-layout result has
// when it is fed back as an operand, and the one the LDS transpose read
// (ds_read_b64_tr_b16) produces.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define ATTN_LDS __attribute__((address_space(3)))

template <typename T> struct Op;
template <> struct Op<__bf16> { using type = bf16x8; };
template <> struct Op<float> { using type = f32x8; };

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// A compile-time integer passed as a value, so generic lambdas can specialise
// on it (register-array indices must be constants for the arrays to stay in
// registers).
template <int N> struct IC { static constexpr int value = N; };

// ---------------------------------------------------------------- MFMA
__device__ __forceinline__ void mma(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], acc, 0, 0, 0);
}

// ---------------------------------------------------------------- conversions
template <typename T> __device__ __forceinline__ typename Op<T>::type to_op(const float* x);
template <> __device__ __forceinline__ bf16x8 to_op<__bf16>(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];  // v_cvt_pk_bf16_f32: nearest-even
  return r;
}
template <> __device__ __forceinline__ f32x8 to_op<float>(const float* x) {
  f32x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = x[e];
  return r;
}

template <typename T> __device__ __forceinline__ typename Op<T>::type zero_op() {
  typename Op<T>::type r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (T)0.0f;
  return r;
}

// A 32x32 accumulator block doubles as storage for four bf16 operands (the
// bits of operand `part` occupy elements 4 part .. 4 part + 3), so waves that
// hold operands and waves that hold accumulators can share one register array.
__device__ __forceinline__ bf16x8 op_part(const f32x16& r, int part) {
  const f32x4 v = {r[4 * part], r[4 * part + 1], r[4 * part + 2], r[4 * part + 3]};
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ void set_op_part(f32x16& r, int part, const bf16x8& x) {
  const f32x4 v = __builtin_bit_cast(f32x4, x);
#pragma unroll
  for (int i = 0; i < 4; ++i) r[4 * part + i] = v[i];
}

// ---------------------------------------------------------------- LDS tiles
// Layout of a row-major [rows][D] tile in LDS, without padding: the 16-byte
// chunk c of row r is stored at chunk position c ^ f(r) of that row.  Two read
// patterns must be free of bank conflicts (64 banks x 4 bytes):
//   row reads:  16 lanes read the same 16-byte chunk of 16 consecutive rows
//               (operands in row order, ld8_tile);
//   transposed: 32 lanes read 8 bytes each from rows 4i..4i+3, 4 consecutive
//               chunks (ld_tr).
// With 256-byte rows (bf16, d = 128) both patterns touch 16 distinct chunk
// positions modulo 256 bytes for f(r) = 4*(r % 4) + (r / 4) % 4; with 128-byte
// rows (bf16, d = 64; two rows per 256 bytes) for
// f(r) = 4*((r / 2) % 2) + (r / 4) % 4.  float32 tiles (the float32 path)
// reuse the first function on their 16-byte chunks.
template <typename T, int D>
struct Tile {
  static constexpr int STRIDE = D;                        // elements per row
  static constexpr int EPC = 16 / (int)sizeof(T);         // elements per chunk
  static constexpr int CH = D / EPC;                      // chunks per row
  static __device__ __forceinline__ int f(int r) {
    if constexpr (sizeof(T) == 2 && D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    else return ((r & 3) << 2) | ((r >> 2) & 3);
  }
  static_assert(CH >= 8, "swizzle needs at least 8 chunks per row");
  static __device__ __forceinline__ int off(int r, int e) {
    return r * D + ((((e / EPC) ^ f(r))) * EPC) + (e % EPC);
  }
};

// ---------------------------------------------------------------- 8-element row reads
// 8 consecutive elements starting at p (16-byte aligned): one or two b128 reads.
template <typename T> __device__ __forceinline__ typename Op<T>::type ld8(const T* p);
template <> __device__ __forceinline__ bf16x8 ld8<__bf16>(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <> __device__ __forceinline__ f32x8 ld8<float>(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f32x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}
// Elements e..e+7 (e a multiple of 8) of row r of an LDS tile.
template <typename T, int D>
__device__ __forceinline__ typename Op<T>::type ld8_tile(const T* tile, int r, int e) {
  if constexpr (sizeof(T) == 2) {
    return ld8<T>(tile + Tile<T, D>::off(r, e));  // one chunk
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(tile + Tile<T, D>::off(r, e));
    const f32x4 b = *reinterpret_cast<const f32x4*>(tile + Tile<T, D>::off(r, e + 4));
    f32x8 v;
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
    return v;
  }
}

// ---------------------------------------------------------------- transposed reads
// Operand chunk in C order from an LDS tile X[k][n] (n the contiguous index):
// lane l receives X[kb + 8*(e/4) + 4*(l/32) + e%4][nb + l % 32] for e = 0..7.
// Usable as an A operand (m = n index) or a B operand (n index), contracting
// over k.  kb must be a multiple of 16 and nb a multiple of 32.
//
// bf16: two ds_read_b64_tr_b16.  Within each 16-lane group the instruction
// hands lane t element e' of the 64-bit word read by source lane 4*e' + t/4,
// column t % 4; so source lane s points at row (s / 4), columns 4*(s % 4).
template <typename T, int D>
__device__ __forceinline__ typename Op<T>::type ld_tr(const T* X, int kb, int nb) {
  const int l = lane_id();
  if constexpr (sizeof(T) == 2) {
    const int s = l & 15, grp = l >> 4;
    const int r0 = kb + 4 * (grp >> 1) + (s >> 2);
    const int e0 = nb + 16 * (grp & 1) + 4 * (s & 3);
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(X + Tile<T, D>::off(r0, e0)));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(X + Tile<T, D>::off(r0 + 8, e0)));
    union { i16x4 v[2]; bf16x8 b; } u;
    u.v[0] = lo;
    u.v[1] = hi;
    return u.b;
  } else {
    const int r0 = kb + 4 * (l >> 5), n = nb + (l & 31);
    f32x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = X[Tile<T, D>::off(r0 + 8 * (e >> 2) + (e & 3), n)];
    return r;
  }
}

// Lane byte offset, inside one 4 KB G_S block, of the transposed read that
// gives the G_Q product its B operand (lane = query row, eight keys in C
// order) for 32-key slice mt and 16-key step st: add mt * 2048 + st * 256,
// and 128 for the second four keys.  The block holds, at 16-byte chunk
// (kb2 * 2 + st') * 64 + kg' * 32 + k', the eight rows 16 st' + 8 (e / 4) +
// 4 kg' + e % 4 (e = 0..7) of key 32 kb2 + k' (the XD waves' operand layout),
// so four consecutive rows of one key are one 8-byte word, which is what
// ds_read_b64_tr_b16 transposes (source lane s of a 16-lane group reads key
// (s / 4) of its group's four and rows 4 (s % 4) .. + 3).
__device__ __forceinline__ int gs_lane_offset(int lane) {
  const int s = lane & 15, grp = lane >> 4;
  return (((grp & 1) * 64 + (s & 1) * 32 + 4 * (grp >> 1) + (s >> 2)) * 16 + 8 * ((s >> 1) & 1));
}

__device__ __forceinline__ bf16x8 gs_read(const __bf16* blk, int off) {
  const char* base = reinterpret_cast<const char*>(blk);
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(base + off));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(base + off + 128));
  union { i16x4 v[2]; bf16x8 b; } u;
  u.v[0] = lo;
  u.v[1] = hi;
  return u.b;
}

// ---------------------------------------------------------------- precomputed LDS offsets
// The swizzle of a tile depends on the row only through row % 16, and every
// read pattern below starts at a multiple of 16 rows, so a lane's byte
// offsets are fixed for the whole kernel; the row block enters as a
// compile-time or uniform displacement.  (float32 tiles use the generic path.)
//
// Row order, A/B operand rows = lane % 32 (+ rb), k chunk 16*ks + 8*(lane/32).
template <typename T, int D>
struct RowOffsets {
  int off[D / 16];
  // byte offset, within a 32-row block, of the operand lane `lane` reads for k-step ks
  static __device__ __forceinline__ int at(int lane, int ks) {
    return Tile<T, D>::off(lane & 31, 16 * ks + 8 * (lane >> 5)) * (int)sizeof(T);
  }
  __device__ __forceinline__ void init(int lane) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) off[ks] = at(lane, ks);
  }
  // rows rb .. rb+31 (rb a multiple of 32)
  __device__ __forceinline__ typename Op<T>::type read(const T* tile, int rb, int ks) const {
    if constexpr (sizeof(T) == 2) {
      return *reinterpret_cast<const typename Op<T>::type*>(reinterpret_cast<const char*>(tile) +
                                                              rb * D * (int)sizeof(T) + off[ks]);
    } else {
      return ld8_tile<T, D>(tile, rb + (lane_id() & 31), 16 * ks + 8 * (lane_id() >> 5));
    }
  }
};
// Transposed reads (ld_tr) with kb a multiple of 16 and nb = 32 * nt.
template <typename T, int D>
struct TrOffsets {
  int off[2][D / 32];
  // byte offset of half h of the transposed operand of column block nt
  static __device__ __forceinline__ int at(int lane, int h, int nt) {
    const int s = lane & 15, grp = lane >> 4;
    const int r0 = 4 * (grp >> 1) + (s >> 2);
    const int e0 = 16 * (grp & 1) + 4 * (s & 3);
    return Tile<T, D>::off(r0 + 8 * h, 32 * nt + e0) * (int)sizeof(T);
  }
  __device__ __forceinline__ void init(int lane) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nt = 0; nt < D / 32; ++nt) off[h][nt] = at(lane, h, nt);
  }
  // bf16 only: the operand from the two byte offsets of at()
  static __device__ __forceinline__ bf16x8 read_at(const T* tile, int kb, int off0, int off1) {
    const char* base = reinterpret_cast<const char*>(tile) + kb * D * (int)sizeof(T);
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(base + off0));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(base + off1));
    union { i16x4 v[2]; bf16x8 b; } u;
    u.v[0] = lo;
    u.v[1] = hi;
    return u.b;
  }
  __device__ __forceinline__ typename Op<T>::type read(const T* tile, int kb, int nt) const {
    if constexpr (sizeof(T) == 2) {
      return read_at(tile, kb, off[0][nt], off[1][nt]);
    } else {
      return ld_tr<T, D>(tile, kb, 32 * nt);
    }
  }
};

// ---------------------------------------------------------------- cross-lane
// Value of lane l ^ 32 (v_permlane32_swap: swaps the upper half of the first
// operand with the lower half of the second).
__device__ __forceinline__ float partner32(float x) {
  const unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned lo = r[0], hi = r[1];
  return __uint_as_float((lane_id() < 32) ? hi : lo);
}

// ---------------------------------------------------------------- stores
template <typename T> __device__ __forceinline__ void st4(T* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void st4<__bf16>(__bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}
template <> __device__ __forceinline__ void st4<float>(float* p, float a, float b, float c, float d) {
  f32x4 v;
  v[0] = a; v[1] = b; v[2] = c; v[3] = d;
  *reinterpret_cast<f32x4*>(p) = v;
}

// 8 consecutive elements (16-byte aligned) from an operand register.
template <typename T> __device__ __forceinline__ void st8(T* p, const typename Op<T>::type& x);
template <> __device__ __forceinline__ void st8<__bf16>(__bf16* p, const bf16x8& x) {
  *reinterpret_cast<bf16x8*>(p) = x;
}
template <> __device__ __forceinline__ void st8<float>(float* p, const f32x8& x) {
  st4<float>(p, x[0], x[1], x[2], x[3]);
  st4<float>(p + 4, x[4], x[5], x[6], x[7]);
}

// ---------------------------------------------------------------- buffer copies
// Tile copies through buffer loads with the LDS flag (buffer_load_dwordx4 ...
// lds): like global_load_lds they move data from memory into LDS without
// registers, but they are not FLAT instructions, so the compiler's wait
// insertion does not treat an in-flight copy as a pending FLAT access that
// forces every later LDS-read wait to lgkmcnt(0): reads of one buffer can be
// waited for one at a time while the next tile's copy is in flight.
//
// A buffer resource names a byte range starting at `base`; offsets are
// 32-bit (per-lane voffset plus a wave-uniform soffset).  Data format word as
// for gfx9 raw buffers (32-bit elements, no swizzle, no stride).
// The base must be the same in every lane of the wave (a resource lives in
// scalar registers); it is read from the first lane, so the compiler never
// wraps the load in a per-lane loop over distinct resources.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  const uint64_t v = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  void* u = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void buf_copy16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (ATTN_LDS void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void buf_copy4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (ATTN_LDS void*)lds, 4, voff, soff, 0, 0);
}
// Can rows [0, rows) of a tensor with this row stride (elements) and width
// (elements) be addressed with 32-bit byte offsets from row 0?
template <typename T>
__device__ __forceinline__ bool fits_u32(int64_t rows, int64_t row_stride, int width) {
  if (row_stride < 0) return false;
  const int64_t r = rows > 1 ? rows : 1;
  // (a shift and a 64-bit compare with zero stay in scalar instructions; an
  // unsigned 64-bit ordered compare would go through vector registers)
  return ((uint64_t)((r - 1) * row_stride * (int64_t)sizeof(T) + (int64_t)width * (int64_t)sizeof(T)) >> 32) == 0;
}

// ---------------------------------------------------------------- tile staging
// Copies ROWS rows of a row-major [n][D] global tensor (unit stride in d, row
// stride in elements) into an LDS tile laid out as Tile<T, D>, with direct
// global-to-LDS loads (global_load_lds_dwordx4): no registers hold the data
// and the copy completes asynchronously (vmcnt), so the next tile can be in
// flight while the current one is consumed.  One instruction moves 64
// consecutive 16-byte chunks of the tile (lane i -> chunk i), so each lane
// fetches the global chunk that the swizzle places there.  Rows at or beyond
// `limit` are filled with copies of row limit - 1 (limit >= 1): every kernel
// masks those rows out before they can reach an output.
template <typename T, int ROWS, int D, int NT>
struct TileLoad {
  using L = Tile<T, D>;
  static constexpr int CHUNKS = ROWS * L::CH;
  static constexpr int N = CHUNKS / NT;  // instructions per thread
  static_assert(CHUNKS % NT == 0, "tile must split evenly over the threads");

  static __device__ __forceinline__ void issue(const T* base, int64_t row_stride, int row0, int limit, T* lds,
                                               int tid) {
    const int wave_base = __builtin_amdgcn_readfirstlane((tid >> 6) * 64), lane = tid & 63;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int first = wave_base + NT * i;  // first chunk written by this wave instruction
      const int pc = first + lane;           // physical chunk this lane fills
      const int row = pc / L::CH;
      const int chunk = (pc % L::CH) ^ L::f(row);
      const int g = min(row0 + row, limit - 1);
      const T* src = base + (int64_t)g * row_stride + chunk * L::EPC;
      __builtin_amdgcn_global_load_lds((const void*)src, (ATTN_LDS void*)(lds + first * L::EPC), 16, 0, 0);
    }
  }

  // Per-lane byte offsets of a tile copy from the tile's first row: fixed for
  // the whole kernel, so the copy of a tile wholly below the limit costs no
  // vector arithmetic (issue_buf_full).  Meaningful when 64 rows of the
  // tensor fit 32-bit offsets (fits_u32).
  static __device__ __forceinline__ void lane_offsets(int64_t row_stride, int tid, uint32_t (&off)[N]) {
    const int wave_base = __builtin_amdgcn_readfirstlane((tid >> 6) * 64), lane = tid & 63;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int pc = wave_base + NT * i + lane;
      const int row = pc / L::CH;
      const int chunk = (pc % L::CH) ^ L::f(row);
      off[i] = (uint32_t)(((int64_t)row * row_stride + chunk * L::EPC) * (int64_t)sizeof(T));
    }
  }
  // Buffer forms (see buf_rsrc).  Whole tile below the limit: the resource
  // starts at row 0 of the tensor, soff = byte offset of the tile's first
  // row, off = the lane offsets of lane_offsets().
  static __device__ __forceinline__ void issue_buf_full(__amdgpu_buffer_rsrc_t r, uint32_t soff,
                                                        const uint32_t (&off)[N], T* lds, int tid) {
    const int wave_base = __builtin_amdgcn_readfirstlane((tid >> 6) * 64);
#pragma unroll
    for (int i = 0; i < N; ++i) buf_copy16(r, lds + (wave_base + NT * i) * L::EPC, off[i], soff);
  }
  // Any tile, rows at or beyond `limit` repeating row limit - 1; the
  // resource starts at row 0 and every row below the limit must be
  // addressable with 32-bit offsets (fits_u32).
  static __device__ __forceinline__ void issue_buf(__amdgpu_buffer_rsrc_t r, uint32_t row_stride_bytes, int row0,
                                                   int limit, T* lds, int tid) {
    const int wave_base = __builtin_amdgcn_readfirstlane((tid >> 6) * 64), lane = tid & 63;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int first = wave_base + NT * i;
      const int pc = first + lane;
      const int row = pc / L::CH;
      const int chunk = (pc % L::CH) ^ L::f(row);
      const uint32_t g = (uint32_t)min(row0 + row, limit - 1);
      buf_copy16(r, lds + first * L::EPC, g * row_stride_bytes + (uint32_t)(chunk * 16), 0u);
    }
  }
  // General form for row strides too large for 32-bit offsets: one resource
  // per tile row (wave-uniform), the lanes of that row enabled.
  static __device__ __forceinline__ void issue_rows(const T* base, int64_t row_stride, int row0, int limit, T* lds,
                                                    int tid) {
    static_assert(64 % L::CH == 0, "a wave instruction covers whole rows");
    const int wave_base = __builtin_amdgcn_readfirstlane((tid >> 6) * 64), lane = tid & 63;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int first = wave_base + NT * i;
      const int row_first = first / L::CH;
      const int my = lane / L::CH;
      const int chunk = ((first + lane) % L::CH) ^ L::f(row_first + my);
#pragma unroll
      for (int rr = 0; rr < 64 / L::CH; ++rr) {
        const int g = min(row0 + row_first + rr, limit - 1);
        const __amdgpu_buffer_rsrc_t r = buf_rsrc(base + (int64_t)g * row_stride, (uint32_t)(L::CH * 16));
        if (my == rr) buf_copy16(r, lds + first * L::EPC, (uint32_t)(chunk * 16), 0u);
      }
    }
  }
};

// Wait until every global-to-LDS copy issued by this wave has landed.
__device__ __forceinline__ void wait_tile_loads() { __builtin_amdgcn_s_waitcnt(0); }

// Workgroup barrier for multi-stage pipelines: waits until at most N of this
// wave's vector-memory operations (issued in order) are still outstanding and
// all of its LDS accesses are complete, then synchronises the workgroup.
// Unlike __syncthreads(), whose fence drains every pending global-to-LDS copy,
// this lets the copies of later stages stay in flight.  The wait is the
// compiler's own s_waitcnt (so its count of copies in flight, which decides
// the waits it inserts before later LDS reads, knows which copies have
// landed); the barrier's memory clobber keeps memory accesses from moving
// across it.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  // s_waitcnt fields: vmcnt[3:0] and [15:14], expcnt[6:4] (7: no wait), lgkmcnt[11:8] (0)
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (7 << 4));
  asm volatile("s_barrier" ::: "memory");
}

// 64 lanes copy one float each into 256 consecutive LDS bytes (lane i ->
// float i), e.g. two rows of 32 per-query scalars.
__device__ __forceinline__ void load_lane_floats(const float* src, float* lds) {
  __builtin_amdgcn_global_load_lds((const void*)src, (ATTN_LDS void*)lds, 4, 0, 0);
}

// ---------------------------------------------------------------- work mapping
// Work is grouped in units (a sequence and a KV head) of `per_group` items.
// With xcd_map, unit u runs on XCD u % 8: workgroups are dealt to the 8 XCDs
// round-robin, so slot `wg / 8` of XCD `wg % 8` takes the slot-th item of that
// XCD's units, and all items of one unit share one XCD's L2.  Returns false
// for the padding workgroups of a unit count that is not a multiple of 8.
// Per-sequence quantities of sequence b of a launch.
struct SeqView {
  int Lq, Lk;          // active query rows, valid keys
  int off;             // causal offset of the sequence (clamped to [0, n_k])
  int nq_lim, nk_lim;  // rows of the sequence present in memory: n_q / n_k in
                       // the padded layout, L_q / L_k in the packed one
                       // (stores stop at them; tile copies clamp to the last
                       // active row / valid key instead, so padding content
                       // never meets a zero probability in a product)
  int64_t q_row0, k_row0;  // first row of the sequence (packed layout; else 0)
};
__device__ __forceinline__ SeqView seq_view(const KernelParams& p, int b) {
  SeqView s;
  s.Lq = p.has_lens ? p.lens_q[b] : p.n_q;
  s.Lk = p.has_lens ? p.lens_k[b] : p.n_k;
  s.off = p.has_offs ? p.offs[b] : p.offset;
  s.nq_lim = p.varlen ? s.Lq : p.n_q;
  s.nk_lim = p.varlen ? s.Lk : p.n_k;
  s.q_row0 = p.varlen ? p.row0_q[b] : 0;
  s.k_row0 = p.varlen ? p.row0_k[b] : 0;
  return s;
}
// Keys [0, key_limit_b) of a sequence are visible to query row i: all L_k
// keys, or with the causal rule those at j <= i + off (off the sequence's
// clamped causal offset).
__device__ __forceinline__ int key_limit_b(int i, int Lk, int causal, int off) {
  return causal ? min(Lk, i + off + 1) : Lk;
}

__device__ __forceinline__ bool map_work(int wg, int groups, int per_group, int xcd_map,
                                         int& unit, int& item) {
  if (!xcd_map) {
    unit = wg / per_group;
    item = wg - unit * per_group;
    return unit < groups;
  }
  const int xcd = wg & 7, slot = wg >> 3;
  const int t = slot / per_group;
  item = slot - t * per_group;
  unit = xcd + 8 * t;
  return unit < groups;
}

// ---------------------------------------------------------------- rotary positions
// Column pair (2k, 2k+1) of a row at position t turns by the angle whose
// cosine and sine the table holds at [t][k] ("Chapter 15: matrix formulas to
// look up", sec. 15.6): x0' = c x0 - s x1, x1' = s x0 + c x1.  Passing -s
// turns back (the backward's transposed rotation, "Chapter 31: attention
// backpropagation", sec. 5).  Every rotation in the library goes through
// this one expression, so a row turned in registers equals the same row
// turned by the standalone kernel bit for bit.
__device__ __forceinline__ void rope_pair(float c, float s, float& x0, float& x1) {
  const float y0 = fmaf(c, x0, -(s * x1));
  const float y1 = fmaf(s, x0, c * x1);
  x0 = y0;
  x1 = y1;
}

// Eight consecutive columns (starting at an even column c0) of a row, turned
// by the four pairs' table entries (t0, t1) = (cos, sin) of each pair in order.
template <typename T>
__device__ __forceinline__ typename Op<T>::type rope8_tab(const typename Op<T>::type& x, const f32x4& t0,
                                                          const f32x4& t1, bool inverse) {
  const float tab[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
#pragma unroll
  for (int m = 0; m < 4; ++m) rope_pair(tab[2 * m], inverse ? -tab[2 * m + 1] : tab[2 * m + 1], v[2 * m], v[2 * m + 1]);
  return to_op<T>(v);
}

// The same reading the entries at cs8 = table row + c0.
template <typename T>
__device__ __forceinline__ typename Op<T>::type rope8(const typename Op<T>::type& x, const float* cs8, bool inverse) {
  return rope8_tab<T>(x, *reinterpret_cast<const f32x4*>(cs8), *reinterpret_cast<const f32x4*>(cs8 + 4), inverse);
}

// A value of column c whose pair partner (column c ^ 1) sits in lane ^ 1:
// turn the pair back by the angle of cs2 = table row + (c & ~1) and keep
// this lane's column.  Every lane of the wave must call it (lane exchange).
__device__ __forceinline__ float rope_back_lanes(float v, float c, float s, bool odd) {
  const float pv = __shfl_xor(v, 1);
  float x0 = odd ? pv : v, x1 = odd ? v : pv;
  rope_pair(c, -s, x0, x1);
  return odd ? x1 : x0;
}

}  // namespace attn
