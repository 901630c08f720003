// LDS tile layouts and MFMA operand reads from them, shared by the attention kernels.
#pragma once

#include "device_common.h"

namespace vtb {

// LDS layout of a tile with COLS elements of E per row. 256-byte rows (bf16 x 128) are
// stored densely with 16-byte chunk c of row r placed at chunk c ^ f(r),
// f(r) = 2 (r mod 8) + (r / 16 mod 2). gfx950 serves a 16-byte-per-lane read in four
// 16-lane groups (per 32-lane half, the lane quads whose index bits 2..4 have even or
// odd parity) and an 8-byte transpose read in two 32-lane halves, over 64 four-byte
// banks. With this f every group of an MFMA operand row read (16 or 32 rows, one chunk
// per lane group), of a transpose read (8 aligned rows x 2 adjacent chunks) and of a
// tile store (16 lanes per row) touches each bank once. Other shapes are padded by 32
// bytes per row.
template <typename E, int COLS>
struct Lds {
  static constexpr bool kSwz = sizeof(E) == 2 && COLS == 128;
  static constexpr int LD = kSwz ? COLS : COLS + 32 / (int)sizeof(E);
  // chunk XOR of row r (swizzled layout only)
  __device__ __forceinline__ static int chunk_xor(int row) { return ((row & 7) << 1) | ((row >> 4) & 1); }
  __device__ __forceinline__ static int off(int row, int col) {
    if constexpr (kSwz) {
      const int f = chunk_xor(row);
      return row * COLS + ((((col >> 3) ^ f) << 3) | (col & 7));
    } else {
      return row * LD + col;
    }
  }
};

// Unswizzled layout with a given row stride (elements).
template <int LD_>
struct Plain {
  static constexpr int LD = LD_;
  __device__ __forceinline__ static int off(int row, int col) { return row * LD_ + col; }
};

template <typename E>
__device__ __forceinline__ const E* row_ptr(const void* base, const int64_t* st, int b, int t, int h) {
  return reinterpret_cast<const E*>(base) + (int64_t)b * st[0] + (int64_t)t * st[1] + (int64_t)h * st[2];
}

// 8 consecutive row elements (row, col .. col+7) of an LDS tile in layout L.
template <typename L, typename E>
__device__ __forceinline__ frag_t<E> row8(const E* tile, int row, int col) {
  if constexpr (sizeof(E) == 2) {
    return load8<E>(tile + L::off(row, col));
  } else {
    frag_t<E> v;
    const f32x4 a = *reinterpret_cast<const f32x4*>(tile + L::off(row, col));
    const f32x4 b = *reinterpret_cast<const f32x4*>(tile + L::off(row, col + 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[e + 4] = b[e];
    }
    return v;
  }
}

// Column operand: element e of the lane is tile[r0 + e][c] for e < 4 and
// tile[r1 + e - 4][c] for e >= 4, c = c0 + lane % 16 (r0, r1 may depend on the lane's
// 16-lane group). bf16 uses the LDS transpose read (see device_common.h).
template <typename L>
__device__ __forceinline__ bf16x8 col8(const __bf16* tile, int r0, int r1, int c0) {
  const int j = threadIdx.x & 15;
  const __bf16* p0 = tile + L::off(r0 + (j >> 2), c0 + 4 * (j & 3));
  const __bf16* p1 = tile + L::off(r1 + (j >> 2), c0 + 4 * (j & 3));
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, both);
}
template <typename L>
__device__ __forceinline__ f32x8 col8(const float* tile, int r0, int r1, int c0) {
  const int c = c0 + (threadIdx.x & 15);
  f32x8 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = tile[L::off(r0 + e, c)];
    v[e + 4] = tile[L::off(r1 + e, c)];
  }
  return v;
}

}  // namespace vtb
