// Device helpers shared by the gfx950 kernels: vector types, MFMA wrappers, LDS
// transpose reads and element conversion.
//
// MFMA operand layouts used throughout (64-lane wavefront, g = lane / 16, c = lane % 16):
//   v_mfma_f32_16x16x32_bf16  A: row c, k = 8g .. 8g+7     B: col c, k = 8g .. 8g+7
//                             C: reg r holds row 4g + r, col c
//   v_mfma_f32_16x16x4_f32    A: row c, k = g               B: col c, k = g
//                             C: same as above
// A contraction only needs A and B to agree on which k each lane/element carries, so
// fp32 operands are kept as 8 values per lane exactly like bf16 ones and issued as 8
// successive 16x16x4 steps (step s uses element s).
//
// ds_read_b64_tr_b16 (gfx950): within each 16-lane group, lane i of the result gets
// element e = word (i % 4) of the 8-byte row loaded by lane 4e + i / 4. When lane j of
// the group points at X[r0 + j/4][c0 + 4 (j%4)] of a row-major bf16 tile, lane i gets
// X[r0 .. r0+3][c0 + i]: four consecutive rows of one column, the "k per lane" operand
// order, read straight from a row-major tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

namespace vtb {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------------ element traits
template <typename E> struct Frag;  // 8 elements of one MFMA operand per lane
template <> struct Frag<__bf16> { using type = bf16x8; };
template <> struct Frag<float> { using type = f32x8; };
template <typename E> using frag_t = typename Frag<E>::type;

// 16 bytes of elements: 4 fp32 or 8 bf16, as one native vector.
template <typename E> struct Vec16;
template <> struct Vec16<float> {
  using type = f32x4;
  static constexpr int n = 4;
};
template <> struct Vec16<__bf16> {
  using type = bf16x8;
  static constexpr int n = 8;
};

__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename E> __device__ __forceinline__ E from_f32(float x);
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// ------------------------------------------------------------------------ MFMA
__device__ __forceinline__ void mma(f32x4& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
}

// ------------------------------------------------------------------------ loads
// 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32 when the row
// stride and column keep that alignment).
template <typename E> __device__ __forceinline__ frag_t<E> load8(const E* p) {
  return *reinterpret_cast<const frag_t<E>*>(p);
}
template <typename E> __device__ __forceinline__ void store8(E* p, const frag_t<E>& v) {
  *reinterpret_cast<frag_t<E>*>(p) = v;
}
template <typename E> __device__ __forceinline__ frag_t<E> zero8() {
  frag_t<E> z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = from_f32<E>(0.f);
  return z;
}

// Column operand from a row-major LDS tile with row stride ld (elements): the lane gets
// tile[r0 + e][col] for e < 4 and tile[r1 + e - 4][col] for e >= 4, where col = c0 + lane%16
// and r0, r1 may depend on the lane's 16-lane group.
__device__ __forceinline__ bf16x8 load_col8(const __bf16* tile, int ld, int r0, int r1, int c0) {
  const int j = threadIdx.x & 15;
  const __bf16* p0 = tile + (r0 + (j >> 2)) * ld + c0 + 4 * (j & 3);
  const __bf16* p1 = tile + (r1 + (j >> 2)) * ld + c0 + 4 * (j & 3);
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, both);
}
__device__ __forceinline__ f32x8 load_col8(const float* tile, int ld, int r0, int r1, int c0) {
  const int c = c0 + (threadIdx.x & 15);
  f32x8 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = tile[(r0 + e) * ld + c];
    v[e + 4] = tile[(r1 + e) * ld + c];
  }
  return v;
}

// ------------------------------------------------------------------------ reductions
// Sum / max over the 16 lanes of a lane's 16-lane group.
__device__ __forceinline__ float group16_sum(float v) {
  v += __shfl_xor(v, 8, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 1, 64);
  return v;
}
__device__ __forceinline__ float group16_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 8, 64));
  v = fmaxf(v, __shfl_xor(v, 4, 64));
  v = fmaxf(v, __shfl_xor(v, 2, 64));
  v = fmaxf(v, __shfl_xor(v, 1, 64));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace vtb
