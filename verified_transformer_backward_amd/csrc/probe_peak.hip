// Measurement probe (not part of the library's C ABI): the bf16 matrix-core rate one
// MI355X actually sustains, for reporting beside the published peak.
//
// Every wave issues independent MFMA accumulations (four accumulators, so no result is
// waited on) with operands held in registers; the loop touches no memory. Each wave
// records its shader-clock cycles (s_memtime) and wall time (s_memrealtime, a 100 MHz
// counter) over the loop, so the caller gets both the sustained FLOP rate and the clock
// the chip ran at while the matrix cores were busy.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

// shape 0: v_mfma_f32_32x32x16_bf16 (32768 FLOP), shape 1: v_mfma_f32_16x16x32_bf16 (16384 FLOP)
template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, float* sink, unsigned long long* clk) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (lane + e));
    b[e] = (__bf16)(0.002f * (lane - e));
  }
  float r = 0.f;
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), t0 = __builtin_amdgcn_s_memrealtime();
  if constexpr (SHAPE == 0) {
    f32x16 acc[4] = {};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int m = 0; m < 4; ++m) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[m]) : "v"(a), "v"(b));
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");   // results complete before they are read
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int e = 0; e < 16; ++e) r += acc[m][e];
  } else {
    f32x4 acc[4] = {};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int m = 0; m < 4; ++m) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[m]) : "v"(a), "v"(b));
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) r += acc[m][e];
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime(), t1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * 256 + threadIdx.x] = r;
  if (lane == 0) {
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    clk[2 * w] = c1 - c0;
    clk[2 * w + 1] = t1 - t0;
  }
}

}  // namespace

extern "C" {

// Runs `blocks` workgroups of 4 waves, each wave issuing 4 * iters MFMAs of the given shape
// (0: 32x32x16, 1: 16x16x32). sink: blocks * 256 floats; clk: blocks * 4 * 2 uint64
// (per wave: shader cycles, 100 MHz ticks). Returns a hipError_t code.
int vtb_probe_mfma_bf16(int shape, int iters, int blocks, float* sink, unsigned long long* clk, void* stream) {
  if (shape < 0 || shape > 1 || iters < 1 || blocks < 1 || !sink || !clk) return (int)hipErrorInvalidValue;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (shape == 0)
    hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(blocks), dim3(256), 0, s, iters, sink, clk);
  else
    hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3(blocks), dim3(256), 0, s, iters, sink, clk);
  return (int)hipGetLastError();
}

}  // extern "C"
