// Elementwise backward tail: RoPE backward, RMSNorm backward and the fused per-row
// RoPE -> RMSNorm -> residual kernel of one layer's backward.
//
// RoPE: "Hesper.Training.VerifiedBackward", section "RoPE (Rotary Position Embedding)",
// ropeBackward = rotation by -theta, theta(pos, i) = pos * base^(-2i/head_dim). The angle
// is formed and reduced modulo 2 pi in fp64 (positions reach 8191 rad, where an fp32
// angle would already be off by ~5e-4 rad), then sin/cos are taken in fp32.
// RMSNorm: same page, section "RMSNorm", rmsNormBackward: with rms = sqrt(mean(x^2)+eps)
// and c = sum_j dy_j gamma_j x_j, dx_i = (dy_i gamma_i - x_i c / (n rms^2)) / rms. Both row
// sums are taken in one pass, in registers, with wavefront shuffles and one LDS exchange.
// Residual: the hidden gradient passes through unchanged and the branch gradient is
// added (Hesper commit log, residual backward).
#include "device_common.h"
#include "launch.h"

namespace vtb {
namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;

__device__ __forceinline__ void rope_sincos(double theta, float* s, float* c) {
  const double red = theta - kTwoPi * rint(theta / kTwoPi);
  sincosf((float)red, s, c);
}

// Sum two values over the whole block (blockDim.x == 256).
__device__ __forceinline__ float2 block_sum2(float a, float b) {
  __shared__ float red[2][8];
  a = wave_sum(a);
  b = wave_sum(b);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    red[0][w] = a;
    red[1][w] = b;
  }
  __syncthreads();
  float ra = 0.f, rb = 0.f;
  const int nw = blockDim.x >> 6;
  for (int i = 0; i < nw; ++i) {
    ra += red[0][i];
    rb += red[1][i];
  }
  __syncthreads();
  return make_float2(ra, rb);
}

// ---------------------------------------------------------------------- RoPE backward
// One thread per (token, pair index i); it rotates pair i of every head of the token
// with one sin/cos, so the transcendental work is shared across heads.
__global__ __launch_bounds__(256) void rope_bwd_kernel(const float* dy, float* dx, int n_tok,
                                                       int n_heads, int hd, int64_t tok_stride,
                                                       const int32_t* __restrict__ pos, int pos0, double base,
                                                       int layout) {
  const int half = hd / 2;
  const int64_t items = (int64_t)n_tok * half;
  for (int64_t it = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; it < items; it += (int64_t)gridDim.x * blockDim.x) {
    const int t = it / half, i = it % half;
    const double pp = pos ? (double)pos[t] : (double)pos0 + t;
    float s, c;
    rope_sincos(pp * pow(base, -2.0 * i / hd), &s, &c);
    const int64_t row = (int64_t)t * tok_stride;
    const int ia = layout == 0 ? 2 * i : i;
    const int ib = layout == 0 ? 2 * i + 1 : i + half;
    for (int h = 0; h < n_heads; ++h) {
      const int64_t o = row + (int64_t)h * hd;
      const float y0 = dy[o + ia], y1 = dy[o + ib];
      dx[o + ia] = y0 * c + y1 * s;
      dx[o + ib] = -y0 * s + y1 * c;
    }
  }
}

// ---------------------------------------------------------------------- RMSNorm backward
// One 256-thread block per row; a row of up to 256*MAXE values stays in registers.
template <int MAXE>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const float* __restrict__ x, const float* __restrict__ gamma,
                                                          const float* __restrict__ dy, float* __restrict__ dx, int n,
                                                          float eps) {
  const int64_t row = blockIdx.x;
  const float* xr = x + row * n;
  const float* dyr = dy + row * n;
  float xv[MAXE], gv[MAXE];
  float ss = 0.f, cc = 0.f;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int idx = threadIdx.x + 256 * e;
    xv[e] = 0.f;
    gv[e] = 0.f;
    if (idx < n) {
      xv[e] = xr[idx];
      gv[e] = dyr[idx] * gamma[idx];
      ss = fmaf(xv[e], xv[e], ss);
      cc = fmaf(gv[e], xv[e], cc);
    }
  }
  const float2 tot = block_sum2(ss, cc);
  const float r2 = tot.x / n + eps;
  const float rinv = rsqrtf(r2);
  const float coef = tot.y / (n * r2);
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int idx = threadIdx.x + 256 * e;
    if (idx < n) dx[row * n + idx] = (gv[e] - xv[e] * coef) * rinv;
  }
}

// Rows too long for registers: two passes over global memory.
__global__ __launch_bounds__(256) void rmsnorm_bwd_long_kernel(const float* __restrict__ x, const float* __restrict__ gamma,
                                                               const float* __restrict__ dy, float* __restrict__ dx, int n,
                                                               float eps) {
  const int64_t row = blockIdx.x;
  const float* xr = x + row * n;
  const float* dyr = dy + row * n;
  float ss = 0.f, cc = 0.f;
  for (int idx = threadIdx.x; idx < n; idx += 256) {
    const float xe = xr[idx];
    ss = fmaf(xe, xe, ss);
    cc = fmaf(dyr[idx] * gamma[idx], xe, cc);
  }
  const float2 tot = block_sum2(ss, cc);
  const float r2 = tot.x / n + eps;
  const float rinv = rsqrtf(r2);
  const float coef = tot.y / (n * r2);
  for (int idx = threadIdx.x; idx < n; idx += 256) dx[row * n + idx] = (dyr[idx] * gamma[idx] - xr[idx] * coef) * rinv;
}

// ---------------------------------------------------------------------- fused layer tail
// dh_in = dh_out + RMSNormBackward(x, gamma, RoPEBackward(dq_scale * dq)), one block per
// token row of C = n_heads * hd values; each thread keeps MAXP rotation pairs in registers.
template <int MAXP>
__global__ __launch_bounds__(256) void rope_rmsnorm_res_kernel(const float* __restrict__ dq, float dq_scale,
                                                               const float* __restrict__ x, const float* __restrict__ gamma,
                                                               const float* dh_out, float* dh_in, int n_heads, int hd,
                                                               int pos0, double base, int layout, float eps) {
  const int t = blockIdx.x;
  const int C = n_heads * hd, half = hd / 2, npairs = C / 2;
  const int64_t ro = (int64_t)t * C;
  const double pp = (double)pos0 + t;
  float ya[MAXP], yb[MAXP], xa[MAXP], xb[MAXP], ga[MAXP], gb[MAXP];
  float ss = 0.f, cc = 0.f;
  int last_i = -1;
  float s = 0.f, c = 1.f;
#pragma unroll
  for (int e = 0; e < MAXP; ++e) {
    const int pidx = threadIdx.x + 256 * e;
    ya[e] = yb[e] = xa[e] = xb[e] = ga[e] = gb[e] = 0.f;
    if (pidx < npairs) {
      const int h = pidx / half, i = pidx % half;
      if (i != last_i) {
        rope_sincos(pp * pow(base, -2.0 * i / hd), &s, &c);
        last_i = i;
      }
      const int ia = h * hd + (layout == 0 ? 2 * i : i);
      const int ib = h * hd + (layout == 0 ? 2 * i + 1 : i + half);
      const float y0 = dq[ro + ia] * dq_scale, y1 = dq[ro + ib] * dq_scale;
      ya[e] = y0 * c + y1 * s;
      yb[e] = -y0 * s + y1 * c;
      xa[e] = x[ro + ia];
      xb[e] = x[ro + ib];
      ga[e] = gamma[ia];
      gb[e] = gamma[ib];
      ss = fmaf(xa[e], xa[e], fmaf(xb[e], xb[e], ss));
      cc = fmaf(ya[e] * ga[e], xa[e], fmaf(yb[e] * gb[e], xb[e], cc));
    }
  }
  const float2 tot = block_sum2(ss, cc);
  const float r2 = tot.x / C + eps;
  const float rinv = rsqrtf(r2);
  const float coef = tot.y / (C * r2);
#pragma unroll
  for (int e = 0; e < MAXP; ++e) {
    const int pidx = threadIdx.x + 256 * e;
    if (pidx < npairs) {
      const int h = pidx / half, i = pidx % half;
      const int ia = h * hd + (layout == 0 ? 2 * i : i);
      const int ib = h * hd + (layout == 0 ? 2 * i + 1 : i + half);
      dh_in[ro + ia] = dh_out[ro + ia] + (ya[e] * ga[e] - xa[e] * coef) * rinv;
      dh_in[ro + ib] = dh_out[ro + ib] + (yb[e] * gb[e] - xb[e] * coef) * rinv;
    }
  }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* x, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) x[i] = 0.f;
}

template <typename E>
__global__ __launch_bounds__(256) void zero_bthd_kernel(E* x, int B, int T, int H, int D, int64_t s0, int64_t s1, int64_t s2) {
  const int64_t n = (int64_t)B * T * H * D;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int d = i % D;
    int64_t r = i / D;
    const int h = r % H;
    r /= H;
    const int t = r % T;
    const int b = r / T;
    x[b * s0 + t * s1 + h * s2 + d] = from_f32<E>(0.f);
  }
}

int grid_for(int64_t n) { return (int)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 8192)); }

}  // namespace

hipError_t launch_rope_bwd(const float* dy, float* dx, int n_tok, int n_heads, int head_dim, int64_t tok_stride,
                           const int32_t* pos, int pos0, double base, int layout, hipStream_t s) {
  const int64_t items = (int64_t)n_tok * (head_dim / 2);
  hipLaunchKernelGGL(rope_bwd_kernel, dim3(grid_for(items)), dim3(256), 0, s, dy, dx, n_tok, n_heads, head_dim, tok_stride,
                     pos, pos0, base, layout);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const float* x, const float* gamma, const float* dy, float* dx, int rows, int n, float eps,
                              hipStream_t s) {
  if (n <= 256 * 4)
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<4>, dim3(rows), dim3(256), 0, s, x, gamma, dy, dx, n, eps);
  else if (n <= 256 * 16)
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<16>, dim3(rows), dim3(256), 0, s, x, gamma, dy, dx, n, eps);
  else
    hipLaunchKernelGGL(rmsnorm_bwd_long_kernel, dim3(rows), dim3(256), 0, s, x, gamma, dy, dx, n, eps);
  return hipGetLastError();
}

hipError_t launch_rope_rmsnorm_res_bwd(const float* dq, float dq_scale, const float* x, const float* gamma,
                                       const float* dh_out, float* dh_in, int T, int n_heads, int head_dim, int pos0,
                                       double base, int layout, float eps, hipStream_t s) {
  const int npairs = n_heads * head_dim / 2;
  if (npairs <= 256 * 2)
    hipLaunchKernelGGL(rope_rmsnorm_res_kernel<2>, dim3(T), dim3(256), 0, s, dq, dq_scale, x, gamma, dh_out, dh_in,
                       n_heads, head_dim, pos0, base, layout, eps);
  else if (npairs <= 256 * 8)
    hipLaunchKernelGGL(rope_rmsnorm_res_kernel<8>, dim3(T), dim3(256), 0, s, dq, dq_scale, x, gamma, dh_out, dh_in,
                       n_heads, head_dim, pos0, base, layout, eps);
  else
    return hipErrorInvalidValue;  // rows beyond 4096 values are rejected by validation
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* x, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_f32_kernel, dim3(grid_for(n)), dim3(256), 0, s, x, n);
  return hipGetLastError();
}

hipError_t launch_zero_bthd(void* x, int bf16, int B, int T, int H, int D, const int64_t st[3], hipStream_t s) {
  const int64_t n = (int64_t)B * T * H * D;
  if (n <= 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(zero_bthd_kernel<__bf16>, dim3(grid_for(n)), dim3(256), 0, s, reinterpret_cast<__bf16*>(x), B, T,
                       H, D, st[0], st[1], st[2]);
  else
    hipLaunchKernelGGL(zero_bthd_kernel<float>, dim3(grid_for(n)), dim3(256), 0, s, reinterpret_cast<float*>(x), B, T, H,
                       D, st[0], st[1], st[2]);
  return hipGetLastError();
}

}  // namespace vtb
