// LayerNorm (no affine) backward and the FFN's ReLU^2 x Mul backward, in fp32 or bf16
// storage with fp32 arithmetic.
//
// LayerNorm: DaisyChain-Train transformer.js page, `lnBwd` ("layernorm (no affine)"). The
// forward saved y = (x - mean x) / sigma and sigma per row; per row of n values
//     dx = (dy - mean(dy) - y * mean(dy * y)) / sigma.
// Both row means come from one pass over the row, in registers, with wavefront shuffles
// and one LDS exchange; the row is then finished from the same registers.
//
// ReLU^2 x Mul: Hesper pull-request commit log, "FFN backward" (FFNBackward.lean): with
// h = ReLU(gate)^2 * up elementwise,
//     dGate = dH * up * 2 * ReLU(gate),   dUp = dH * ReLU(gate)^2.
// Pure streaming work: 16-byte loads and stores, grid-stride, no LDS.
#include "device_common.h"

#include <algorithm>
#include <cstdint>
#include "launch.h"

namespace vtb {
namespace {

// Sum two values over a 256-thread block.
__device__ __forceinline__ float2 block_sum2_256(float a, float b) {
  __shared__ float red[2][4];
  a = wave_sum(a);
  b = wave_sum(b);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    red[0][w] = a;
    red[1][w] = b;
  }
  __syncthreads();
  const float ra = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
  const float rb = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  return make_float2(ra, rb);
}

// ---------------------------------------------------------------------- LayerNorm backward
// One 256-thread block per row; each thread holds NV 16-byte vectors of dy and y. Loads of
// vectors past the row end are clamped to the row's last vector and masked out of the
// sums and stores, so every load is issued before the reduction.
// With dres (may be null) the residual is added: dx = dres + lnBwd(...); dx == dres is
// allowed, each element of dres being read before the same thread writes it.
template <typename E, int NV>
__global__ __launch_bounds__(256) void layernorm_bwd_vec_kernel(const E* __restrict__ dy, const E* __restrict__ y,
                                                                const float* __restrict__ sig, const E* dres, E* dx,
                                                                int n) {
  using V = typename Vec16<E>::type;
  constexpr int W = Vec16<E>::n;
  const int64_t row = blockIdx.x;
  const int nvec = n / W;
  const V* dyr = reinterpret_cast<const V*>(dy + row * n);
  const V* yr = reinterpret_cast<const V*>(y + row * n);
  V* dxr = reinterpret_cast<V*>(dx + row * n);
  const V* rr = reinterpret_cast<const V*>(dres + row * n);
  V a[NV], b[NV], c[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int u = min((int)threadIdx.x + 256 * e, nvec - 1);
    a[e] = dyr[u];
    b[e] = yr[u];
    if (dres) c[e] = rr[u];
  }
  const float s = sig[row];
  float sdy = 0.f, sdyy = 0.f;
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    if ((int)threadIdx.x + 256 * e < nvec) {
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const float g = to_f32(a[e][k]);
        sdy += g;
        sdyy = fmaf(g, to_f32(b[e][k]), sdyy);
      }
    }
  }
  const float2 tot = block_sum2_256(sdy, sdyy);
  const float mdy = tot.x / n, mdyy = tot.y / n;
  const float rs = 1.0f / s;
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int u = (int)threadIdx.x + 256 * e;
    if (u < nvec) {
      V o;
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const float g = (to_f32(a[e][k]) - mdy - to_f32(b[e][k]) * mdyy) * rs;
        o[k] = from_f32<E>(dres ? to_f32(c[e][k]) + g : g);
      }
      __builtin_nontemporal_store(o, &dxr[u]);
    }
  }
}

// Any row width or alignment: two passes over the row in global memory, one element per
// thread per step.
template <typename E>
__global__ __launch_bounds__(256) void layernorm_bwd_any_kernel(const E* __restrict__ dy, const E* __restrict__ y,
                                                                const float* __restrict__ sig, const E* dres, E* dx,
                                                                int n) {
  const int64_t row = blockIdx.x;
  const E* dyr = dy + row * n;
  const E* yr = y + row * n;
  float sdy = 0.f, sdyy = 0.f;
  for (int j = threadIdx.x; j < n; j += 256) {
    const float g = to_f32(dyr[j]);
    sdy += g;
    sdyy = fmaf(g, to_f32(yr[j]), sdyy);
  }
  const float2 tot = block_sum2_256(sdy, sdyy);
  const float mdy = tot.x / n, mdyy = tot.y / n;
  const float rs = 1.0f / sig[row];
  for (int j = threadIdx.x; j < n; j += 256) {
    const float g = (to_f32(dyr[j]) - mdy - to_f32(yr[j]) * mdyy) * rs;
    dx[row * n + j] = from_f32<E>(dres ? to_f32(dres[row * n + j]) + g : g);
  }
}

// ---------------------------------------------------------------------- ReLU^2 x Mul backward
__device__ __forceinline__ void relu2_mul_grad(float g, float u, float d, float* dg, float* du) {
  const float r = fmaxf(g, 0.f);
  *dg = d * u * 2.f * r;
  *du = d * r * r;
}

// 16-byte vectors over [0, nvec): each thread takes U vectors per round, spaced one grid
// apart, and issues all of their loads before any arithmetic; rounds repeat grid-stride.
// The scalar tail [nvec * W, n) is taken by the first threads of the grid.
template <typename E, int U>
__global__ __launch_bounds__(256) void relu2_mul_bwd_vec_kernel(const E* __restrict__ gate, const E* __restrict__ up,
                                                                const E* __restrict__ dh, E* __restrict__ dgate,
                                                                E* __restrict__ dup, int64_t n) {
  using V = typename Vec16<E>::type;
  constexpr int W = Vec16<E>::n;
  const int64_t nvec = n / W;
  const int64_t grid = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const V* g4 = reinterpret_cast<const V*>(gate);
  const V* u4 = reinterpret_cast<const V*>(up);
  const V* d4 = reinterpret_cast<const V*>(dh);
  V* og = reinterpret_cast<V*>(dgate);
  V* ou = reinterpret_cast<V*>(dup);
  for (int64_t base = t0; base < nvec; base += U * grid) {
    V g[U], u[U], d[U];
#pragma unroll
    for (int r = 0; r < U; ++r) {
      const int64_t i = min(base + r * grid, nvec - 1);
      g[r] = __builtin_nontemporal_load(&g4[i]);
      u[r] = __builtin_nontemporal_load(&u4[i]);
      d[r] = __builtin_nontemporal_load(&d4[i]);
    }
#pragma unroll
    for (int r = 0; r < U; ++r) {
      const int64_t i = base + r * grid;
      if (i < nvec) {
        V rg, ru;
#pragma unroll
        for (int k = 0; k < W; ++k) {
          float a, b;
          relu2_mul_grad(to_f32(g[r][k]), to_f32(u[r][k]), to_f32(d[r][k]), &a, &b);
          rg[k] = from_f32<E>(a);
          ru[k] = from_f32<E>(b);
        }
        // streamed once: nontemporal stores keep the outputs from displacing the inputs in cache
        __builtin_nontemporal_store(rg, &og[i]);
        __builtin_nontemporal_store(ru, &ou[i]);
      }
    }
  }
  const int64_t j = nvec * W + t0;
  if (j < n) {
    float a, b;
    relu2_mul_grad(to_f32(gate[j]), to_f32(up[j]), to_f32(dh[j]), &a, &b);
    dgate[j] = from_f32<E>(a);
    dup[j] = from_f32<E>(b);
  }
}

// Unaligned pointers: one element per step.
template <typename E>
__global__ __launch_bounds__(256) void relu2_mul_bwd_any_kernel(const E* __restrict__ gate, const E* __restrict__ up,
                                                                const E* __restrict__ dh, E* __restrict__ dgate,
                                                                E* __restrict__ dup, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    float a, b;
    relu2_mul_grad(to_f32(gate[i]), to_f32(up[i]), to_f32(dh[i]), &a, &b);
    dgate[i] = from_f32<E>(a);
    dup[i] = from_f32<E>(b);
  }
}

// ---------------------------------------------------------------------- FFN block tail pieces
// Sub-norm backward fused with ReLU^2 x Mul backward, one 256-thread block per token row:
//     h = ReLU(gate)^2 * up                        (formed again from the saved gate and up)
//     dh = RMSNormBackward(h, gamma2, dhn)        (rms over the row's F values)
//     dgate, dup = ReLU^2 x Mul backward(gate, up, dh)
// gate and up are the two halves of a [T, 2F] row (gu), and dgate, dup are written to the
// two halves of dgu the same way, so the gate/up projection's backward is one product.
// Vector form: F a multiple of 4 and 16-byte aligned rows; each thread keeps NV float4s
// of gate, up, dhn and gamma2 between the row sums and the stores.
template <int NV>
__global__ __launch_bounds__(256) void subnorm_relu2_bwd_vec_kernel(const f32x4* __restrict__ gu,
                                                                    const f32x4* __restrict__ dhn,
                                                                    const f32x4* __restrict__ gamma2,
                                                                    f32x4* __restrict__ dgu, int F, float eps) {
  const int64_t t = blockIdx.x;
  const int F4 = F / 4;
  const f32x4* gr = gu + t * 2 * F4;
  const f32x4* dr = dhn + t * F4;
  f32x4 g[NV], u[NV], d[NV], gm[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int c = min((int)threadIdx.x + 256 * e, F4 - 1);
    g[e] = gr[c];
    u[e] = gr[F4 + c];
    d[e] = dr[c];
    gm[e] = gamma2[c];
  }
  float ss = 0.f, cc = 0.f;
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    if ((int)threadIdx.x + 256 * e < F4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float r = fmaxf(g[e][k], 0.f), h = r * r * u[e][k];
        ss = fmaf(h, h, ss);
        cc = fmaf(d[e][k] * gm[e][k], h, cc);
      }
    }
  }
  const float2 tot = block_sum2_256(ss, cc);
  const float r2 = tot.x / F + eps;
  const float rinv = rsqrtf(r2);
  const float coef = tot.y / (F * r2);
  f32x4* orow = dgu + t * 2 * F4;
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int c = (int)threadIdx.x + 256 * e;
    if (c < F4) {
      f32x4 og, ou;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float r = fmaxf(g[e][k], 0.f), h = r * r * u[e][k];
        const float dh = (d[e][k] * gm[e][k] - h * coef) * rinv;
        float a, b;
        relu2_mul_grad(g[e][k], u[e][k], dh, &a, &b);
        og[k] = a;
        ou[k] = b;
      }
      __builtin_nontemporal_store(og, &orow[c]);
      __builtin_nontemporal_store(ou, &orow[F4 + c]);
    }
  }
}

// Any F: two passes over the row in global memory.
__global__ __launch_bounds__(256) void subnorm_relu2_bwd_any_kernel(const float* __restrict__ gu,
                                                                    const float* __restrict__ dhn,
                                                                    const float* __restrict__ gamma2,
                                                                    float* __restrict__ dgu, int F, float eps) {
  const int64_t t = blockIdx.x;
  const float* gr = gu + t * 2 * F;
  const float* dr = dhn + t * F;
  float ss = 0.f, cc = 0.f;
  for (int j = threadIdx.x; j < F; j += 256) {
    const float r = fmaxf(gr[j], 0.f), h = r * r * gr[F + j];
    ss = fmaf(h, h, ss);
    cc = fmaf(dr[j] * gamma2[j], h, cc);
  }
  const float2 tot = block_sum2_256(ss, cc);
  const float r2 = tot.x / F + eps;
  const float rinv = rsqrtf(r2);
  const float coef = tot.y / (F * r2);
  for (int j = threadIdx.x; j < F; j += 256) {
    const float g = gr[j], u = gr[F + j];
    const float r = fmaxf(g, 0.f), h = r * r * u;
    const float dh = (dr[j] * gamma2[j] - h * coef) * rinv;
    relu2_mul_grad(g, u, dh, &dgu[t * 2 * F + j], &dgu[t * 2 * F + F + j]);
  }
}

// RMSNorm backward plus the residual, one 256-thread block per row of n values:
//     dx = dres + RMSNormBackward(x, gamma, dy),
// and, when rinv is not null, the row's 1 / r in rinv[row] (for the gain gradient).
// dx == dres is allowed: each element of dres is read before the same thread writes it.
template <int NV>
__global__ __launch_bounds__(256) void rmsnorm_res_bwd_vec_kernel(const f32x4* __restrict__ x,
                                                                  const f32x4* __restrict__ gamma,
                                                                  const f32x4* __restrict__ dy, const f32x4* dres,
                                                                  f32x4* dx, int n, float eps, float* rinv_out) {
  const int64_t t = blockIdx.x;
  const int n4 = n / 4;
  f32x4 xv[NV], gy[NV], rv[NV];
  float ss = 0.f, cc = 0.f;
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int c = min((int)threadIdx.x + 256 * e, n4 - 1);
    xv[e] = x[t * n4 + c];
    gy[e] = dy[t * n4 + c] * gamma[c];
    rv[e] = dres[t * n4 + c];
  }
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    if ((int)threadIdx.x + 256 * e < n4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ss = fmaf(xv[e][k], xv[e][k], ss);
        cc = fmaf(gy[e][k], xv[e][k], cc);
      }
    }
  }
  const float2 tot = block_sum2_256(ss, cc);
  const float r2 = tot.x / n + eps;
  const float rinv = rsqrtf(r2);
  const float coef = tot.y / (n * r2);
  if (rinv_out && threadIdx.x == 0) rinv_out[t] = rinv;
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int c = (int)threadIdx.x + 256 * e;
    if (c < n4) {
      f32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = rv[e][k] + (gy[e][k] - xv[e][k] * coef) * rinv;
      __builtin_nontemporal_store(o, &dx[t * n4 + c]);
    }
  }
}

__global__ __launch_bounds__(256) void rmsnorm_res_bwd_any_kernel(const float* __restrict__ x,
                                                                  const float* __restrict__ gamma,
                                                                  const float* __restrict__ dy, const float* dres,
                                                                  float* dx, int n, float eps, float* rinv_out) {
  const int64_t t = blockIdx.x;
  const float* xr = x + t * n;
  const float* dyr = dy + t * n;
  float ss = 0.f, cc = 0.f;
  for (int j = threadIdx.x; j < n; j += 256) {
    ss = fmaf(xr[j], xr[j], ss);
    cc = fmaf(dyr[j] * gamma[j], xr[j], cc);
  }
  const float2 tot = block_sum2_256(ss, cc);
  const float r2 = tot.x / n + eps;
  const float rinv = rsqrtf(r2);
  const float coef = tot.y / (n * r2);
  if (rinv_out && threadIdx.x == 0) rinv_out[t] = rinv;
  for (int j = threadIdx.x; j < n; j += 256) dx[t * n + j] = dres[t * n + j] + (dyr[j] * gamma[j] - xr[j] * coef) * rinv;
}

// RMSNorm gain gradient over rows of n values: dgamma_c = sum_t dy_tc x_tc rinv_t. One
// 1024-thread block per 64 columns: lane = column, wave w sums rows w, w + 16, ... in
// order, then the 16 wave partials are added in wave order (bitwise reproducible).
__global__ __launch_bounds__(1024) void rmsnorm_gamma_kernel(const float* __restrict__ x, const float* __restrict__ dy,
                                                             const float* __restrict__ rinv, float* dgamma, int rows,
                                                             int n) {
  __shared__ float part[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  const int cc = min(c, n - 1);
  float acc = 0.f;
  int t = w;
  for (; t + 48 < rows; t += 64) {   // four rows' loads in flight
    float xv[4], dv[4], rv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      xv[u] = x[(int64_t)(t + 16 * u) * n + cc];
      dv[u] = dy[(int64_t)(t + 16 * u) * n + cc];
      rv[u] = rinv[t + 16 * u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = fmaf(dv[u] * xv[u], rv[u], acc);
  }
  for (; t < rows; t += 16) acc = fmaf(dy[(int64_t)t * n + cc] * x[(int64_t)t * n + cc], rinv[t], acc);
  part[w][lane] = acc;
  __syncthreads();
  if (w == 0 && c < n) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += part[i][lane];
    dgamma[c] = s;
  }
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <typename E>
hipError_t layernorm_bwd_t(const E* dy, const E* y, const float* sig, const E* dres, E* dx, int rows, int n,
                           hipStream_t s) {
  constexpr int W = Vec16<E>::n;
  const bool vec = n % W == 0 && n <= 256 * W * 4 && al16(dy) && al16(y) && al16(dx) && al16(dres);
  if (vec) {
    const int nv = (n / W + 255) / 256;
    if (nv <= 1)
      hipLaunchKernelGGL((layernorm_bwd_vec_kernel<E, 1>), dim3(rows), dim3(256), 0, s, dy, y, sig, dres, dx, n);
    else if (nv <= 2)
      hipLaunchKernelGGL((layernorm_bwd_vec_kernel<E, 2>), dim3(rows), dim3(256), 0, s, dy, y, sig, dres, dx, n);
    else if (nv <= 3)
      hipLaunchKernelGGL((layernorm_bwd_vec_kernel<E, 3>), dim3(rows), dim3(256), 0, s, dy, y, sig, dres, dx, n);
    else
      hipLaunchKernelGGL((layernorm_bwd_vec_kernel<E, 4>), dim3(rows), dim3(256), 0, s, dy, y, sig, dres, dx, n);
  } else {
    hipLaunchKernelGGL(layernorm_bwd_any_kernel<E>, dim3(rows), dim3(256), 0, s, dy, y, sig, dres, dx, n);
  }
  return hipGetLastError();
}

template <typename E>
hipError_t relu2_mul_bwd_t(const E* gate, const E* up, const E* dh, E* dgate, E* dup, int64_t n, hipStream_t s) {
  constexpr int W = Vec16<E>::n;
  if (al16(gate) && al16(up) && al16(dh) && al16(dgate) && al16(dup)) {
    // four vectors per thread per round, at most 8192 workgroups (larger inputs take more rounds)
    const int64_t units = std::max<int64_t>(n / W, 1);
    const int grid = (int)std::min<int64_t>((units + 1023) / 1024, 8192);
    hipLaunchKernelGGL((relu2_mul_bwd_vec_kernel<E, 4>), dim3(grid), dim3(256), 0, s, gate, up, dh, dgate, dup, n);
  } else {
    const int grid = (int)std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(relu2_mul_bwd_any_kernel<E>, dim3(grid), dim3(256), 0, s, gate, up, dh, dgate, dup, n);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_subnorm_relu2_bwd(const float* gu, const float* dhn, const float* gamma2, float* dgu, int T, int F,
                             float eps, hipStream_t s) {
  const int F4 = F / 4;
  const bool vec = F % 4 == 0 && F4 <= 256 * 8 && al16(gu) && al16(dhn) && al16(gamma2) && al16(dgu);
  if (vec) {
    const int nv = (F4 + 255) / 256;
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(T), dim3(256), 0, s, reinterpret_cast<const f32x4*>(gu),
                         reinterpret_cast<const f32x4*>(dhn), reinterpret_cast<const f32x4*>(gamma2),
                         reinterpret_cast<f32x4*>(dgu), F, eps);
    };
    if (nv <= 1) go(subnorm_relu2_bwd_vec_kernel<1>);
    else if (nv <= 2) go(subnorm_relu2_bwd_vec_kernel<2>);
    else if (nv <= 4) go(subnorm_relu2_bwd_vec_kernel<4>);
    else if (nv <= 6) go(subnorm_relu2_bwd_vec_kernel<6>);
    else if (nv <= 7) go(subnorm_relu2_bwd_vec_kernel<7>);
    else go(subnorm_relu2_bwd_vec_kernel<8>);
  } else {
    hipLaunchKernelGGL(subnorm_relu2_bwd_any_kernel, dim3(T), dim3(256), 0, s, gu, dhn, gamma2, dgu, F, eps);
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm_res_bwd(const float* x, const float* gamma, const float* dy, const float* dres, float* dx, int T,
                           int n, float eps, hipStream_t s, float* rinv) {
  const int n4 = n / 4;
  const bool vec = n % 4 == 0 && n4 <= 256 * 4 && al16(x) && al16(gamma) && al16(dy) && al16(dres) && al16(dx);
  if (vec) {
    const int nv = (n4 + 255) / 256;
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(T), dim3(256), 0, s, reinterpret_cast<const f32x4*>(x),
                         reinterpret_cast<const f32x4*>(gamma), reinterpret_cast<const f32x4*>(dy),
                         reinterpret_cast<const f32x4*>(dres), reinterpret_cast<f32x4*>(dx), n, eps, rinv);
    };
    if (nv <= 1) go(rmsnorm_res_bwd_vec_kernel<1>);
    else if (nv <= 2) go(rmsnorm_res_bwd_vec_kernel<2>);
    else if (nv <= 3) go(rmsnorm_res_bwd_vec_kernel<3>);
    else go(rmsnorm_res_bwd_vec_kernel<4>);
  } else {
    hipLaunchKernelGGL(rmsnorm_res_bwd_any_kernel, dim3(T), dim3(256), 0, s, x, gamma, dy, dres, dx, n, eps, rinv);
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm_gamma(const float* x, const float* dy, const float* rinv, float* dgamma, int rows, int n,
                                hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_gamma_kernel, dim3((n + 63) / 64), dim3(1024), 0, s, x, dy, rinv, dgamma, rows, n);
  return hipGetLastError();
}

hipError_t launch_layernorm_bwd(int bf16, const void* dy, const void* y, const float* sig, const void* dres, void* dx,
                                int rows, int n, hipStream_t s) {
  if (bf16)
    return layernorm_bwd_t(static_cast<const __bf16*>(dy), static_cast<const __bf16*>(y), sig,
                           static_cast<const __bf16*>(dres), static_cast<__bf16*>(dx), rows, n, s);
  return layernorm_bwd_t(static_cast<const float*>(dy), static_cast<const float*>(y), sig, static_cast<const float*>(dres),
                         static_cast<float*>(dx), rows, n, s);
}

hipError_t launch_relu2_mul_bwd(int bf16, const void* gate, const void* up, const void* dh, void* dgate, void* dup,
                                int64_t n, hipStream_t s) {
  if (bf16)
    return relu2_mul_bwd_t(static_cast<const __bf16*>(gate), static_cast<const __bf16*>(up),
                           static_cast<const __bf16*>(dh), static_cast<__bf16*>(dgate), static_cast<__bf16*>(dup), n, s);
  return relu2_mul_bwd_t(static_cast<const float*>(gate), static_cast<const float*>(up), static_cast<const float*>(dh),
                         static_cast<float*>(dgate), static_cast<float*>(dup), n, s);
}

}  // namespace vtb
