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

#include <cmath>
#include <cstdint>
#include "launch.h"

namespace vtb {
namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;

__device__ __forceinline__ void rope_sincos(double theta, float* s, float* c) {
  const double red = theta - kTwoPi * rint(theta / kTwoPi);
  sincosf((float)red, s, c);
}

// A float4 store that bypasses cache retention (written once, never read back here).
__device__ __forceinline__ void nt_store4(float4* p, const float4& v) {
  const f32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(p));
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
template <typename E>
__global__ __launch_bounds__(256) void rope_bwd_kernel(const E* dy, E* dx, int n_tok,
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
      const float y0 = to_f32(dy[o + ia]), y1 = to_f32(dy[o + ib]);
      dx[o + ia] = from_f32<E>(y0 * c + y1 * s);
      dx[o + ib] = from_f32<E>(-y0 * s + y1 * c);
    }
  }
}

// Vector form: one 256-thread workgroup per token, float4 moves. Every load of the token's
// row is issued first; meanwhile the first head_dim/2 threads put the token's (cos, sin)
// per frequency into LDS (angle formed and reduced in fp64, sin/cos in fp32), so each
// angle is computed once per token and shared by all heads.
// A 16-byte vector holds W = 4 (fp32) or 8 (bf16) elements. LAYOUT 0 pairs (2i, 2i+1): a
// vector holds W/2 pairs. LAYOUT 1 pairs (i, i + d/2): a unit is the vector at i and the
// vector at i + d/2 of the same head, W pairs.
// dx == dy is allowed: a thread stores only what it loaded itself, after the barrier.
template <typename E, int LAYOUT, int NV>
__global__ __launch_bounds__(256) void rope_bwd_vec_kernel(const E* dy_, E* dx_, int n_heads, int hd,
                                                           int64_t tok_stride_v, const int32_t* __restrict__ pos,
                                                           int pos0, double log2_base) {
  using V = typename Vec16<E>::type;
  constexpr int W = Vec16<E>::n;
  extern __shared__ float2 cs[];   // [hd / 2] (cos, sin)
  const V* dy = reinterpret_cast<const V*>(dy_);
  V* dx = reinterpret_cast<V*>(dx_);
  const int t = blockIdx.x, tid = threadIdx.x;
  const int hdv = hd / W, Cv = n_heads * hdv;
  const int units = LAYOUT == 0 ? Cv : Cv / 2;
  const int64_t ro = (int64_t)t * tok_stride_v;
  V a[NV], b[NV];
  int ia[NV], ib[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int u = min(tid + 256 * e, units - 1);
    if (LAYOUT == 0) {
      ia[e] = ib[e] = u;
    } else {
      const int h = u / (hdv / 2), j = u % (hdv / 2);
      ia[e] = h * hdv + j;
      ib[e] = ia[e] + hdv / 2;
    }
    a[e] = dy[ro + ia[e]];
    if (LAYOUT == 1) b[e] = dy[ro + ib[e]];
  }
  const double pp = pos ? (double)pos[t] : (double)pos0 + t;
  for (int i = tid; i < hd / 2; i += 256) {
    float sn, cn;
    rope_sincos(pp * exp2(-(2.0 * i / hd) * log2_base), &sn, &cn);
    cs[i] = make_float2(cn, sn);
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    if (tid + 256 * e >= units) continue;
    if (LAYOUT == 0) {
      const int i0 = ((W * ia[e]) % hd) / 2;
      V r;
#pragma unroll
      for (int k = 0; k < W / 2; ++k) {
        const float2 c = cs[i0 + k];
        const float y0 = to_f32(a[e][2 * k]), y1 = to_f32(a[e][2 * k + 1]);
        r[2 * k] = from_f32<E>(y0 * c.x + y1 * c.y);
        r[2 * k + 1] = from_f32<E>(-y0 * c.y + y1 * c.x);
      }
      __builtin_nontemporal_store(r, &dx[ro + ia[e]]);
    } else {
      const int i0 = W * (ia[e] % hdv);
      V ra, rb;
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const float2 c = cs[i0 + k];
        const float ya = to_f32(a[e][k]), yb = to_f32(b[e][k]);
        ra[k] = from_f32<E>(ya * c.x + yb * c.y);
        rb[k] = from_f32<E>(-ya * c.y + yb * c.x);
      }
      __builtin_nontemporal_store(ra, &dx[ro + ia[e]]);
      __builtin_nontemporal_store(rb, &dx[ro + ib[e]]);
    }
  }
}

// ---------------------------------------------------------------------- RMSNorm backward
// One 256-thread block per row; a row of up to 256*MAXE values stays in registers.
template <typename E, int MAXE>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const E* __restrict__ x, const float* __restrict__ gamma,
                                                          const E* __restrict__ dy, E* __restrict__ dx, int n,
                                                          float eps) {
  const int64_t row = blockIdx.x;
  const E* xr = x + row * n;
  const E* dyr = dy + row * n;
  float xv[MAXE], gv[MAXE];
  float ss = 0.f, cc = 0.f;
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int idx = threadIdx.x + 256 * e;
    xv[e] = 0.f;
    gv[e] = 0.f;
    if (idx < n) {
      xv[e] = to_f32(xr[idx]);
      gv[e] = to_f32(dyr[idx]) * gamma[idx];
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
    if (idx < n) __builtin_nontemporal_store(from_f32<E>((gv[e] - xv[e] * coef) * rinv), &dx[row * n + idx]);
  }
}

// Vector form: one 256-thread block per row, 16-byte vectors of x and dy (W = 4 fp32 or 8
// bf16 elements) held in registers between the two row sums and the store; gamma is read
// as W fp32 values per vector. Vectors past the row end are clamped to its last vector and
// masked out of the sums and stores, so every load is issued before the reduction.
template <typename E, int NV>
__global__ __launch_bounds__(256) void rmsnorm_bwd_vec_kernel(const E* __restrict__ x, const float* __restrict__ gamma,
                                                              const E* __restrict__ dy, E* __restrict__ dx, int n,
                                                              float eps) {
  using V = typename Vec16<E>::type;
  constexpr int W = Vec16<E>::n;
  const int64_t row = blockIdx.x;
  const int nv = n / W;
  const V* xr = reinterpret_cast<const V*>(x + row * n);
  const V* dyr = reinterpret_cast<const V*>(dy + row * n);
  V xv[NV], yv[NV];
  float gv[NV][W];
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int u = min((int)threadIdx.x + 256 * e, nv - 1);
    xv[e] = xr[u];
    yv[e] = dyr[u];
#pragma unroll
    for (int k = 0; k < W; k += 4) {
      const f32x4 g4 = *reinterpret_cast<const f32x4*>(gamma + W * u + k);
      gv[e][k] = g4[0];
      gv[e][k + 1] = g4[1];
      gv[e][k + 2] = g4[2];
      gv[e][k + 3] = g4[3];
    }
  }
  float ss = 0.f, cc = 0.f;
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    if ((int)threadIdx.x + 256 * e < nv) {
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const float xe = to_f32(xv[e][k]);
        gv[e][k] *= to_f32(yv[e][k]);
        ss = fmaf(xe, xe, ss);
        cc = fmaf(gv[e][k], xe, cc);
      }
    }
  }
  const float2 tot = block_sum2(ss, cc);
  const float r2 = tot.x / n + eps;
  const float rinv = rsqrtf(r2);
  const float coef = tot.y / (n * r2);
  V* dxr = reinterpret_cast<V*>(dx + row * n);
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int u = (int)threadIdx.x + 256 * e;
    if (u < nv) {
      V o;
#pragma unroll
      for (int k = 0; k < W; ++k) o[k] = from_f32<E>((gv[e][k] - to_f32(xv[e][k]) * coef) * rinv);
      __builtin_nontemporal_store(o, &dxr[u]);
    }
  }
}

// Rows too long for registers: two passes over global memory.
template <typename E>
__global__ __launch_bounds__(256) void rmsnorm_bwd_long_kernel(const E* __restrict__ x, const float* __restrict__ gamma,
                                                               const E* __restrict__ dy, E* __restrict__ dx, int n,
                                                               float eps) {
  const int64_t row = blockIdx.x;
  const E* xr = x + row * n;
  const E* dyr = dy + row * n;
  float ss = 0.f, cc = 0.f;
  for (int idx = threadIdx.x; idx < n; idx += 256) {
    const float xe = to_f32(xr[idx]);
    ss = fmaf(xe, xe, ss);
    cc = fmaf(to_f32(dyr[idx]) * gamma[idx], xe, cc);
  }
  const float2 tot = block_sum2(ss, cc);
  const float r2 = tot.x / n + eps;
  const float rinv = rsqrtf(r2);
  const float coef = tot.y / (n * r2);
  for (int idx = threadIdx.x; idx < n; idx += 256)
    dx[row * n + idx] = from_f32<E>((to_f32(dyr[idx]) * gamma[idx] - to_f32(xr[idx]) * coef) * rinv);
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

// Vector form of the fused tail (row width a multiple of 4, heads split into whole
// float4s, 16-byte aligned rows). One workgroup per token row:
//  * every global load of the row is issued first, unconditionally (indices clamped);
//  * meanwhile the first head_dim/2 threads build the row's (cos, sin) table in LDS, one
//    angle per frequency instead of one per pair: theta_i = p * 2^(-(2i/d) log2 base),
//    formed and reduced modulo 2 pi in fp64, sin/cos in fp32;
//  * rotation, the two RMSNorm row sums, one block reduction, and float4 stores.
// LAYOUT 0 pairs (2i, 2i+1): a float4 holds two pairs. LAYOUT 1 pairs (i, i + d/2): a unit
// is the float4 at i and the float4 at i + d/2 of the same head, four pairs.
template <int LAYOUT, int NV>
__global__ __launch_bounds__(256) void rope_rmsnorm_res_vec_kernel(const float4* __restrict__ dq, float dq_scale,
                                                                   const float4* __restrict__ x,
                                                                   const float4* __restrict__ gamma, const float4* dh_out,
                                                                   float4* dh_in, int n_heads, int hd, int pos0,
                                                                   double log2_base, float eps) {
  extern __shared__ float2 cs[];   // [hd / 2] (cos, sin) of this row's angles
  const int t = blockIdx.x, tid = threadIdx.x;
  const int C = n_heads * hd, C4 = C / 4, hd4 = hd / 4;
  const int units = LAYOUT == 0 ? C4 : C4 / 2;
  const int64_t ro = (int64_t)t * C4;
  float4 qa[NV], qb[NV], xa[NV], xb[NV], ga[NV], gb[NV], ha[NV], hb[NV];
  int ia[NV], ib[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int u = min(tid + 256 * e, units - 1);
    if (LAYOUT == 0) {
      ia[e] = u;
      ib[e] = u;
    } else {
      const int h = u / (hd4 / 2), j = u % (hd4 / 2);
      ia[e] = h * hd4 + j;
      ib[e] = ia[e] + hd4 / 2;
    }
    qa[e] = dq[ro + ia[e]];
    xa[e] = x[ro + ia[e]];
    ha[e] = dh_out[ro + ia[e]];
    ga[e] = gamma[ia[e]];
    if (LAYOUT == 1) {
      qb[e] = dq[ro + ib[e]];
      xb[e] = x[ro + ib[e]];
      hb[e] = dh_out[ro + ib[e]];
      gb[e] = gamma[ib[e]];
    }
  }
  const int half = hd / 2;
  const double pp = (double)pos0 + t;
  for (int i = tid; i < half; i += 256) {
    float sn, cn;
    rope_sincos(pp * exp2(-(2.0 * i / hd) * log2_base), &sn, &cn);
    cs[i] = make_float2(cn, sn);
  }
  __syncthreads();
  float ss = 0.f, cc = 0.f;
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const bool on = tid + 256 * e < units;
    if (LAYOUT == 0) {
      const int i0 = ((4 * ia[e]) % hd) / 2;
      const float2 c0 = cs[i0], c1 = cs[i0 + 1];
      const float y0 = qa[e].x * dq_scale, y1 = qa[e].y * dq_scale, y2 = qa[e].z * dq_scale, y3 = qa[e].w * dq_scale;
      qa[e] = make_float4(y0 * c0.x + y1 * c0.y, -y0 * c0.y + y1 * c0.x, y2 * c1.x + y3 * c1.y, -y2 * c1.y + y3 * c1.x);
      if (on) {
        ss += xa[e].x * xa[e].x + xa[e].y * xa[e].y + xa[e].z * xa[e].z + xa[e].w * xa[e].w;
        cc += qa[e].x * ga[e].x * xa[e].x + qa[e].y * ga[e].y * xa[e].y + qa[e].z * ga[e].z * xa[e].z +
              qa[e].w * ga[e].w * xa[e].w;
      }
    } else {
      const int i0 = 4 * (ia[e] % hd4);
      const float ya[4] = {qa[e].x * dq_scale, qa[e].y * dq_scale, qa[e].z * dq_scale, qa[e].w * dq_scale};
      const float yb[4] = {qb[e].x * dq_scale, qb[e].y * dq_scale, qb[e].z * dq_scale, qb[e].w * dq_scale};
      float ra[4], rb[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float2 c = cs[i0 + k];
        ra[k] = ya[k] * c.x + yb[k] * c.y;
        rb[k] = -ya[k] * c.y + yb[k] * c.x;
      }
      qa[e] = make_float4(ra[0], ra[1], ra[2], ra[3]);
      qb[e] = make_float4(rb[0], rb[1], rb[2], rb[3]);
      if (on) {
        ss += xa[e].x * xa[e].x + xa[e].y * xa[e].y + xa[e].z * xa[e].z + xa[e].w * xa[e].w +
              xb[e].x * xb[e].x + xb[e].y * xb[e].y + xb[e].z * xb[e].z + xb[e].w * xb[e].w;
        cc += qa[e].x * ga[e].x * xa[e].x + qa[e].y * ga[e].y * xa[e].y + qa[e].z * ga[e].z * xa[e].z +
              qa[e].w * ga[e].w * xa[e].w + qb[e].x * gb[e].x * xb[e].x + qb[e].y * gb[e].y * xb[e].y +
              qb[e].z * gb[e].z * xb[e].z + qb[e].w * gb[e].w * xb[e].w;
      }
    }
  }
  const float2 tot = block_sum2(ss, cc);
  const float r2 = tot.x / C + eps;
  const float rinv = rsqrtf(r2);
  const float coef = tot.y / (C * r2);
  auto out = [&](const float4& y, const float4& g, const float4& xx, const float4& h) {
    return make_float4(h.x + (y.x * g.x - xx.x * coef) * rinv, h.y + (y.y * g.y - xx.y * coef) * rinv,
                       h.z + (y.z * g.z - xx.z * coef) * rinv, h.w + (y.w * g.w - xx.w * coef) * rinv);
  };
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    if (tid + 256 * e < units) {
      nt_store4(&dh_in[ro + ia[e]], out(qa[e], ga[e], xa[e], ha[e]));
      if (LAYOUT == 1) nt_store4(&dh_in[ro + ib[e]], out(qb[e], gb[e], xb[e], hb[e]));
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

template <typename E>
hipError_t rope_bwd_t(const E* dy, E* dx, int n_tok, int n_heads, int head_dim, int64_t tok_stride, const int32_t* pos,
                      int pos0, double base, int layout, hipStream_t s) {
  constexpr int W = Vec16<E>::n;
  const int64_t C = (int64_t)n_heads * head_dim;
  const bool vec = (layout == 0 ? head_dim % W == 0 : head_dim % (2 * W) == 0) && tok_stride % W == 0 &&
                   C / W <= 256 * 8 && ((uintptr_t)dy | (uintptr_t)dx) % 16 == 0;
  if (vec) {
    const int units = (int)(layout == 0 ? C / W : C / (2 * W));
    const int nv = (units + 255) / 256;
    const size_t lds = (size_t)(head_dim / 2) * sizeof(float2);
    const double l2b = std::log2(base);
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(n_tok), dim3(256), lds, s, dy, dx, n_heads, head_dim, tok_stride / W, pos, pos0, l2b);
    };
    if (layout == 0) {
      if (nv <= 1) go(rope_bwd_vec_kernel<E, 0, 1>);
      else if (nv <= 2) go(rope_bwd_vec_kernel<E, 0, 2>);
      else if (nv <= 4) go(rope_bwd_vec_kernel<E, 0, 4>);
      else go(rope_bwd_vec_kernel<E, 0, 8>);
    } else {
      if (nv <= 1) go(rope_bwd_vec_kernel<E, 1, 1>);
      else if (nv <= 2) go(rope_bwd_vec_kernel<E, 1, 2>);
      else if (nv <= 4) go(rope_bwd_vec_kernel<E, 1, 4>);
      else go(rope_bwd_vec_kernel<E, 1, 8>);
    }
    return hipGetLastError();
  }
  const int64_t items = (int64_t)n_tok * (head_dim / 2);
  hipLaunchKernelGGL(rope_bwd_kernel<E>, dim3(grid_for(items)), dim3(256), 0, s, dy, dx, n_tok, n_heads, head_dim,
                     tok_stride, pos, pos0, base, layout);
  return hipGetLastError();
}

template <typename E>
hipError_t rmsnorm_bwd_t(const E* x, const float* gamma, const E* dy, E* dx, int rows, int n, float eps, hipStream_t s) {
  constexpr int W = Vec16<E>::n;
  if (n % W == 0 && n <= 256 * W * 4 && ((uintptr_t)x | (uintptr_t)gamma | (uintptr_t)dy | (uintptr_t)dx) % 16 == 0) {
    const int nv = (n / W + 255) / 256;
    if (nv <= 1)
      hipLaunchKernelGGL((rmsnorm_bwd_vec_kernel<E, 1>), dim3(rows), dim3(256), 0, s, x, gamma, dy, dx, n, eps);
    else if (nv <= 2)
      hipLaunchKernelGGL((rmsnorm_bwd_vec_kernel<E, 2>), dim3(rows), dim3(256), 0, s, x, gamma, dy, dx, n, eps);
    else if (nv <= 3)
      hipLaunchKernelGGL((rmsnorm_bwd_vec_kernel<E, 3>), dim3(rows), dim3(256), 0, s, x, gamma, dy, dx, n, eps);
    else
      hipLaunchKernelGGL((rmsnorm_bwd_vec_kernel<E, 4>), dim3(rows), dim3(256), 0, s, x, gamma, dy, dx, n, eps);
    return hipGetLastError();
  }
  if (n <= 256 * 4)
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<E, 4>), dim3(rows), dim3(256), 0, s, x, gamma, dy, dx, n, eps);
  else if (n <= 256 * 16)
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<E, 16>), dim3(rows), dim3(256), 0, s, x, gamma, dy, dx, n, eps);
  else
    hipLaunchKernelGGL(rmsnorm_bwd_long_kernel<E>, dim3(rows), dim3(256), 0, s, x, gamma, dy, dx, n, eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_bwd(int bf16, const void* dy, void* dx, int n_tok, int n_heads, int head_dim, int64_t tok_stride,
                           const int32_t* pos, int pos0, double base, int layout, hipStream_t s) {
  if (bf16)
    return rope_bwd_t(static_cast<const __bf16*>(dy), static_cast<__bf16*>(dx), n_tok, n_heads, head_dim, tok_stride, pos,
                      pos0, base, layout, s);
  return rope_bwd_t(static_cast<const float*>(dy), static_cast<float*>(dx), n_tok, n_heads, head_dim, tok_stride, pos,
                    pos0, base, layout, s);
}

hipError_t launch_rmsnorm_bwd(int bf16, const void* x, const float* gamma, const void* dy, void* dx, int rows, int n,
                              float eps, hipStream_t s) {
  if (bf16)
    return rmsnorm_bwd_t(static_cast<const __bf16*>(x), gamma, static_cast<const __bf16*>(dy), static_cast<__bf16*>(dx),
                         rows, n, eps, s);
  return rmsnorm_bwd_t(static_cast<const float*>(x), gamma, static_cast<const float*>(dy), static_cast<float*>(dx), rows, n,
                       eps, s);
}

hipError_t launch_rope_rmsnorm_res_bwd(const float* dq, float dq_scale, const float* x, const float* gamma,
                                       const float* dh_out, float* dh_in, int T, int n_heads, int head_dim, int pos0,
                                       double base, int layout, float eps, hipStream_t s) {
  const int npairs = n_heads * head_dim / 2;
  const int C = n_heads * head_dim;
  const bool vec = C % 4 == 0 && (layout == 0 ? head_dim % 4 == 0 : head_dim % 8 == 0) &&
                   ((uintptr_t)dq | (uintptr_t)x | (uintptr_t)gamma | (uintptr_t)dh_out | (uintptr_t)dh_in) % 16 == 0;
  if (vec) {
    const int units = layout == 0 ? C / 4 : C / 8;
    const int nv = (units + 255) / 256;   // 1 .. 4 (rows hold at most 4096 values)
    const size_t lds = (size_t)(head_dim / 2) * sizeof(float2);
    const double l2b = std::log2(base);
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(T), dim3(256), lds, s, reinterpret_cast<const float4*>(dq), dq_scale,
                         reinterpret_cast<const float4*>(x), reinterpret_cast<const float4*>(gamma),
                         reinterpret_cast<const float4*>(dh_out), reinterpret_cast<float4*>(dh_in), n_heads, head_dim, pos0,
                         l2b, eps);
    };
    if (layout == 0) {
      if (nv <= 1) go(rope_rmsnorm_res_vec_kernel<0, 1>);
      else if (nv <= 2) go(rope_rmsnorm_res_vec_kernel<0, 2>);
      else go(rope_rmsnorm_res_vec_kernel<0, 4>);
    } else {
      if (nv <= 1) go(rope_rmsnorm_res_vec_kernel<1, 1>);
      else if (nv <= 2) go(rope_rmsnorm_res_vec_kernel<1, 2>);
      else go(rope_rmsnorm_res_vec_kernel<1, 4>);
    }
    return hipGetLastError();
  }
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

hipError_t launch_zero_bthd(void* x, int bf16, int B, int T, int H, int D, const int64_t st[3], hipStream_t s,
                            KernelEvents ev) {
  const int64_t n = (int64_t)B * T * H * D;
  if (n <= 0) return hipSuccess;
  if (bf16)
    launch_kernel(zero_bthd_kernel<__bf16>, dim3(grid_for(n)), dim3(256), 0, s, ev, reinterpret_cast<__bf16*>(x), B, T,
                       H, D, st[0], st[1], st[2]);
  else
    launch_kernel(zero_bthd_kernel<float>, dim3(grid_for(n)), dim3(256), 0, s, ev, reinterpret_cast<float*>(x), B, T, H,
                       D, st[0], st[1], st[2]);
  return hipGetLastError();
}

}  // namespace vtb
