// Linear backward of Y = X W on fp32 MFMA (v_mfma_f32_16x16x4_f32).
//
// The Hesper commit log states linear backward as an outer-product dW and a transposed
// dX; the transformer.js `backward` writes the same for Wo (gWo = ctxOut^T dx2,
// dctx = dx2 Wo^T):
//     dX = dY W^T   (T x K)       contraction over N, both operands N-contiguous
//     dW = X^T dY   (K x N)       contraction over the T tokens, operands row-strided
// One launch holds the tiles of both products: dX tiles first (their contraction is the
// long one), then dW tiles. Each 256-thread workgroup computes a 64 x 64 tile; each wave
// a 32 x 32 quarter as 2 x 2 MFMA tiles. A and B tiles are staged in LDS k-contiguous,
// transposing on the way in when the global operand is m- or n-contiguous.
#include "device_common.h"
#include "launch.h"

namespace vtb {
namespace {

constexpr int BMG = 64, BNG = 64, KT = 32, LDT = KT + 8;

struct GemmDesc {
  const float* A;
  int64_t am, ak;  // A(m, k) = A[m * am + k * ak]
  const float* B;
  int64_t bk, bn;  // B(k, n) = B[k * bk + n * bn]
  float* C;
  int64_t ldc;     // C[m * ldc + n]
  int M, N, K;
  int a_kc;        // 1: A is k-contiguous (ak == 1); 0: m-contiguous (am == 1)
  int b_kc;        // 1: B is k-contiguous (bk == 1); 0: n-contiguous (bn == 1)
  int vec;         // float4 loads are valid along the contiguous dimensions
};

// Stage rows [r0, r0+64) x k [k0, k0+KT) of an operand X(r, k) = X[r*sr + k*sk] into
// tile[r][k]. kc: X is k-contiguous (sk == 1); else r-contiguous (sr == 1).
__device__ __forceinline__ void stage(float* tile, const float* X, int64_t sr, int64_t sk, int kc, int vec, int r0,
                                      int k0, int R, int K) {
  const int tid = threadIdx.x;
  if (kc) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int idx = tid + 256 * e;  // 64 rows x 8 float4
      const int r = idx >> 3, kq = (idx & 7) * 4;
      const int gr = r0 + r, gk = k0 + kq;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (gr < R) {
        const float* src = X + (int64_t)gr * sr + gk;
        if (vec) {
          if (gk < K) v = *reinterpret_cast<const float4*>(src);
        } else {
          if (gk < K) v.x = src[0];
          if (gk + 1 < K) v.y = src[1];
          if (gk + 2 < K) v.z = src[2];
          if (gk + 3 < K) v.w = src[3];
        }
      }
      *reinterpret_cast<float4*>(tile + r * LDT + kq) = v;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int idx = tid + 256 * e;  // KT k-rows x 16 float4 along r
      const int k = idx >> 4, rq = (idx & 15) * 4;
      const int gr = r0 + rq, gk = k0 + k;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (gk < K) {
        const float* src = X + (int64_t)gk * sk + gr;
        if (vec) {
          if (gr < R) v = *reinterpret_cast<const float4*>(src);
        } else {
          if (gr < R) v.x = src[0];
          if (gr + 1 < R) v.y = src[1];
          if (gr + 2 < R) v.z = src[2];
          if (gr + 3 < R) v.w = src[3];
        }
      }
      tile[(rq + 0) * LDT + k] = v.x;
      tile[(rq + 1) * LDT + k] = v.y;
      tile[(rq + 2) * LDT + k] = v.z;
      tile[(rq + 3) * LDT + k] = v.w;
    }
  }
}

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmDesc d0, GemmDesc d1, int tiles0) {
  __shared__ __attribute__((aligned(32))) float sA[BMG * LDT];
  __shared__ __attribute__((aligned(32))) float sB[BNG * LDT];
  const bool first = (int)blockIdx.x < tiles0;
  const GemmDesc& d = first ? d0 : d1;
  const int tile = first ? blockIdx.x : blockIdx.x - tiles0;
  const int ntn = (d.N + BNG - 1) / BNG;
  const int m0 = (tile / ntn) * BMG, n0 = (tile % ntn) * BNG;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  const int wm = (w >> 1) * 32, wn = (w & 1) * 32;

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < d.K; k0 += KT) {
    __syncthreads();
    stage(sA, d.A, d.am, d.ak, d.a_kc, d.vec, m0, k0, d.M, d.K);
    stage(sB, d.B, d.bn, d.bk, d.b_kc, d.vec, n0, k0, d.N, d.K);
    __syncthreads();
    f32x8 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = load8<float>(sA + (wm + 16 * i + lc) * LDT + 8 * lg);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = load8<float>(sB + (wn + 16 * j + lc) * LDT + 8 * lg);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) mma(acc[i][j], a[i], b[j]);
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm + 16 * i + 4 * lg + r, n = n0 + wn + 16 * j + lc;
        if (m < d.M && n < d.N) d.C[(int64_t)m * d.ldc + n] = acc[i][j][r];
      }
}

int tiles_of(const GemmDesc& d) { return ((d.M + BMG - 1) / BMG) * ((d.N + BNG - 1) / BNG); }

}  // namespace

hipError_t launch_linear_bwd(const float* x, const float* w, const float* dy, float* dx, float* dw, int T, int K, int N,
                             hipStream_t s) {
  // dX(t, k) = sum_n dY(t, n) W(k, n): A = dY (k-contiguous), B(n_c, k_out) = W[k_out*N + n_c]
  GemmDesc gx{};
  gx.A = dy; gx.am = N; gx.ak = 1; gx.a_kc = 1;
  gx.B = w; gx.bk = 1; gx.bn = N; gx.b_kc = 1;
  gx.C = dx; gx.ldc = K; gx.M = T; gx.N = K; gx.K = N;
  gx.vec = (N % 4 == 0);
  // dW(k, n) = sum_t X(t, k) dY(t, n): A(k, t) = X[t*K + k] (m-contiguous), B(t, n) = dY[t*N + n] (n-contiguous)
  GemmDesc gw{};
  gw.A = x; gw.am = 1; gw.ak = K; gw.a_kc = 0;
  gw.B = dy; gw.bk = N; gw.bn = 1; gw.b_kc = 0;
  gw.C = dw; gw.ldc = N; gw.M = K; gw.N = N; gw.K = T;
  gw.vec = (K % 4 == 0) && (N % 4 == 0);
  const int tx = dx ? tiles_of(gx) : 0;
  const int tw = dw ? tiles_of(gw) : 0;
  if (tx + tw == 0) return hipSuccess;
  if (tx)
    hipLaunchKernelGGL(gemm_f32_kernel, dim3(tx + tw), dim3(256), 0, s, gx, gw, tx);
  else
    hipLaunchKernelGGL(gemm_f32_kernel, dim3(tw), dim3(256), 0, s, gw, gw, tw);
  return hipGetLastError();
}

}  // namespace vtb
