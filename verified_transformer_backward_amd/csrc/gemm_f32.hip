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

// One operand tile, rows [r0, r0+64) x k [k0, k0+KT) of X(r, k) = X[r*sr + k*sk], held
// in registers between its global loads and its LDS store (two 16-byte chunks per
// thread). load() issues every load at once, always in bounds (indices clamped, an
// element outside the matrix is zeroed by store()), so the loads of the next k step
// run under the current step's MFMAs. store() writes tile[r][k] (k-contiguous rows),
// transposing when X is r-contiguous.
struct OpRegs {
  float4 v[2];
  unsigned valid;   // bit 4e + i: element i of chunk e is inside the matrix
  __device__ __forceinline__ void load(const float* X, int64_t sr, int64_t sk, int kc, int vec, int r0, int k0, int R,
                                       int K) {
    const int tid = threadIdx.x;
    valid = 0;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int idx = tid + 256 * e;
      // kc: 64 rows x 8 chunks of 4 k;  !kc: KT k x 16 chunks of 4 rows
      const int gr = kc ? r0 + (idx >> 3) : r0 + (idx & 15) * 4;
      const int gk = kc ? k0 + (idx & 7) * 4 : k0 + (idx >> 4);
      if (vec) {
        const int cr = min(gr, R - (kc ? 1 : 4)), ck = min(gk, K - (kc ? 4 : 1));
        v[e] = *reinterpret_cast<const float4*>(X + (int64_t)cr * sr + (int64_t)ck * sk);
        if (gr < R && gk < K) valid |= 0xFu << (4 * e);
      } else {
        float t[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = kc ? gr : gr + i, kk = kc ? gk + i : gk;
          t[i] = X[(int64_t)min(rr, R - 1) * sr + (int64_t)min(kk, K - 1) * sk];
          if (rr < R && kk < K) valid |= 1u << (4 * e + i);
        }
        v[e] = make_float4(t[0], t[1], t[2], t[3]);
      }
    }
  }
  __device__ __forceinline__ void store(float* tile, int kc) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int idx = tid + 256 * e;
      const unsigned m = valid >> (4 * e);
      const float4 x = make_float4(m & 1u ? v[e].x : 0.f, m & 2u ? v[e].y : 0.f, m & 4u ? v[e].z : 0.f,
                                   m & 8u ? v[e].w : 0.f);
      if (kc) {
        *reinterpret_cast<float4*>(tile + (idx >> 3) * LDT + (idx & 7) * 4) = x;
      } else {
        const int k = idx >> 4, rq = (idx & 15) * 4;
        tile[(rq + 0) * LDT + k] = x.x;
        tile[(rq + 1) * LDT + k] = x.y;
        tile[(rq + 2) * LDT + k] = x.z;
        tile[(rq + 3) * LDT + k] = x.w;
      }
    }
  }
};

// Tiles of two GEMMs in one grid: blocks [0, tiles0) compute d0, the rest d1. Per k
// step: one barrier (step k in LDS, step k-1 retired), the next step's loads issued into
// registers, this step's MFMAs, then the registers stored into the other LDS buffer.
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmDesc d0, GemmDesc d1, int tiles0) {
  __shared__ __attribute__((aligned(32))) float sA[2][BMG * LDT];
  __shared__ __attribute__((aligned(32))) float sB[2][BNG * LDT];
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

  OpRegs ra, rb;
  ra.load(d.A, d.am, d.ak, d.a_kc, d.vec, m0, 0, d.M, d.K);
  rb.load(d.B, d.bn, d.bk, d.b_kc, d.vec, n0, 0, d.N, d.K);
  ra.store(sA[0], d.a_kc);
  rb.store(sB[0], d.b_kc);
  const int nk = (d.K + KT - 1) / KT;
  for (int s = 0; s < nk; ++s) {
    __syncthreads();
    const bool more = s + 1 < nk;
    if (more) {
      ra.load(d.A, d.am, d.ak, d.a_kc, d.vec, m0, (s + 1) * KT, d.M, d.K);
      rb.load(d.B, d.bn, d.bk, d.b_kc, d.vec, n0, (s + 1) * KT, d.N, d.K);
    }
    const float* a_t = sA[s & 1];
    const float* b_t = sB[s & 1];
    f32x8 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = load8<float>(a_t + (wm + 16 * i + lc) * LDT + 8 * lg);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = load8<float>(b_t + (wn + 16 * j + lc) * LDT + 8 * lg);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) mma(acc[i][j], a[i], b[j]);
    if (more) {
      ra.store(sA[(s + 1) & 1], d.a_kc);
      rb.store(sB[(s + 1) & 1], d.b_kc);
    }
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
  // The kernel's clamped loads need every extent, the contraction included, >= 1.
  if (T < 1 || K < 1 || N < 1) return hipErrorInvalidValue;
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
