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
// transposing on the way in when the global operand is m- or n-contiguous. Large linear
// products whose tiles all lie inside the matrices take 128 x 128 tiles instead (below).
#include "device_common.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>

namespace vtb {
namespace {

constexpr int BMG = 64, BNG = 64, KT = 32, LDT = KT + 4;

// LDS tiles are [row][k] with rows of LDT = 36 floats: sixteen rows read 16 bytes each at
// one column cover all 64 banks once. Within every group of 16 rows the k index is XORed
// with 8 * (group mod 4), which keeps each 8-float run contiguous (the operand reads take
// 8 k) and spreads the transposing scalar stores of r-contiguous operands over the banks.
__device__ __forceinline__ int lds_col(int r, int k) { return k ^ (((r >> 4) & 3) << 3); }

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
  int nsplit;      // the contraction is cut into nsplit chunks of kchunk (a multiple of KT);
  int kchunk;      // chunk s writes its partial product to C + s * c_split
  int64_t c_split;
  int batch;       // independent products of this shape: product i at A + i a_b, B + i b_b, C + i c_b
  int64_t a_b, b_b, c_b;
  float alpha;     // C = alpha A B
  int tri;         // causal structure with key j visible to query i iff j <= i + tri_off:
  int tri_off;     //   TRI_SCORES: C is a (query, key) score grid; tiles wholly invisible are skipped
};                 //   TRI_KLE: k is the key of row query m (k <= m + off); TRI_KGE: k is the query of row key m (k >= m - off)
enum { TRI_NONE = 0, TRI_SCORES = 1, TRI_KLE = 2, TRI_KGE = 3 };

// One operand tile, rows [r0, r0+64) x k [k0, k0+KT) of X(r, k) = X[r*sr + k*sk], held
// in registers between its global loads and its LDS store (two 16-byte chunks per
// thread). KC: 1 when X is k-contiguous (64 rows x 8 chunks of 4 k), 0 when r-contiguous
// (KT k x 16 chunks of 4 rows). store() writes tile[r][k] (k-contiguous rows),
// transposing when KC == 0.
//
// OpEdge serves tiles that reach past an edge of the matrix: every load is clamped in
// bounds and the elements outside are zeroed by store(). OpInner serves tiles wholly
// inside: the two chunk addresses are computed once and advanced by one k step per load.
template <int KC>
__device__ __forceinline__ void chunk_of(int idx, int& r, int& k) {
  r = KC ? (idx >> 3) : (idx & 15) * 4;
  k = KC ? (idx & 7) * 4 : (idx >> 4);
}

// The two chunks travel as two named float4 values rather than an array: an array member
// that the compiler fails to keep in registers lands in scratch memory, and the wait for
// its store then sits right behind the global loads, exposing their latency every step.
template <int KC>
__device__ __forceinline__ void store_chunk(float* tile, int idx, float4 v) {
  int r, k;
  chunk_of<KC>(idx, r, k);
  if (KC) {
    *reinterpret_cast<float4*>(tile + r * LDT + lds_col(r, k)) = v;
  } else {   // rows r .. r + 3 share one 16-row group, so one column for all four
    const int kk = lds_col(r, k);
    tile[(r + 0) * LDT + kk] = v.x;
    tile[(r + 1) * LDT + kk] = v.y;
    tile[(r + 2) * LDT + kk] = v.z;
    tile[(r + 3) * LDT + kk] = v.w;
  }
}

template <int KC>
struct OpEdge {
  const float* X;
  int64_t sr, sk;
  int r0, R, K, vec;   // K: end of the contraction range being read
  float4 v0, v1;
  unsigned m0, m1;     // bit i: element i of the chunk is inside the matrix
  __device__ __forceinline__ float4 load_chunk(int idx, int k0, unsigned& m) const {
    int r, k;
    chunk_of<KC>(idx, r, k);
    const int gr = r0 + r, gk = k0 + k;
    m = 0;
    if (vec) {
      const int cr = min(gr, R - (KC ? 1 : 4)), ck = min(gk, K - (KC ? 4 : 1));
      if (gr < R && gk < K) m = 0xFu;
      return *reinterpret_cast<const float4*>(X + (int64_t)cr * sr + (int64_t)ck * sk);
    }
    float t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = KC ? gr : gr + i, kk = KC ? gk + i : gk;
      t[i] = X[(int64_t)min(rr, R - 1) * sr + (int64_t)min(kk, K - 1) * sk];
      if (rr < R && kk < K) m |= 1u << i;
    }
    return make_float4(t[0], t[1], t[2], t[3]);
  }
  __device__ __forceinline__ void load(int k0) {
    v0 = load_chunk(threadIdx.x, k0, m0);
    v1 = load_chunk(threadIdx.x + 256, k0, m1);
  }
  static __device__ __forceinline__ float4 masked(float4 v, unsigned m) {
    return make_float4(m & 1u ? v.x : 0.f, m & 2u ? v.y : 0.f, m & 4u ? v.z : 0.f, m & 8u ? v.w : 0.f);
  }
  __device__ __forceinline__ void store(float* tile) const {
    store_chunk<KC>(tile, threadIdx.x, masked(v0, m0));
    store_chunk<KC>(tile, threadIdx.x + 256, masked(v1, m1));
  }
};

template <int KC>
struct OpInner {
  const float *p0, *p1;   // the thread's two chunks at the next k step
  int64_t step;           // elements between consecutive loads (nstep k steps)
  float4 v0, v1;
  __device__ __forceinline__ void init(const float* X, int64_t sr, int64_t sk, int r0, int k0, int nstep) {
    int r, k;
    chunk_of<KC>(threadIdx.x, r, k);
    p0 = X + (int64_t)(r0 + r) * sr + (int64_t)(k0 + k) * sk;
    chunk_of<KC>(threadIdx.x + 256, r, k);
    p1 = X + (int64_t)(r0 + r) * sr + (int64_t)(k0 + k) * sk;
    step = (int64_t)nstep * KT * sk;
  }
  __device__ __forceinline__ void load() {
    v0 = *reinterpret_cast<const float4*>(p0);
    v1 = *reinterpret_cast<const float4*>(p1);
    p0 += step;
    p1 += step;
  }
  __device__ __forceinline__ void store(float* tile) const {
    store_chunk<KC>(tile, threadIdx.x, v0);
    store_chunk<KC>(tile, threadIdx.x + 256, v1);
  }
};

// One 64 x 64 tile of C = alpha A B over k in [kbeg, kend). Per k step: one barrier (step k
// in LDS, step k-1 retired), the next step's loads issued into registers, this step's
// MFMAs, then the registers stored into the other LDS buffer. The last step, which loads
// nothing, is peeled off so that the loop body holds no branch around its loads.
template <bool INNER, int AKC, int BKC>
__device__ __forceinline__ void gemm_tile(const GemmDesc& d, const float* A, const float* Bm, float* C, int m0, int n0,
                                          int kbeg, int kend, float (*sA)[BMG * LDT], float (*sB)[BNG * LDT]) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  const int wm = (w >> 1) * 32, wn = (w & 1) * 32;

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Two register sets per operand: set 0 carries the even k steps, set 1 the odd ones, so
  // a step's loads are issued two steps before its LDS store and have a whole step of
  // MFMAs more to land.
  using OpA = typename std::conditional<INNER, OpInner<AKC>, OpEdge<AKC>>::type;
  using OpB = typename std::conditional<INNER, OpInner<BKC>, OpEdge<BKC>>::type;
  OpA ra0, ra1;
  OpB rb0, rb1;
  if constexpr (INNER) {
    ra0.init(A, d.am, d.ak, m0, kbeg, 2);
    rb0.init(Bm, d.bn, d.bk, n0, kbeg, 2);
    ra1.init(A, d.am, d.ak, m0, kbeg + KT, 2);
    rb1.init(Bm, d.bn, d.bk, n0, kbeg + KT, 2);
  } else {
    ra0.X = A; ra0.sr = d.am; ra0.sk = d.ak; ra0.r0 = m0; ra0.R = d.M; ra0.K = kend; ra0.vec = d.vec;
    rb0.X = Bm; rb0.sr = d.bn; rb0.sk = d.bk; rb0.r0 = n0; rb0.R = d.N; rb0.K = kend; rb0.vec = d.vec;
    ra1 = ra0;
    rb1 = rb0;
  }
  auto load = [&](auto& ra, auto& rb, int k0) {
    if constexpr (INNER) {
      (void)k0;
      ra.load();
      rb.load();
    } else {
      ra.load(k0);
      rb.load(k0);
    }
  };
  auto step_mma = [&](int buf) {
    const float* a_t = sA[buf];
    const float* b_t = sB[buf];
    f32x8 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm + 16 * i + lc;
      a[i] = load8<float>(a_t + r * LDT + lds_col(r, 8 * lg));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = wn + 16 * j + lc;
      b[j] = load8<float>(b_t + r * LDT + lds_col(r, 8 * lg));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) mma(acc[i][j], a[i], b[j]);
  };
  // Step s: LDS buffer s & 1 holds step s. Set L = s & 1 was stored at step s - 1 and now
  // takes step s + 2; the other set, loaded at step s - 1, holds step s + 1 and is stored
  // into the other buffer after the MFMAs.
  //   s_waitcnt lgkmcnt(0) before each barrier: this wave's LDS stores have landed before
  //   the barrier publishes them (written out because the barrier's own fence did not get
  //   this wait onto the loop's back edge in every build).
  //   The scheduling barriers keep the loads ahead of the MFMAs and the LDS stores (which
  //   wait for loads) behind them: left alone, the scheduler moves one or the other across
  //   the MFMAs and the load latency shows.
  auto body = [&](auto set, int s, bool ld, bool st) {
    constexpr int L = decltype(set)::value;
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __syncthreads();
    if (ld) {
      if constexpr (L == 0) load(ra0, rb0, kbeg + (s + 2) * KT);
      else load(ra1, rb1, kbeg + (s + 2) * KT);
    }
    __builtin_amdgcn_sched_barrier(0);
    step_mma(s & 1);
    __builtin_amdgcn_sched_barrier(0);
    if (st) {
      if constexpr (L == 0) {
        ra1.store(sA[(s + 1) & 1]);
        rb1.store(sB[(s + 1) & 1]);
      } else {
        ra0.store(sA[(s + 1) & 1]);
        rb0.store(sB[(s + 1) & 1]);
      }
    }
  };
  const std::integral_constant<int, 0> set0;
  const std::integral_constant<int, 1> set1;
  const int nk = kend > kbeg ? (kend - kbeg + KT - 1) / KT : 0;
  if (nk > 0) {
    load(ra0, rb0, kbeg);
    if (nk > 1) load(ra1, rb1, kbeg + KT);
    ra0.store(sA[0]);
    rb0.store(sB[0]);
  }
  int s = 0;
  for (; s + 3 < nk; s += 2) {
    body(set0, s, true, true);
    body(set1, s + 1, true, true);
  }
  // the last one to three steps (s is even here)
  if (s < nk) body(set0, s, s + 2 < nk, s + 1 < nk);
  if (s + 1 < nk) body(set1, s + 1, false, s + 2 < nk);
  if (s + 2 < nk) body(set0, s + 2, false, false);

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm + 16 * i + 4 * lg + r, n = n0 + wn + 16 * j + lc;
        if (INNER || (m < d.M && n < d.N)) C[(int64_t)m * d.ldc + n] = d.alpha * acc[i][j][r];
      }
}

// Tiles of up to three GEMMs in one grid: blocks [0, t0) compute d0, [t0, t0 + t1) d1,
// the rest d2. A GEMM's tiles are ordered (batch, contraction chunk, m tile, n tile).
__global__ __launch_bounds__(256, 4) void gemm_f32_kernel(GemmDesc d0, GemmDesc d1, GemmDesc d2, int t0, int t1) {
  __shared__ __attribute__((aligned(32))) float sA[2][BMG * LDT];
  __shared__ __attribute__((aligned(32))) float sB[2][BNG * LDT];
  const int bid = blockIdx.x;
  const int which = bid < t0 ? 0 : (bid < t0 + t1 ? 1 : 2);
  const GemmDesc& d = which == 0 ? d0 : (which == 1 ? d1 : d2);
  const int ntn = (d.N + BNG - 1) / BNG, tiles_mn = ((d.M + BMG - 1) / BMG) * ntn;
  const int t = bid - (which == 0 ? 0 : (which == 1 ? t0 : t0 + t1));
  const int bi = t / (tiles_mn * d.nsplit), t2 = t % (tiles_mn * d.nsplit);
  const int split = t2 / tiles_mn, tile = t2 % tiles_mn;
  const int m0 = (tile / ntn) * BMG, n0 = (tile % ntn) * BNG;
  if (d.tri == TRI_SCORES && n0 > m0 + BMG - 1 + d.tri_off) return;   // no visible (query, key) pair
  int kbeg = split * d.kchunk, kend = min(d.K, kbeg + d.kchunk);
  if (d.tri == TRI_KLE) kend = min(kend, m0 + BMG + d.tri_off);
  if (d.tri == TRI_KGE) kbeg = max(kbeg, ((m0 - d.tri_off) / KT) * KT);
  const float* const A = d.A + bi * d.a_b;
  const float* const Bm = d.B + bi * d.b_b;
  float* const C = d.C + split * d.c_split + bi * d.c_b;
  // wholly inside: every chunk in bounds along rows and k, so no clamps or masks
  const bool inner = d.vec && m0 + BMG <= d.M && n0 + BNG <= d.N && kend > kbeg && (kend - kbeg) % KT == 0;
  const int kc = d.a_kc * 2 + d.b_kc;
  if (inner) {
    if (kc == 3) gemm_tile<true, 1, 1>(d, A, Bm, C, m0, n0, kbeg, kend, sA, sB);
    else if (kc == 2) gemm_tile<true, 1, 0>(d, A, Bm, C, m0, n0, kbeg, kend, sA, sB);
    else if (kc == 1) gemm_tile<true, 0, 1>(d, A, Bm, C, m0, n0, kbeg, kend, sA, sB);
    else gemm_tile<true, 0, 0>(d, A, Bm, C, m0, n0, kbeg, kend, sA, sB);
  } else {
    if (kc == 3) gemm_tile<false, 1, 1>(d, A, Bm, C, m0, n0, kbeg, kend, sA, sB);
    else if (kc == 2) gemm_tile<false, 1, 0>(d, A, Bm, C, m0, n0, kbeg, kend, sA, sB);
    else if (kc == 1) gemm_tile<false, 0, 1>(d, A, Bm, C, m0, n0, kbeg, kend, sA, sB);
    else gemm_tile<false, 0, 0>(d, A, Bm, C, m0, n0, kbeg, kend, sA, sB);
  }
}

int tiles_of(const GemmDesc& d) { return ((d.M + BMG - 1) / BMG) * ((d.N + BNG - 1) / BNG) * d.nsplit * d.batch; }

// ------------------------------------------------------------------ 128 x 128 tiles
// Products whose tiles all lie inside the matrices (M and N multiples of 128, every
// contraction chunk a multiple of KT, float4 rows) and that give enough tiles to keep both
// workgroup slots of every CU busy take 128 x 128 tiles. Each wave computes a 64 x 64
// quarter as 4 x 4 MFMA tiles: every operand fragment read from LDS feeds four MFMA tiles
// instead of two, and a k step carries four times the MFMAs of a 64 x 64 tile per barrier
// and per global load. One register set holds the next k step (a step's 128 MFMAs per wave
// outlast its loads). An r-contiguous operand is loaded as 4 x 4 blocks (four float4 along
// r at four consecutive k) and stored k-contiguous, one float4 per row (a transpose in
// registers), so every LDS store is 16 bytes wide.
constexpr int BMB = 128;
constexpr int kBigMinTiles = 1024;   // 2 workgroups per CU, each given two tiles or more

// The thread's four load addresses of one operand at k step k0 (all four advance by KT k
// per step). KC = 1: rows tid / 8 + 32 c at k 4 (tid % 8); KC = 0: rows 4 (tid % 32) .. + 3
// at k 4 (tid / 32) + c, c = 0 .. 3.
template <int KC>
__device__ __forceinline__ void big_ptrs(const float* X, int64_t sr, int64_t sk, int r0, int k0, const float*& p0,
                                         const float*& p1, const float*& p2, const float*& p3) {
  const int tid = threadIdx.x;
  if constexpr (KC) {
    p0 = X + (int64_t)(r0 + (tid >> 3)) * sr + (int64_t)(k0 + 4 * (tid & 7)) * sk;
    p1 = p0 + 32 * sr;
    p2 = p0 + 64 * sr;
    p3 = p0 + 96 * sr;
  } else {
    p0 = X + (int64_t)(r0 + 4 * (tid & 31)) * sr + (int64_t)(k0 + 4 * (tid >> 5)) * sk;
    p1 = p0 + sk;
    p2 = p1 + sk;
    p3 = p2 + sk;
  }
}

// The four loaded float4 of one operand into the k-contiguous LDS tile.
template <int KC>
__device__ __forceinline__ void big_store(float* tile, float4 v0, float4 v1, float4 v2, float4 v3) {
  const int tid = threadIdx.x;
  if constexpr (KC) {
    const int r = tid >> 3, k = 4 * (tid & 7);
    *reinterpret_cast<float4*>(tile + (r + 0) * LDT + lds_col(r + 0, k)) = v0;
    *reinterpret_cast<float4*>(tile + (r + 32) * LDT + lds_col(r + 32, k)) = v1;
    *reinterpret_cast<float4*>(tile + (r + 64) * LDT + lds_col(r + 64, k)) = v2;
    *reinterpret_cast<float4*>(tile + (r + 96) * LDT + lds_col(r + 96, k)) = v3;
  } else {
    const int r = 4 * (tid & 31), k = 4 * (tid >> 5);
    *reinterpret_cast<float4*>(tile + (r + 0) * LDT + lds_col(r + 0, k)) = make_float4(v0.x, v1.x, v2.x, v3.x);
    *reinterpret_cast<float4*>(tile + (r + 1) * LDT + lds_col(r + 1, k)) = make_float4(v0.y, v1.y, v2.y, v3.y);
    *reinterpret_cast<float4*>(tile + (r + 2) * LDT + lds_col(r + 2, k)) = make_float4(v0.z, v1.z, v2.z, v3.z);
    *reinterpret_cast<float4*>(tile + (r + 3) * LDT + lds_col(r + 3, k)) = make_float4(v0.w, v1.w, v2.w, v3.w);
  }
}

// One 128 x 128 tile of C = alpha A B over k in [kbeg, kend), (kend - kbeg) a multiple of
// KT. Per k step: one barrier (step s in LDS, step s - 1 retired), the next step's loads
// issued into registers, this step's MFMAs, then the registers stored into the other buffer.
template <int AKC, int BKC>
__device__ __forceinline__ void gemm_tile_big(const GemmDesc& d, const float* A, const float* Bm, float* C, int m0, int n0,
                                              int kbeg, int kend, float (*sA)[BMB * LDT], float (*sB)[BMB * LDT]) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float *pa0, *pa1, *pa2, *pa3, *pb0, *pb1, *pb2, *pb3;
  big_ptrs<AKC>(A, d.am, d.ak, m0, kbeg, pa0, pa1, pa2, pa3);
  big_ptrs<BKC>(Bm, d.bn, d.bk, n0, kbeg, pb0, pb1, pb2, pb3);
  const int64_t sa = (int64_t)KT * d.ak, sb = (int64_t)KT * d.bk;
  float4 a0, a1, a2, a3, b0, b1, b2, b3;
  auto load = [&]() {
    a0 = *reinterpret_cast<const float4*>(pa0);
    a1 = *reinterpret_cast<const float4*>(pa1);
    a2 = *reinterpret_cast<const float4*>(pa2);
    a3 = *reinterpret_cast<const float4*>(pa3);
    b0 = *reinterpret_cast<const float4*>(pb0);
    b1 = *reinterpret_cast<const float4*>(pb1);
    b2 = *reinterpret_cast<const float4*>(pb2);
    b3 = *reinterpret_cast<const float4*>(pb3);
    pa0 += sa; pa1 += sa; pa2 += sa; pa3 += sa;
    pb0 += sb; pb1 += sb; pb2 += sb; pb3 += sb;
  };
  auto store = [&](int buf) {
    big_store<AKC>(sA[buf], a0, a1, a2, a3);
    big_store<BKC>(sB[buf], b0, b1, b2, b3);
  };
  auto step_mma = [&](int buf) {
    const float* a_t = sA[buf];
    const float* b_t = sB[buf];
    f32x8 b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn + 16 * j + lc;
      b[j] = load8<float>(b_t + r * LDT + lds_col(r, 8 * lg));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm + 16 * i + lc;
      const f32x8 a = load8<float>(a_t + r * LDT + lds_col(r, 8 * lg));
#pragma unroll
      for (int j = 0; j < 4; ++j) mma(acc[i][j], a, b[j]);
    }
  };
  const int nk = (kend - kbeg) / KT;
  if (nk > 0) {
    load();
    store(0);
  }
  //   s_waitcnt lgkmcnt(0) before each barrier: this wave's LDS stores have landed before
  //   the barrier publishes them. The scheduling barriers keep the loads ahead of the
  //   MFMAs and the LDS stores (which wait for the loads) behind them.
  auto body = [&](auto buf_c, int s) {
    constexpr int buf = decltype(buf_c)::value;
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __syncthreads();
    const bool more = s + 1 < nk;
    if (more) load();
    __builtin_amdgcn_sched_barrier(0);
    step_mma(buf);
    __builtin_amdgcn_sched_barrier(0);
    if (more) store(buf ^ 1);
  };
  int s = 0;
  for (; s + 1 < nk; s += 2) {
    body(std::integral_constant<int, 0>{}, s);
    body(std::integral_constant<int, 1>{}, s + 1);
  }
  if (s < nk) body(std::integral_constant<int, 0>{}, s);

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm + 16 * i + 4 * lg + r, n = n0 + wn + 16 * j + lc;
        C[(int64_t)m * d.ldc + n] = d.alpha * acc[i][j][r];
      }
}

// Tiles of up to three GEMMs that all satisfy big_tiles_ok, ordered as in gemm_f32_kernel.
__global__ __launch_bounds__(256, 2) void gemm_f32_big_kernel(GemmDesc d0, GemmDesc d1, GemmDesc d2, int t0, int t1) {
  __shared__ __attribute__((aligned(32))) float sA[2][BMB * LDT];
  __shared__ __attribute__((aligned(32))) float sB[2][BMB * LDT];
  const int bid = blockIdx.x;
  const int which = bid < t0 ? 0 : (bid < t0 + t1 ? 1 : 2);
  const GemmDesc& d = which == 0 ? d0 : (which == 1 ? d1 : d2);
  const int ntn = d.N / BMB, tiles_mn = (d.M / BMB) * ntn;
  const int t = bid - (which == 0 ? 0 : (which == 1 ? t0 : t0 + t1));
  const int bi = t / (tiles_mn * d.nsplit), t2 = t % (tiles_mn * d.nsplit);
  const int split = t2 / tiles_mn, tile = t2 % tiles_mn;
  const int m0 = (tile / ntn) * BMB, n0 = (tile % ntn) * BMB;
  const int kbeg = split * d.kchunk, kend = min(d.K, kbeg + d.kchunk);
  const float* const A = d.A + bi * d.a_b;
  const float* const Bm = d.B + bi * d.b_b;
  float* const C = d.C + split * d.c_split + bi * d.c_b;
  const int kc = d.a_kc * 2 + d.b_kc;
  if (kc == 3) gemm_tile_big<1, 1>(d, A, Bm, C, m0, n0, kbeg, kend, sA, sB);
  else if (kc == 2) gemm_tile_big<1, 0>(d, A, Bm, C, m0, n0, kbeg, kend, sA, sB);
  else if (kc == 1) gemm_tile_big<0, 1>(d, A, Bm, C, m0, n0, kbeg, kend, sA, sB);
  else gemm_tile_big<0, 0>(d, A, Bm, C, m0, n0, kbeg, kend, sA, sB);
}

bool big_tiles_ok(const GemmDesc& d) {
  return d.vec && d.tri == TRI_NONE && d.M % BMB == 0 && d.N % BMB == 0 && d.K % KT == 0 && d.kchunk % KT == 0 &&
         d.kchunk > 0;
}
int tiles_big(const GemmDesc& d) { return (d.M / BMB) * (d.N / BMB) * d.nsplit * d.batch; }

// One launch of the dX and dW products of a linear backward (either may be null).
void launch_linear_pair(const GemmDesc* gx, const GemmDesc* gw, hipStream_t s) {
  const bool big = (!gx || big_tiles_ok(*gx)) && (!gw || big_tiles_ok(*gw)) &&
                   (gx ? tiles_big(*gx) : 0) + (gw ? tiles_big(*gw) : 0) >= kBigMinTiles;
  const GemmDesc& a = gx ? *gx : *gw;
  const GemmDesc& b = gw ? *gw : *gx;
  if (big) {
    const int ta = tiles_big(a), tb = gx && gw ? tiles_big(b) : 0;
    hipLaunchKernelGGL(gemm_f32_big_kernel, dim3(ta + tb), dim3(256), 0, s, a, b, b, ta, tb);
  } else {
    const int ta = tiles_of(a), tb = gx && gw ? tiles_of(b) : 0;
    hipLaunchKernelGGL(gemm_f32_kernel, dim3(ta + tb), dim3(256), 0, s, a, b, b, ta, tb);
  }
}

// out[i] = sum over s of part[s * stride4 + i], in order s = 0, 1, ... (four elements per
// lane; stride4 >= n4 in float4 units)
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float4* __restrict__ part, int ns, int64_t n4,
                                                         float4* __restrict__ out, int64_t stride4) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    float4 a = part[i];
    for (int s = 1; s < ns; ++s) {
      const float4 b = part[s * stride4 + i];
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    out[i] = a;
  }
}

// dX = dY W^T and dW = X^T dY descriptors (whole contraction; see launch_linear_bwd).
void linear_descs(const float* x, const float* w, const float* dy, float* dx, float* dw, int T, int K, int N,
                  GemmDesc& gx, GemmDesc& gw) {
  // dX(t, k) = sum_n dY(t, n) W(k, n): A = dY (k-contiguous), B(n_c, k_out) = W[k_out*N + n_c]
  gx = GemmDesc{};
  gx.A = dy; gx.am = N; gx.ak = 1; gx.a_kc = 1;
  gx.B = w; gx.bk = 1; gx.bn = N; gx.b_kc = 1;
  gx.C = dx; gx.ldc = K; gx.M = T; gx.N = K; gx.K = N;
  gx.vec = (N % 4 == 0);
  gx.nsplit = 1; gx.kchunk = N; gx.c_split = 0;
  gx.batch = 1; gx.alpha = 1.f;
  // dW(k, n) = sum_t X(t, k) dY(t, n): A(k, t) = X[t*K + k] (m-contiguous), B(t, n) = dY[t*N + n] (n-contiguous)
  gw = GemmDesc{};
  gw.A = x; gw.am = 1; gw.ak = K; gw.a_kc = 0;
  gw.B = dy; gw.bk = N; gw.bn = 1; gw.b_kc = 0;
  gw.C = dw; gw.ldc = N; gw.M = K; gw.N = N; gw.K = T;
  gw.vec = (K % 4 == 0) && (N % 4 == 0);
  gw.nsplit = 1; gw.kchunk = T; gw.c_split = 0;
  gw.batch = 1; gw.alpha = 1.f;
}

}  // namespace

hipError_t launch_linear_bwd(const float* x, const float* w, const float* dy, float* dx, float* dw, int T, int K, int N,
                             hipStream_t s) {
  // The kernel's clamped loads need every extent, the contraction included, >= 1.
  if (T < 1 || K < 1 || N < 1) return hipErrorInvalidValue;
  GemmDesc gx, gw;
  linear_descs(x, w, dy, dx, dw, T, K, N, gx, gw);
  if (!dx && !dw) return hipSuccess;
  launch_linear_pair(dx ? &gx : nullptr, dw ? &gw : nullptr, s);
  return hipGetLastError();
}

#ifndef VTB_SPLITK_STEPS           // target k steps per dX chunk of the split contraction
#define VTB_SPLITK_STEPS 24
#endif

int linear_bwd_splits(int T, int K, int N) {
  (void)T;
  (void)K;
  const int nk = (N + KT - 1) / KT;   // k steps of dX's contraction
  const int want = std::max(1, std::min(8, nk / VTB_SPLITK_STEPS));
  const int per = (nk + want - 1) / want;
  return (nk + per - 1) / per;        // every chunk non-empty
}

hipError_t launch_linear_bwd_split(const float* x, const float* w, const float* dy, float* dx, float* dw, int T, int K,
                                   int N, float* part, hipStream_t s) {
  if (T < 1 || K < 1 || N < 1 || !dx || !dw) return hipErrorInvalidValue;
  const int ns = linear_bwd_splits(T, K, N);
  if (ns == 1 || ((int64_t)T * K) % 4) return launch_linear_bwd(x, w, dy, dx, dw, T, K, N, s);
  GemmDesc gx, gw;
  linear_descs(x, w, dy, part, dw, T, K, N, gx, gw);
  const int nk = (N + KT - 1) / KT;
  gx.nsplit = ns;
  gx.kchunk = ((nk + ns - 1) / ns) * KT;
  gx.c_split = (int64_t)T * K;
  launch_linear_pair(&gx, &gw, s);
  const int64_t n4 = (int64_t)T * K / 4;
  const int blocks = (int)std::min<int64_t>((n4 + 255) / 256, 2048);
  hipLaunchKernelGGL(splitk_sum_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<const float4*>(part), ns, n4,
                     reinterpret_cast<float4*>(dx), n4);
  return hipGetLastError();
}

hipError_t launch_linear_bwd_parts(const float* x, const float* w, const float* dy, float* dx, float* dw, int T, int K,
                                   int N, float* part, int* ns_out, hipStream_t s) {
  if (T < 1 || K < 1 || N < 1 || !dx || !dw || !ns_out) return hipErrorInvalidValue;
  const int ns = linear_bwd_splits(T, K, N);
  if (ns == 1 || ((int64_t)T * K) % 4) {
    *ns_out = 1;
    return launch_linear_bwd(x, w, dy, dx, dw, T, K, N, s);
  }
  GemmDesc gx, gw;
  linear_descs(x, w, dy, part, dw, T, K, N, gx, gw);
  const int nk = (N + KT - 1) / KT;
  gx.nsplit = ns;
  gx.kchunk = ((nk + ns - 1) / ns) * KT;
  gx.c_split = (int64_t)T * K;
  launch_linear_pair(&gx, &gw, s);
  *ns_out = ns;
  return hipGetLastError();
}

// ------------------------------------------------------------ attention with a saved P
namespace {

// D_i = sum_j P_ij dP_ij over the visible keys and dS_ij = P_ij (dP_ij - D_i) (zero where
// invisible), in place over dP; one wave per (head, query) row of the [H, T, T] grid.
__global__ __launch_bounds__(256) void softmax_bwd_rows_kernel(const float* __restrict__ P, float* __restrict__ ds,
                                                               int rows, int T, int causal) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= rows) return;
  const int i = r % T, lim = causal ? i : T - 1;
  const float* pr = P + (int64_t)r * T;
  float* dr = ds + (int64_t)r * T;
  float acc = 0.f;
  for (int j = lane; j <= lim; j += 64) acc = fmaf(pr[j], dr[j], acc);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  for (int j = lane; j < T; j += 64) dr[j] = j <= lim ? pr[j] * (dr[j] - acc) : 0.f;
}

// The same with float4 moves for rows of T = 4 T4 <= 256 NV values (16-byte aligned): lane l
// holds float4s l, l + 64, ... of P and dP in registers between the sum and the store, and
// float4s wholly past the row's last visible key are neither read nor summed.
template <int NV>
__global__ __launch_bounds__(256) void softmax_bwd_rows_vec_kernel(const f32x4* __restrict__ P, f32x4* __restrict__ ds,
                                                                   int rows, int T, int causal) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= rows) return;
  const int i = r % T, lim = causal ? i : T - 1, T4 = T / 4;
  const f32x4* pr = P + (int64_t)r * T4;
  f32x4* dr = ds + (int64_t)r * T4;
  f32x4 pv[NV], dv[NV];
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int c = lane + 64 * e, j = 4 * c;
    pv[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[e] = pv[e];
    if (c < T4 && j <= lim) {
      pv[e] = pr[c];
      dv[e] = dr[c];
#pragma unroll
      for (int k = 0; k < 4; ++k) acc = j + k <= lim ? fmaf(pv[e][k], dv[e][k], acc) : acc;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int c = lane + 64 * e, j = 4 * c;
    if (c < T4) {
      f32x4 out;
#pragma unroll
      for (int k = 0; k < 4; ++k) out[k] = j + k <= lim ? pv[e][k] * (dv[e][k] - acc) : 0.f;
      dr[c] = out;
    }
  }
}

// dP, D and dS of 16 QB query rows of one head per workgroup, in one kernel:
//     dO = sum_s part_s (the split-K partials of the product that made it, summed in
//          chunk order on the way in and written once to dout for the dV product),
//     dP = dO V^T on the fp32 matrix cores (16x16x4), D = rowsum(P o dP) over the visible
//     keys, dS = P o (dP - D), zero where invisible,
// for T <= 256 NT (each wave keeps its tiles' dP in registers). Sixteen waves: wave w takes
// the 16-key tiles w, w + 16, ... for every 16-row sub-block of the workgroup, so a V tile
// is loaded once for QB sub-blocks and a workgroup's loads are all in flight at once.
// Lane (m, g) = (lane % 16, lane / 16) holds d = 16 j + 4 g .. 4 g + 3 of query row m of a
// sub-block (A, from LDS) and of key row k0 + m (B); step (j, e) contracts
// d = 16 j + 4 g + e across the four lane groups, so A and B agree on every k. Result
// register r of a tile is (query 4 g + r of the sub-block, key k0 + m). Causal rows write
// dS up to the end of their 64-query block (what the following products read), zeros past
// the visible keys.
constexpr int kDpWaves = 16, kDpQB = 2;
template <int DJ, int NT>
__global__ __launch_bounds__(64 * kDpWaves) void attn_dp_ds_kernel(const float* __restrict__ part, int ns,
                                                                   int64_t part_stride, float* __restrict__ dout,
                                                                   const float* __restrict__ v,
                                                                   const float* __restrict__ P, float* __restrict__ ds,
                                                                   int T, int ld_do, int ld_in, int causal) {
  constexpr int D = 16 * DJ, QB = kDpQB, ROWS = 16 * QB;
  __shared__ float sD[kDpWaves][ROWS];
  __shared__ __attribute__((aligned(16))) float sA[ROWS][D + 4];   // the block's dO rows
  const int h = blockIdx.y, q0 = blockIdx.x * ROWS;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, m = lane & 15, g = lane >> 4;
  const int kvis = causal ? min(T, q0 + ROWS) : T;                  // keys any row of the block sees
  const int kwrite = causal ? min(T, (q0 / 64 + 1) * 64) : T;       // keys whose dS is written
  const int ntile = (kwrite + 15) / 16;
  const float* Ph = P + (int64_t)h * T * T;
  float* dsh = ds + (int64_t)h * T * T;
  // every load of the wave first: its V rows and P values (rows and keys past the ends
  // clamped in bounds; their products are masked)
  f32x4 bv[NT][DJ], pv[QB][NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int k0 = 16 * (w + kDpWaves * i), key = min(k0 + m, T - 1);
    const float* vb = v + (int64_t)key * ld_in + h * D + 4 * g;
#pragma unroll
    for (int j = 0; j < DJ; ++j) bv[i][j] = *reinterpret_cast<const f32x4*>(vb + 16 * j);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[qb][i][r] = Ph[(int64_t)min(q0 + 16 * qb + 4 * g + r, T - 1) * T + key];
  }
  // dO rows: the partials summed in chunk order once per workgroup (one float4 per thread
  // and pass), kept in LDS for every wave's A operand and written to dout for the dV
  // product; rows past T re-read row T - 1 and are not written.
  {
    constexpr int C4 = D / 4;
    for (int idx = threadIdx.x; idx < ROWS * C4; idx += 64 * kDpWaves) {
      const int r = idx / C4, c4 = idx % C4;
      const float* src = part + (int64_t)min(q0 + r, T - 1) * ld_do + h * D + 4 * c4;
      f32x4 x = *reinterpret_cast<const f32x4*>(src);
      for (int sp = 1; sp < ns; ++sp) x += *reinterpret_cast<const f32x4*>(src + sp * part_stride);
      *reinterpret_cast<f32x4*>(&sA[r][4 * c4]) = x;
      if (q0 + r < T && dout != part) *reinterpret_cast<f32x4*>(dout + (int64_t)(q0 + r) * ld_do + h * D + 4 * c4) = x;
    }
  }
  __syncthreads();
  f32x4 dp[QB][NT];
  float dsum[QB][4] = {};
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int k0 = 16 * (w + kDpWaves * i), key = k0 + m;
      dp[qb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (k0 < min(kvis, q0 + 16 * qb + 16) || !causal) {   // uniform over the wave
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
          const f32x4 aj = *reinterpret_cast<const f32x4*>(&sA[16 * qb + m][16 * j + 4 * g]);
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[qb][i] = __builtin_amdgcn_mfma_f32_16x16x4f32(aj[e], bv[i][j][e], dp[qb][i], 0, 0, 0);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = q0 + 16 * qb + 4 * g + r;
        const bool vis = q < T && key < T && (!causal || key <= q);
        pv[qb][i][r] = vis ? pv[qb][i][r] : 0.f;
        dsum[qb][r] = fmaf(pv[qb][i][r], dp[qb][i][r], dsum[qb][r]);
      }
    }
  }
  // D per query: the 16 lanes of a group hold other keys of the same rows, then the waves
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) dsum[qb][r] += __shfl_xor(dsum[qb][r], o, 64);
    }
  if (m == 0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 4; ++r) sD[w][16 * qb + 4 * g + r] = dsum[qb][r];
  }
  __syncthreads();
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float Dq[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float t = 0.f;
#pragma unroll
      for (int ww = 0; ww < kDpWaves; ++ww) t += sD[ww][16 * qb + 4 * g + r];
      Dq[r] = t;
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int t = w + kDpWaves * i, key = 16 * t + m;
      if (t < ntile && key < T) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = q0 + 16 * qb + 4 * g + r;
          if (q < T) dsh[(int64_t)q * T + key] = pv[qb][i][r] * (dp[qb][i][r] - Dq[r]);   // pv = 0 where invisible
        }
      }
    }
  }
}

template <int DJ>
void launch_dp_ds(int nt, dim3 grid, hipStream_t s, const float* part, int ns, int64_t ps, float* dout, const float* v,
                  const float* P, float* ds, int T, int ld_do, int ld_in, int causal) {
  if (nt <= 1)
    hipLaunchKernelGGL((attn_dp_ds_kernel<DJ, 1>), grid, dim3(64 * kDpWaves), 0, s, part, ns, ps, dout, v, P, ds, T, ld_do,
                       ld_in, causal);
  else
    hipLaunchKernelGGL((attn_dp_ds_kernel<DJ, 2>), grid, dim3(64 * kDpWaves), 0, s, part, ns, ps, dout, v, P, ds, T, ld_do,
                       ld_in, causal);
}

}  // namespace

hipError_t launch_attn_saved_p_bwd(const float* q, const float* k, const float* v, const float* dout, const float* P,
                                   float* ds, float* dq, float* dk, float* dv, int T, int H, int D, int ld, float scale,
                                   int causal, hipStream_t s) {
  return launch_attn_saved_p_bwd_ld(q, k, v, dout, P, ds, dq, dk, dv, T, H, D, ld, ld, ld, scale, causal, s);
}

namespace {

// dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO per head, contraction limited to the
// visible keys (dQ) or queries (dK, dV); one launch.
hipError_t launch_attn_dqkv(const float* q, const float* k, const float* dout, const float* P, const float* ds, float* dq,
                            float* dk, float* dv, int T, int H, int D, int ld_in, int ld_do, int ld_out, float scale,
                            int causal, bool v4, hipStream_t s) {
  auto base = [&](GemmDesc& g) {
    g = GemmDesc{};
    g.nsplit = 1;
    g.c_split = 0;
    g.batch = H;
    g.alpha = 1.f;
    g.vec = v4;
  };
  GemmDesc gq, gk;
  base(gq);
  gq.A = ds; gq.am = T; gq.ak = 1; gq.a_kc = 1; gq.a_b = (int64_t)T * T;
  gq.B = k; gq.bk = ld_in; gq.bn = 1; gq.b_kc = 0; gq.b_b = D;
  gq.C = dq; gq.ldc = ld_out; gq.c_b = D;
  gq.M = T; gq.N = D; gq.K = T; gq.kchunk = T;
  gq.alpha = scale;
  gq.tri = causal ? TRI_KLE : TRI_NONE;
  base(gk);
  gk.A = ds; gk.am = 1; gk.ak = T; gk.a_kc = 0; gk.a_b = (int64_t)T * T;
  gk.B = q; gk.bk = ld_in; gk.bn = 1; gk.b_kc = 0; gk.b_b = D;
  gk.C = dk; gk.ldc = ld_out; gk.c_b = D;
  gk.M = T; gk.N = D; gk.K = T; gk.kchunk = T;
  gk.alpha = scale;
  gk.tri = causal ? TRI_KGE : TRI_NONE;
  GemmDesc gv = gk;
  gv.A = P;
  gv.B = dout;
  gv.bk = ld_do;
  gv.C = dv;
  gv.alpha = 1.f;
  const int t0 = tiles_of(gq), t1 = tiles_of(gk), t2 = tiles_of(gv);
  hipLaunchKernelGGL(gemm_f32_kernel, dim3(t0 + t1 + t2), dim3(256), 0, s, gq, gk, gv, t0, t1);
  return hipGetLastError();
}

// dP = dO V^T per head on the (query, key) tiles that hold a visible pair, then the dS rows.
void launch_dp_then_ds_rows(const float* v, const float* dout, const float* P, float* ds, int T, int H, int D, int ld_in,
                            int ld_do, int causal, bool v4, hipStream_t s) {
  GemmDesc gp = GemmDesc{};
  gp.nsplit = 1;
  gp.c_split = 0;
  gp.batch = H;
  gp.alpha = 1.f;
  gp.vec = v4;
  gp.A = dout; gp.am = ld_do; gp.ak = 1; gp.a_kc = 1; gp.a_b = D;
  gp.B = v; gp.bk = 1; gp.bn = ld_in; gp.b_kc = 1; gp.b_b = D;
  gp.C = ds; gp.ldc = T; gp.c_b = (int64_t)T * T;
  gp.M = T; gp.N = T; gp.K = D; gp.kchunk = D;
  gp.tri = causal ? TRI_SCORES : TRI_NONE;
  const int tp = tiles_of(gp);
  hipLaunchKernelGGL(gemm_f32_kernel, dim3(tp), dim3(256), 0, s, gp, gp, gp, tp, 0);
  const int rows = H * T;
  const bool rv = T % 4 == 0 && T <= 1024 && ((uintptr_t)P | (uintptr_t)ds) % 16 == 0;
  const int nv = (T / 4 + 63) / 64;
  if (rv && nv <= 1)
    hipLaunchKernelGGL(softmax_bwd_rows_vec_kernel<1>, dim3((rows + 3) / 4), dim3(256), 0, s,
                       reinterpret_cast<const f32x4*>(P), reinterpret_cast<f32x4*>(ds), rows, T, causal);
  else if (rv)
    hipLaunchKernelGGL(softmax_bwd_rows_vec_kernel<4>, dim3((rows + 3) / 4), dim3(256), 0, s,
                       reinterpret_cast<const f32x4*>(P), reinterpret_cast<f32x4*>(ds), rows, T, causal);
  else
    hipLaunchKernelGGL(softmax_bwd_rows_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, P, ds, rows, T, causal);
}

}  // namespace

hipError_t launch_attn_saved_p_bwd_ld(const float* q, const float* k, const float* v, const float* dout, const float* P,
                                      float* ds, float* dq, float* dk, float* dv, int T, int H, int D, int ld_in,
                                      int ld_do, int ld_out, float scale, int causal, hipStream_t s) {
  if (T < 1 || H < 1 || D < 1 || ld_in < H * D || ld_do < H * D || ld_out < H * D) return hipErrorInvalidValue;
  const bool v4 = T % 4 == 0 && D % 4 == 0 && ld_in % 4 == 0 && ld_do % 4 == 0 && ld_out % 4 == 0;
  launch_dp_then_ds_rows(v, dout, P, ds, T, H, D, ld_in, ld_do, causal, v4, s);
  return launch_attn_dqkv(q, k, dout, P, ds, dq, dk, dv, T, H, D, ld_in, ld_do, ld_out, scale, causal, v4, s);
}

bool attn_dp_ds_fused_applicable(int T, int D, int ld_in, int ld_do, const void* part, const void* v) {
  return T >= 1 && T <= 2 * 16 * kDpWaves && (D == 32 || D == 64 || D == 128) && ld_in % 4 == 0 && ld_do % 4 == 0 &&
         ((uintptr_t)part | (uintptr_t)v) % 16 == 0;
}

hipError_t launch_attn_saved_p_bwd_parts(const float* q, const float* k, const float* v, const float* part, int ns,
                                         int64_t part_stride, float* dout, const float* P, float* ds, float* dq,
                                         float* dk, float* dv, int T, int H, int D, int ld_in, int ld_do, int ld_out,
                                         float scale, int causal, hipStream_t s) {
  if (T < 1 || H < 1 || D < 1 || ns < 1 || ld_in < H * D || ld_do < H * D || ld_out < H * D) return hipErrorInvalidValue;
  const bool v4 = T % 4 == 0 && D % 4 == 0 && ld_in % 4 == 0 && ld_do % 4 == 0 && ld_out % 4 == 0;
  if (attn_dp_ds_fused_applicable(T, D, ld_in, ld_do, part, v) && (ns == 1 || part_stride % 4 == 0) &&
      (uintptr_t)dout % 16 == 0) {
    const dim3 grid((T + 16 * kDpQB - 1) / (16 * kDpQB), H);
    const int nt = (T + 16 * kDpWaves - 1) / (16 * kDpWaves);   // 16-key tiles per wave
    if (D == 32) launch_dp_ds<2>(nt, grid, s, part, ns, part_stride, dout, v, P, ds, T, ld_do, ld_in, causal);
    else if (D == 64) launch_dp_ds<4>(nt, grid, s, part, ns, part_stride, dout, v, P, ds, T, ld_do, ld_in, causal);
    else launch_dp_ds<8>(nt, grid, s, part, ns, part_stride, dout, v, P, ds, T, ld_do, ld_in, causal);
  } else {
    if (ns > 1 || dout != part) {   // dO = sum of the partials, then the two-launch dP / dS form
      if (ld_do != H * D || ((int64_t)T * ld_do) % 4 || part_stride % 4 || part_stride < (int64_t)T * ld_do ||
          ((uintptr_t)part | (uintptr_t)dout) % 16)
        return hipErrorInvalidValue;
      const int64_t n4 = (int64_t)T * ld_do / 4;
      const int blocks = (int)std::min<int64_t>((n4 + 255) / 256, 2048);
      hipLaunchKernelGGL(splitk_sum_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<const float4*>(part), ns, n4,
                         reinterpret_cast<float4*>(dout), part_stride / 4);
    }
    launch_dp_then_ds_rows(v, dout, P, ds, T, H, D, ld_in, ld_do, causal, v4, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attn_dqkv(q, k, dout, P, ds, dq, dk, dv, T, H, D, ld_in, ld_do, ld_out, scale, causal, v4, s);
}

}  // namespace vtb
