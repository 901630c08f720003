// Attention backward for gfx950, recomputing P from the saved row log-sum-exp.
//
// The chain is the one "Hesper.Training.VerifiedBackward" states for one query
// (section "Attention (full single-head)": attentionBackwardQ / attentionBackwardV built
// from softmaxBackward and scaledDotBackwardQ/K), for every query row of every head:
//   P = exp(scale Q K^T - lse);  dP = dO V^T;  D = rowsum(P o dP);  dS = P o (dP - D)
//   dQ = scale dS K;  dK = scale dS^T Q;  dV = P^T dO
// with the causal mask of the DaisyChain-Train transformer.js `backward` (key j visible
// to query i iff j <= i + Tk - Tq).
//
// Three launches:
//   pre   Q-parallel. Recomputes S and dP over the visible keys of each row and reduces
//         D_i (and, when no lse is given, lse_i by a lane-local online max/sum merged
//         across lanes at the end). Zeroes the fp32 dQ accumulator rows it owns.
//   main  KV-parallel: one workgroup owns BN keys of one kv-head and walks every query
//         block (of every q-head of the group) that sees them. K and V stay in
//         registers as MFMA operands; Q and dO tiles are staged in LDS and read both
//         row-wise (for S, dP) and column-wise through the gfx950 LDS transpose read
//         (for dK^T += Q^T dS and dV^T += dO^T P), so no transposed copy is stored.
//         dS goes through LDS once for dQ = dS K; dQ partials are added to the fp32
//         accumulator with hardware float atomics. dK, dV are summed over the group in a
//         fixed head order and written once.
//   final dQ = scale * accumulator, cast to the output type.
#include "device_common.h"
#include "launch.h"

namespace vtb {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <typename E> constexpr int pad_elems() { return 32 / (int)sizeof(E); }

template <typename E>
__device__ __forceinline__ const E* row_ptr(const void* base, const int64_t* st, int b, int t, int h) {
  return reinterpret_cast<const E*>(base) + (int64_t)b * st[0] + (int64_t)t * st[1] + (int64_t)h * st[2];
}

// Copy `rows` rows of D elements (starting at token t0 of head h) into an LDS tile with
// row stride LD, zero-filling rows at or beyond `tlimit`.
template <typename E, int D, int LD>
__device__ __forceinline__ void stage_rows(E* tile, const void* base, const int64_t* st, int b, int h,
                                           int t0, int rows, int tlimit) {
  constexpr int CH = 16 / (int)sizeof(E);  // elements per 16-byte chunk
  constexpr int CPR = D / CH;
  for (int idx = threadIdx.x; idx < rows * CPR; idx += kThreads) {
    const int r = idx / CPR, c = idx % CPR;
    const int t = t0 + r;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (t < tlimit) val = *reinterpret_cast<const uint4*>(row_ptr<E>(base, st, b, t, h) + c * CH);
    *reinterpret_cast<uint4*>(tile + r * LD + c * CH) = val;
  }
}

// ------------------------------------------------------------------------------ pre-pass
template <typename E, int D, int MODE>
__global__ __launch_bounds__(kThreads) void flash_pre_kernel(AttnParams p) {
  constexpr int QT = 2;                    // 16-row query tiles per wave
  constexpr int BMP = kWaves * QT * 16;    // rows per workgroup
  constexpr int BNP = 64;                  // keys per staged block
  constexpr int NKS = D / 32;
  constexpr int LD = D + pad_elems<E>();
  constexpr bool kNeedS = MODE != PRE_P_GIVEN;
  constexpr bool kNeedDP = MODE != PRE_LSE_ONLY;
  __shared__ __attribute__((aligned(32))) E sK[kNeedS ? BNP * LD : 1];
  __shared__ __attribute__((aligned(32))) E sV[kNeedDP ? BNP * LD : 1];

  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = p.Hq / p.Hkv, kvh = h / G;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  const int q0 = qb * BMP + w * QT * 16;
  const int Tq = p.Tq, Tk = p.Tk, off = Tk - Tq;
  const float sl2 = p.scale * kLog2e;

  frag_t<E> qa[QT][NKS], da[QT][NKS];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int row = q0 + 16 * t + lc;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (kNeedS)
        qa[t][ks] = row < Tq ? load8<E>(row_ptr<E>(p.q, p.sq, b, row, h) + 32 * ks + 8 * lg) : zero8<E>();
      if constexpr (kNeedDP)
        da[t][ks] = row < Tq ? load8<E>(row_ptr<E>(p.dout, p.sdo, b, row, h) + 32 * ks + 8 * lg) : zero8<E>();
    }
  }

  float lse2[QT][4], acc[QT][4], mrun[QT][4], lrun[QT][4], urun[QT][4];
#pragma unroll
  for (int t = 0; t < QT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = q0 + 16 * t + 4 * lg + r;
      lse2[t][r] = (MODE == PRE_LSE_GIVEN && i < Tq) ? p.lse[((int64_t)b * p.Hq + h) * Tq + i] * kLog2e : 0.f;
      acc[t][r] = 0.f;
      mrun[t][r] = -INFINITY;
      lrun[t][r] = 0.f;
      urun[t][r] = 0.f;
    }

  const int last_row = min(Tq, (qb + 1) * BMP) - 1;
  const int kend = p.causal ? min(Tk, last_row + off + 1) : Tk;
  for (int jb = 0; jb < kend; jb += BNP) {
    __syncthreads();
    if constexpr (kNeedS) stage_rows<E, D, LD>(sK, p.k, p.sk, b, kvh, jb, BNP, Tk);
    if constexpr (kNeedDP) stage_rows<E, D, LD>(sV, p.v, p.sv, b, kvh, jb, BNP, Tk);
    __syncthreads();
    f32x4 S[QT][4], dP[QT][4];
#pragma unroll
    for (int t = 0; t < QT; ++t)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        S[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dP[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if constexpr (kNeedS) {
          const frag_t<E> bk = load8<E>(sK + (16 * kt + lc) * LD + 32 * ks + 8 * lg);
#pragma unroll
          for (int t = 0; t < QT; ++t) mma(S[t][kt], qa[t][ks], bk);
        }
        if constexpr (kNeedDP) {
          const frag_t<E> bv = load8<E>(sV + (16 * kt + lc) * LD + 32 * ks + 8 * lg);
#pragma unroll
          for (int t = 0; t < QT; ++t) mma(dP[t][kt], da[t][ks], bv);
        }
      }
#pragma unroll
    for (int t = 0; t < QT; ++t)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = q0 + 16 * t + 4 * lg + r;
          const int j = jb + 16 * kt + lc;
          const bool vis = i < Tq && j < Tk && (!p.causal || j <= i + off);
          if constexpr (MODE == PRE_LSE_GIVEN) {
            const float pr = vis ? exp2f(S[t][kt][r] * sl2 - lse2[t][r]) : 0.f;
            acc[t][r] += pr * dP[t][kt][r];
          } else if constexpr (MODE == PRE_P_GIVEN) {
            const float pr = vis ? p.P[(((int64_t)b * p.Hq + h) * Tq + i) * Tk + j] : 0.f;
            acc[t][r] += pr * dP[t][kt][r];
          } else {
            if (vis) {
              const float s2 = S[t][kt][r] * sl2;
              const float mn = fmaxf(mrun[t][r], s2);
              const float a = exp2f(mrun[t][r] - mn);
              const float e = exp2f(s2 - mn);
              lrun[t][r] = lrun[t][r] * a + e;
              if constexpr (MODE == PRE_LSE_COMPUTE) urun[t][r] = urun[t][r] * a + e * dP[t][kt][r];
              mrun[t][r] = mn;
            }
          }
        }
  }

#pragma unroll
  for (int t = 0; t < QT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = q0 + 16 * t + 4 * lg + r;
      const int64_t ri = ((int64_t)b * p.Hq + h) * Tq + i;
      if constexpr (MODE == PRE_LSE_GIVEN || MODE == PRE_P_GIVEN) {
        const float dsum = group16_sum(acc[t][r]);
        if (lc == 0 && i < Tq) p.dlt[ri] = dsum;
      } else {
        const float M = group16_max(mrun[t][r]);
        const float sc = mrun[t][r] == -INFINITY ? 0.f : exp2f(mrun[t][r] - M);
        const float L = group16_sum(lrun[t][r] * sc);
        if (lc == 0 && i < Tq) {
          p.lse_out[ri] = (M + log2f(L)) * kLn2;
        }
        if constexpr (MODE == PRE_LSE_COMPUTE) {
          const float U = group16_sum(urun[t][r] * sc);
          if (lc == 0 && i < Tq) p.dlt[ri] = U / L;
        }
      }
    }

  if constexpr (MODE != PRE_LSE_ONLY) {
    // zero this workgroup's rows of the dQ accumulator
    constexpr int C4 = D / 4;
    for (int idx = tid; idx < BMP * C4; idx += kThreads) {
      const int r = idx / C4, c = idx % C4;
      const int i = qb * BMP + r;
      if (i < Tq)
        *reinterpret_cast<float4*>(p.dq_acc + (((int64_t)b * Tq + i) * p.Hq + h) * D + 4 * c) =
            make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// ------------------------------------------------------------------------------ main pass
template <typename E, int D, int KW>
constexpr int main_smem_kt_bytes() {
  constexpr int BN = kWaves * 16 * KW;
  constexpr int a = BN * (D + pad_elems<E>()) * (int)sizeof(E);
  constexpr int b = kWaves * 16 * (D + 4) * 4;  // epilogue staging
  return a > b ? a : b;
}

template <typename E, int D, int KW, bool PGIVEN>
__global__ __launch_bounds__(kThreads) void flash_main_kernel(AttnParams p) {
  constexpr int BN = kWaves * 16 * KW;   // keys per workgroup
  constexpr int BM = 32;                 // query rows per iteration
  constexpr int NKS = D / 32;
  constexpr int NDT = D / 16;
  constexpr int NDQ = NDT / 2;           // d tiles of the dQ product per wave
  constexpr int NC = BN / 32;            // key chunks of the dQ product
  constexpr int LD = D + pad_elems<E>();
  constexpr int LDS_S = BN + pad_elems<E>();
  __shared__ __attribute__((aligned(32))) E sQ[BM * LD];
  __shared__ __attribute__((aligned(32))) E sdO[BM * LD];
  __shared__ __attribute__((aligned(32))) E sdS[BM * LDS_S];
  __shared__ __attribute__((aligned(32))) char smem_kt[main_smem_kt_bytes<E, D, KW>()];
  __shared__ float sL[BM], sDl[BM];
  E* sK = reinterpret_cast<E*>(smem_kt);

  const int b = blockIdx.x / p.Hkv, kvh = blockIdx.x % p.Hkv;
  const int kb = blockIdx.y * BN;
  const int G = p.Hq / p.Hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  const int Tq = p.Tq, Tk = p.Tk, off = Tk - Tq;
  const float sl2 = p.scale * kLog2e;

  // K and V rows of this wave as B operands of S = Q K^T and dP = dO V^T.
  frag_t<E> kr[KW][NKS], vr[KW][NKS];
#pragma unroll
  for (int kt = 0; kt < KW; ++kt) {
    const int key = kb + (w * KW + kt) * 16 + lc;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (!PGIVEN)
        kr[kt][ks] = key < Tk ? load8<E>(row_ptr<E>(p.k, p.sk, b, key, kvh) + 32 * ks + 8 * lg) : zero8<E>();
      vr[kt][ks] = key < Tk ? load8<E>(row_ptr<E>(p.v, p.sv, b, key, kvh) + 32 * ks + 8 * lg) : zero8<E>();
    }
  }

  // K columns for dQ = dS K: this wave owns query tile tq and d tiles dq0 .. dq0+NDQ-1.
  stage_rows<E, D, LD>(sK, p.k, p.sk, b, kvh, kb, BN, Tk);
  __syncthreads();
  const int tq = w & 1;
  const int dq0 = (w >> 1) * NDQ;
  frag_t<E> kq[NDQ][NC];
#pragma unroll
  for (int dd = 0; dd < NDQ; ++dd)
#pragma unroll
    for (int c = 0; c < NC; ++c) kq[dd][c] = load_col8(sK, LD, 32 * c + 8 * lg, 32 * c + 8 * lg + 4, 16 * (dq0 + dd));

  f32x4 adV[KW][NDT], adK[KW][NDT];
#pragma unroll
  for (int kt = 0; kt < KW; ++kt)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      adV[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      adK[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const int q_first = p.causal ? max(0, kb - off) : 0;
  for (int hj = 0; hj < G; ++hj) {
    const int h = kvh * G + hj;
    const int64_t rowbase = ((int64_t)b * p.Hq + h) * Tq;
    for (int q0 = (q_first / BM) * BM; q0 < Tq; q0 += BM) {
      __syncthreads();
      stage_rows<E, D, LD>(sQ, p.q, p.sq, b, h, q0, BM, Tq);
      stage_rows<E, D, LD>(sdO, p.dout, p.sdo, b, h, q0, BM, Tq);
      if (tid < BM) {
        const int i = q0 + tid;
        sL[tid] = (!PGIVEN && i < Tq) ? p.lse[rowbase + i] * kLog2e : 0.f;
        sDl[tid] = i < Tq ? p.dlt[rowbase + i] : 0.f;
      }
      __syncthreads();

      f32x4 S[2][KW], dP[2][KW];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kt = 0; kt < KW; ++kt) {
          S[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
          dP[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const frag_t<E> ado = load8<E>(sdO + (16 * t + lc) * LD + 32 * ks + 8 * lg);
#pragma unroll
          for (int kt = 0; kt < KW; ++kt) mma(dP[t][kt], ado, vr[kt][ks]);
          if constexpr (!PGIVEN) {
            const frag_t<E> aq = load8<E>(sQ + (16 * t + lc) * LD + 32 * ks + 8 * lg);
#pragma unroll
            for (int kt = 0; kt < KW; ++kt) mma(S[t][kt], aq, kr[kt][ks]);
          }
        }

      // P and dS; element e of the packed operands is query 16*(e/4) + 4*lg + e%4.
      frag_t<E> pb[KW], sb[KW];
#pragma unroll
      for (int kt = 0; kt < KW; ++kt) {
        const int j = kb + (w * KW + kt) * 16 + lc;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = e >> 2, r = e & 3;
          const int il = 16 * t + 4 * lg + r;
          const int i = q0 + il;
          const bool vis = i < Tq && j < Tk && (!p.causal || j <= i + off);
          float pr;
          if constexpr (PGIVEN)
            pr = vis ? p.P[(rowbase + i) * Tk + j] : 0.f;
          else
            pr = vis ? exp2f(S[t][kt][r] * sl2 - sL[il]) : 0.f;
          const float ds = pr * (dP[t][kt][r] - sDl[il]);
          pb[kt][e] = from_f32<E>(pr);
          sb[kt][e] = from_f32<E>(ds);
          sdS[il * LDS_S + (w * KW + kt) * 16 + lc] = from_f32<E>(ds);
        }
      }

      // dV^T += dO^T P and dK^T += Q^T dS (scale applied at the end)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const frag_t<E> ado = load_col8(sdO, LD, 4 * lg, 16 + 4 * lg, 16 * dt);
        const frag_t<E> aq = load_col8(sQ, LD, 4 * lg, 16 + 4 * lg, 16 * dt);
#pragma unroll
        for (int kt = 0; kt < KW; ++kt) {
          mma(adV[kt][dt], ado, pb[kt]);
          mma(adK[kt][dt], aq, sb[kt]);
        }
      }
      __syncthreads();

      // dQ partial for query tile tq, d tiles dq0..: dS (LDS, row-wise) times K columns.
      f32x4 aq_[NDQ];
#pragma unroll
      for (int dd = 0; dd < NDQ; ++dd) aq_[dd] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const frag_t<E> a = load8<E>(sdS + (16 * tq + lc) * LDS_S + 32 * c + 8 * lg);
#pragma unroll
        for (int dd = 0; dd < NDQ; ++dd) mma(aq_[dd], a, kq[dd][c]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = q0 + 16 * tq + 4 * lg + r;
        if (i < Tq) {
          float* dst = p.dq_acc + (((int64_t)b * Tq + i) * p.Hq + h) * D + 16 * dq0 + lc;
#pragma unroll
          for (int dd = 0; dd < NDQ; ++dd) unsafeAtomicAdd(dst + 16 * dd, aq_[dd][r]);
        }
      }
    }
  }

  // Epilogue: stage each 16-key tile through LDS (transposing d-major accumulators to
  // key-major rows) and write dK = scale * acc, dV = acc with coalesced row stores.
  __syncthreads();
  float* stage = reinterpret_cast<float*>(smem_kt) + w * 16 * (D + 4);
#pragma unroll
  for (int kt = 0; kt < KW; ++kt) {
#pragma unroll
    for (int which = 0; which < 2; ++which) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          stage[lc * (D + 4) + 16 * dt + 4 * lg + r] = which == 0 ? adK[kt][dt][r] * p.scale : adV[kt][dt][r];
      __syncthreads();
      const int kl = lane >> 2;
      const int key = kb + (w * KW + kt) * 16 + kl;
      if (key < Tk) {
        const int64_t* st = which == 0 ? p.sdk : p.sdv;
        void* base = which == 0 ? p.dk : p.dv;
        const int64_t o = (int64_t)b * st[0] + (int64_t)key * st[1] + (int64_t)kvh * st[2];
        const float* src = stage + kl * (D + 4);
        constexpr int PER = D / 4;
        const int c0 = (lane & 3) * PER;
        if (p.out_bf16) {
          __bf16* dst = reinterpret_cast<__bf16*>(base) + o;
#pragma unroll
          for (int c = 0; c < PER; c += 8) {
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (__bf16)src[c0 + c + e];
            *reinterpret_cast<bf16x8*>(dst + c0 + c) = v;
          }
        } else {
          float* dst = reinterpret_cast<float*>(base) + o;
#pragma unroll
          for (int c = 0; c < PER; c += 4)
            *reinterpret_cast<float4*>(dst + c0 + c) =
                make_float4(src[c0 + c], src[c0 + c + 1], src[c0 + c + 2], src[c0 + c + 3]);
        }
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------------------ dQ final
template <typename EO>
__global__ __launch_bounds__(256) void dq_finalize_kernel(const float* __restrict__ acc, EO* __restrict__ dq,
                                                          int B, int Tq, int Hq, int D, int64_t s0, int64_t s1,
                                                          int64_t s2, float scale) {
  const int64_t n4 = (int64_t)B * Tq * Hq * D / 4;
  const int D4 = D / 4;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < n4; idx += (int64_t)gridDim.x * blockDim.x) {
    const int c = idx % D4;
    int64_t rest = idx / D4;
    const int h = rest % Hq;
    rest /= Hq;
    const int t = rest % Tq;
    const int b = rest / Tq;
    const float4 a = reinterpret_cast<const float4*>(acc)[idx];
    EO* dst = dq + b * s0 + t * s1 + h * s2 + 4 * c;
    dst[0] = from_f32<EO>(a.x * scale);
    dst[1] = from_f32<EO>(a.y * scale);
    dst[2] = from_f32<EO>(a.z * scale);
    dst[3] = from_f32<EO>(a.w * scale);
  }
}

template <typename E, int D>
hipError_t pre_dispatch(const AttnParams& p, int mode, hipStream_t s) {
  const dim3 grid((p.Tq + 127) / 128, p.Hq, p.B);
  switch (mode) {
    case PRE_LSE_GIVEN: hipLaunchKernelGGL((flash_pre_kernel<E, D, PRE_LSE_GIVEN>), grid, dim3(kThreads), 0, s, p); break;
    case PRE_LSE_COMPUTE: hipLaunchKernelGGL((flash_pre_kernel<E, D, PRE_LSE_COMPUTE>), grid, dim3(kThreads), 0, s, p); break;
    case PRE_LSE_ONLY: hipLaunchKernelGGL((flash_pre_kernel<E, D, PRE_LSE_ONLY>), grid, dim3(kThreads), 0, s, p); break;
    default: hipLaunchKernelGGL((flash_pre_kernel<E, D, PRE_P_GIVEN>), grid, dim3(kThreads), 0, s, p); break;
  }
  return hipGetLastError();
}

template <typename E, int D, int KW>
hipError_t main_dispatch(const AttnParams& p, hipStream_t s) {
  constexpr int BN = kWaves * 16 * KW;
  // x = (batch, kv-head) so that every head's heaviest (earliest) key block is issued first.
  const dim3 grid(p.B * p.Hkv, (p.Tk + BN - 1) / BN);
  if (p.P)
    hipLaunchKernelGGL((flash_main_kernel<E, D, KW, true>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((flash_main_kernel<E, D, KW, false>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_flash_pre(const AttnParams& p, int mode, hipStream_t s) {
  if (p.in_bf16) return p.D == 128 ? pre_dispatch<__bf16, 128>(p, mode, s) : pre_dispatch<__bf16, 64>(p, mode, s);
  return p.D == 128 ? pre_dispatch<float, 128>(p, mode, s) : pre_dispatch<float, 64>(p, mode, s);
}

hipError_t launch_flash_main(const AttnParams& p, hipStream_t s) {
  if (p.in_bf16) return p.D == 128 ? main_dispatch<__bf16, 128, 2>(p, s) : main_dispatch<__bf16, 64, 2>(p, s);
  return p.D == 128 ? main_dispatch<float, 128, 1>(p, s) : main_dispatch<float, 64, 1>(p, s);
}

hipError_t launch_dq_finalize(const AttnParams& p, hipStream_t s) {
  const int64_t n4 = (int64_t)p.B * p.Tq * p.Hq * p.D / 4;
  const int blocks = (int)std::min<int64_t>((n4 + 255) / 256, 4096);
  if (p.out_bf16)
    hipLaunchKernelGGL((dq_finalize_kernel<__bf16>), dim3(blocks), dim3(256), 0, s, p.dq_acc,
                       reinterpret_cast<__bf16*>(p.dq), p.B, p.Tq, p.Hq, p.D, p.sdq[0], p.sdq[1], p.sdq[2], p.scale);
  else
    hipLaunchKernelGGL((dq_finalize_kernel<float>), dim3(blocks), dim3(256), 0, s, p.dq_acc,
                       reinterpret_cast<float*>(p.dq), p.B, p.Tq, p.Hq, p.D, p.sdq[0], p.sdq[1], p.sdq[2], p.scale);
  return hipGetLastError();
}

}  // namespace vtb
