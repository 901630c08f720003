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
// Two launches, no atomics (results are bitwise reproducible):
//   dq    query-parallel: sweep 1 over the visible keys reduces D_i (and lse_i when it
//         is not given); sweep 2 recomputes S and dP, forms dS and accumulates dQ in
//         registers. Writes dQ and the row term D.
//   dkdv  key-parallel: recomputes S and dP per query block, forms P and dS and
//         accumulates dV = P^T dO and dK = scale dS^T Q in registers.
// S and dP are recomputed once more than a single fused pass would need; in exchange
// there is no cross-workgroup reduction of dQ.
//
// Memory pipeline: every tile is fetched into registers one step ahead with loads that
// are always in bounds (rows past the end are clamped and zeroed when written to LDS),
// so no load sits behind a divergent branch and the wait for it falls at its first use.
// bf16 tiles with 128-element rows use an XOR-swizzled LDS layout that is free of bank
// conflicts both for the row-wise 16-byte operand reads and for the transpose reads.
// Both kernels fit 256 registers per lane for bf16, so two workgroups share a CU.
#include "device_common.h"
#include "launch.h"
#include "lds_tile.h"

namespace vtb {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// A ROWS x D tile of one head held in registers, 16 bytes per chunk, spread over the
// workgroup. load() issues every global load of the tile at once; rows at or beyond
// tlimit (>= 1) read the last valid row instead and are zeroed by store(), which writes
// the tile into LDS layout L.
template <typename E, int D, int ROWS>
struct TileRegs {
  static constexpr int CH = 16 / (int)sizeof(E);
  static constexpr int CPR = D / CH;
  static constexpr int N = ROWS * CPR / kThreads;
  static_assert(ROWS * CPR % kThreads == 0, "tile must spread evenly over the workgroup");
  uint4 v[N];
  uint32_t valid;
  __device__ __forceinline__ void load(const void* base, const int64_t* st, int b, int h, int t0, int tlimit) {
    valid = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = threadIdx.x + i * kThreads;
      const int r = idx / CPR, c = idx % CPR;
      const int t = t0 + r;
      valid |= (uint32_t)(t < tlimit) << i;
      v[i] = *reinterpret_cast<const uint4*>(row_ptr<E>(base, st, b, min(t, tlimit - 1), h) + c * CH);
    }
  }
  template <typename L>
  __device__ __forceinline__ void store(E* tile) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = threadIdx.x + i * kThreads;
      const int r = idx / CPR, c = idx % CPR;
      const bool ok = (valid >> i) & 1u;   // value selects: a select of lvalues would move v[] to scratch
      const uint4 x = make_uint4(ok ? v[i].x : 0u, ok ? v[i].y : 0u, ok ? v[i].z : 0u, ok ? v[i].w : 0u);
      *reinterpret_cast<uint4*>(tile + L::off(r, c * CH)) = x;
    }
  }
};

// ------------------------------------------------------------------------------ dq kernel
// One workgroup = 64 query rows of one q-head (16 per wave). The wave computes the
// transposed score tile S^T = K Q^T (keys as rows), so each lane owns one query column:
// its row statistics are per-lane scalars and dS^T comes out of the MFMA already in the
// operand order of dQ^T += K^T dS^T.
//   sweep 1 over visible keys: D = rowsum(P o dP)  (and lse, when not given)
//   sweep 2 over visible keys: dS = P o (dP - D),  dQ = scale dS K
template <typename E, int D>
constexpr int dq_smem_bytes() {
  constexpr int tiles = 2 * 64 * Lds<E, D>::LD * (int)sizeof(E);   // K and V blocks of 64 keys
  constexpr int stage = kWaves * 16 * (D + 4) * 4;                   // dQ output staging
  return tiles > stage ? tiles : stage;
}

template <typename E, int D, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(E) == 2 ? 2 : 1, sizeof(E) == 2 ? 2 : 1)))
void flash_dq_kernel(AttnParams p) {
  using L = Lds<E, D>;
  constexpr int BM = kWaves * 16;          // query rows per workgroup
  constexpr int BN = 64;                   // keys per staged block
  constexpr int NKS = D / 32, NDT = D / 16;
  constexpr bool kNeedS = MODE != ROW_P_GIVEN;
  constexpr bool kNeedDP = MODE != ROW_LSE_ONLY && MODE != ROW_FWD;
  constexpr bool kNeedV = kNeedDP || MODE == ROW_FWD;   // V staged: dP operand, or P V in the forward
  constexpr bool kOnline = MODE == ROW_LSE_COMPUTE || MODE == ROW_LSE_ONLY;
  __shared__ __attribute__((aligned(32))) char smem[dq_smem_bytes<E, D>()];
  E* sK = reinterpret_cast<E*>(smem);
  E* sV = sK + BN * L::LD;

  const int b = blockIdx.x / p.Hq, h = blockIdx.x % p.Hq;
  const int nqb = (p.Tq + BM - 1) / BM;
  const int qb = nqb - 1 - (int)blockIdx.y;            // causal: heaviest query block first
  const int G = p.Hq / p.Hkv, kvh = h / G;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  const int Tq = p.Tq, Tk = p.Tk, off = Tk - Tq;
  const float sl2 = p.scale * kLog2e;
  const int64_t rowbase = ((int64_t)b * p.Hq + h) * Tq;
  const int qrow = qb * BM + 16 * w + lc;             // this lane's query
  const int qc = min(qrow, Tq - 1);                    // clamped for loads; never written when >= Tq
  const bool qok = qrow < Tq;

  // Q and dO rows of the lane's query: B operands (k = d, n = query) of S^T and dP^T.
  frag_t<E> qa[NKS], da[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if constexpr (kNeedS) qa[ks] = load8<E>(row_ptr<E>(p.q, p.sq, b, qc, h) + 32 * ks + 8 * lg);
    if constexpr (kNeedDP) da[ks] = load8<E>(row_ptr<E>(p.dout, p.sdo, b, qc, h) + 32 * ks + 8 * lg);
  }
  float lrow = (MODE == ROW_LSE_GIVEN || MODE == ROW_D_GIVEN) ? p.lse[rowbase + qc] * kLog2e : 0.f;   // log2 domain

  const int last_row = min(Tq, (qb + 1) * BM) - 1;
  const int kend = p.causal ? min(Tk, last_row + off + 1) : Tk;
  TileRegs<E, D, BN> kt_regs, vt_regs;

  // S^T and dP^T of one staged block: tile kt covers keys jb + 16 kt + 4 lg + r (r = reg).
  auto block_scores = [&](f32x4 (&sT)[4], f32x4 (&dpT)[4]) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sT[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dpT[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (kNeedS) {
        frag_t<E> ak[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) ak[ks] = row8<L>(sK, 16 * kt + lc, 32 * ks + 8 * lg);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) mma(sT[kt], ak[ks], qa[ks]);
      }
      if constexpr (kNeedDP) {
        frag_t<E> av[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) av[ks] = row8<L>(sV, 16 * kt + lc, 32 * ks + 8 * lg);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) mma(dpT[kt], av[ks], da[ks]);
      }
    }
  };
  // Stage key block jb (already in registers) and start fetching block jb + BN.
  auto stage_block = [&](int jb) {
    __syncthreads();
    kt_regs.template store<L>(sK);   // K: S^T operand and, in sweep 2, the dQ operand
    if constexpr (kNeedV) vt_regs.template store<L>(sV);
    __syncthreads();
    if (jb + BN < kend) {
      kt_regs.load(p.k, p.sk, b, kvh, jb + BN, Tk);
      if constexpr (kNeedV) vt_regs.load(p.v, p.sv, b, kvh, jb + BN, Tk);
    }
  };
  auto start_sweep = [&]() {
    if (kend > 0) {
      kt_regs.load(p.k, p.sk, b, kvh, 0, Tk);
      if constexpr (kNeedV) vt_regs.load(p.v, p.sv, b, kvh, 0, Tk);
    }
  };
  // acc^T (lane: d = 16 dt + 4 lg + r of the lane's query) times mult, transposed to
  // query-major rows through LDS, then stored as rows of dq (dQ, or O in the forward).
  auto store_rows = [&](const f32x4 (&accT)[NDT], float mult) {
    __syncthreads();
    float* stage = reinterpret_cast<float*>(smem) + w * 16 * (D + 4);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) stage[lc * (D + 4) + 16 * dt + 4 * lg + r] = accT[dt][r] * mult;
    __syncthreads();
    const int rl = lane >> 2;
    const int qo = qb * BM + 16 * w + rl;
    if (qo < Tq) {
      const int64_t o = (int64_t)b * p.sdq[0] + (int64_t)qo * p.sdq[1] + (int64_t)h * p.sdq[2];
      const float* src = stage + rl * (D + 4);
      constexpr int PER = D / 4;
      const int c0 = (lane & 3) * PER;
      if (p.out_bf16) {
        __bf16* dst = reinterpret_cast<__bf16*>(p.dq) + o;
#pragma unroll
        for (int c = 0; c < PER; c += 8) {
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (__bf16)src[c0 + c + e];
          *reinterpret_cast<bf16x8*>(dst + c0 + c) = v;
        }
      } else {
        float* dst = reinterpret_cast<float*>(p.dq) + o;
#pragma unroll
        for (int c = 0; c < PER; c += 4)
          *reinterpret_cast<float4*>(dst + c0 + c) = make_float4(src[c0 + c], src[c0 + c + 1], src[c0 + c + 2], src[c0 + c + 3]);
      }
    }
  };

  if constexpr (MODE == ROW_FWD) {
    // ---- forward, one sweep with online softmax. Every 16-lane group holds other keys
    // of the lane's query, so each block's maximum is taken over the four groups first:
    // then all of a query's probabilities share one reference and feed one MFMA.
    f32x4 oT[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oT[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;   // log2-domain running maximum; this lane's sum of exponentials
    start_sweep();
    for (int jb = 0; jb < kend; jb += BN) {
      stage_block(jb);
      f32x4 sT[4], dpT[4];
      block_scores(sT, dpT);
      float s2[4][4], bm = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = jb + 16 * kt + 4 * lg + r;
          const bool vis = qok & (j < Tk) & (!p.causal | (j <= qrow + off));
          s2[kt][r] = vis ? sT[kt][r] * sl2 : -INFINITY;
          bm = fmaxf(bm, s2[kt][r]);
        }
      bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
      const float mn = fmaxf(m, bm);
      const float mref = mn == -INFINITY ? 0.f : mn;    // no visible key yet: every term is 0
      const float a = __builtin_amdgcn_exp2f(m - mref);  // 0 while m is -inf
      l *= a;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oT[dt] *= a;
      frag_t<E> pb[2];   // keys 32c + 4lg + (0..3) and 32c + 16 + 4lg + (0..3)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(s2[kt][r] - mref);
          l += e;
          pb[kt >> 1][4 * (kt & 1) + r] = from_f32<E>(e);
        }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) mma(oT[dt], col8<L>(sV, 32 * c + 4 * lg, 32 * c + 16 + 4 * lg, 16 * dt), pb[c]);
      m = mn;
    }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (lg == 0 && qok && p.lse_out) p.lse_out[rowbase + qrow] = (m + log2f(l)) * kLn2;
    store_rows(oT, l > 0.f ? 1.f / l : 0.f);
    return;
  }
  auto prob = [&](float s_t, int j) -> float {   // P of (this lane's query, key j), 0 when invisible
    const bool vis = qok & (j < Tk) & (!p.causal | (j <= qrow + off));
    if constexpr (MODE == ROW_P_GIVEN) {
      const float pv = p.P[(rowbase + qc) * Tk + min(j, Tk - 1)];
      return vis ? pv : 0.f;
    } else {
      const float pe = __builtin_amdgcn_exp2f(s_t * sl2 - lrow);
      return vis ? pe : 0.f;
    }
  };

  // ---- sweep 1: row term D (and lse); with D given, none
  float accd = 0.f, mrun = -INFINITY, lrun = 0.f, urun = 0.f;
  if constexpr (MODE != ROW_D_GIVEN) start_sweep();
  for (int jb = 0; MODE != ROW_D_GIVEN && jb < kend; jb += BN) {
    stage_block(jb);
    f32x4 sT[4], dpT[4];
    block_scores(sT, dpT);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = jb + 16 * kt + 4 * lg + r;
        if constexpr (kOnline) {
          const bool vis = qok & (j < Tk) & (!p.causal | (j <= qrow + off));
          const float s2 = vis ? sT[kt][r] * sl2 : -INFINITY;
          const float mn = fmaxf(mrun, s2);
          const float a = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mrun - mn);
          const float e = vis ? __builtin_amdgcn_exp2f(s2 - mn) : 0.f;
          lrun = lrun * a + e;
          if constexpr (kNeedDP) urun = urun * a + e * dpT[kt][r];
          mrun = mn;
        } else {
          accd += prob(sT[kt][r], j) * dpT[kt][r];
        }
      }
  }
  // combine the four 16-lane groups that hold the same query
  float drow;
  if constexpr (kOnline) {
    float M = fmaxf(mrun, __shfl_xor(mrun, 16, 64));
    M = fmaxf(M, __shfl_xor(M, 32, 64));
    const float sc = mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun - M);
    float Ls = lrun * sc, U = urun * sc;
    Ls += __shfl_xor(Ls, 16, 64);
    Ls += __shfl_xor(Ls, 32, 64);
    U += __shfl_xor(U, 16, 64);
    U += __shfl_xor(U, 32, 64);
    lrow = M + log2f(Ls);
    drow = U / Ls;
    if (lg == 0 && qok) p.lse_out[rowbase + qrow] = lrow * kLn2;
  } else if constexpr (MODE == ROW_D_GIVEN) {
    // D = dO . O: the lane's dO pieces (d = 32 ks + 8 lg + e) against the same pieces of O,
    // then the four 16-lane groups that hold the row
    drow = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const frag_t<E> o8 = load8<E>(row_ptr<E>(p.o, p.so, b, qc, h) + 32 * ks + 8 * lg);
#pragma unroll
      for (int e = 0; e < 8; ++e) drow = fmaf(to_f32(da[ks][e]), to_f32(o8[e]), drow);
    }
    drow += __shfl_xor(drow, 16, 64);
    drow += __shfl_xor(drow, 32, 64);
  } else {
    drow = accd + __shfl_xor(accd, 16, 64);
    drow += __shfl_xor(drow, 32, 64);
  }
  if constexpr (MODE == ROW_LSE_ONLY) {
    return;
  } else {
    if (lg == 0 && qok) p.dlt[rowbase + qrow] = drow;

    // ---- sweep 2: dQ^T += K^T dS^T
    f32x4 dqT[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dqT[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    start_sweep();
    for (int jb = 0; jb < kend; jb += BN) {
      stage_block(jb);
      f32x4 sT[4], dpT[4];
      block_scores(sT, dpT);
      frag_t<E> dsb[2];   // keys 32c + 4lg + (0..3) and 32c + 16 + 4lg + (0..3)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = jb + 16 * kt + 4 * lg + r;
          const float ds = prob(sT[kt][r], j) * (dpT[kt][r] - drow);
          dsb[kt >> 1][4 * (kt & 1) + r] = from_f32<E>(ds);
        }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) mma(dqT[dt], col8<L>(sK, 32 * c + 4 * lg, 32 * c + 16 + 4 * lg, 16 * dt), dsb[c]);
    }

    // dQ = scale dQ^T
    store_rows(dqT, p.scale);
  }
}

// ------------------------------------------------------------------------------ dkdv kernel
// One workgroup = 64 keys of one kv-head (16 per wave); it walks every query block (of
// every q-head of the group) that sees them. K and V rows of the wave are B operands in
// registers; Q and dO tiles go through LDS and are read row-wise (S, dP) and through
// the LDS transpose read (dV^T += dO^T P, dK^T += Q^T dS). dK, dV are summed over the
// group in a fixed head order and written once.
template <typename E, int D>
constexpr int dkdv_stage_bytes() {
  return kWaves * 16 * (D + 4) * 4;
}

template <typename E, int D, bool PGIVEN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(E) == 2 ? 2 : 1, sizeof(E) == 2 ? 2 : 1)))
void flash_dkdv_kernel(AttnParams p) {
  constexpr int BN = kWaves * 16;        // keys per workgroup
  constexpr int BM = 32;                 // query rows per iteration
  constexpr int NKS = D / 32;
  constexpr int NDT = D / 16;
  using LQ = Lds<E, D>;
  constexpr int QBYTES = BM * LQ::LD * (int)sizeof(E);
  constexpr int SMEM = 2 * QBYTES > dkdv_stage_bytes<E, D>() ? 2 * QBYTES : dkdv_stage_bytes<E, D>();
  __shared__ __attribute__((aligned(32))) char smem[SMEM];
  __shared__ __attribute__((aligned(16))) float sL[BM], sDl[BM];
  E* sQ = reinterpret_cast<E*>(smem);
  E* sdO = reinterpret_cast<E*>(smem + QBYTES);

  const int b = blockIdx.x / p.Hkv, kvh = blockIdx.x % p.Hkv;
  const int kb = blockIdx.y * BN;
  const int G = p.Hq / p.Hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
  const int Tq = p.Tq, Tk = p.Tk, off = Tk - Tq;
  const float sl2 = p.scale * kLog2e;
  const int jl = 16 * w + lc;            // this lane's key within the block
  const int j = kb + jl;
  const int jc = min(j, Tk - 1);

  // K and V rows of this wave as B operands of S = Q K^T and dP = dO V^T.
  frag_t<E> kr[NKS], vr[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if constexpr (!PGIVEN) {
      kr[ks] = load8<E>(row_ptr<E>(p.k, p.sk, b, jc, kvh) + 32 * ks + 8 * lg);
      if (j >= Tk) kr[ks] = zero8<E>();
    }
    vr[ks] = load8<E>(row_ptr<E>(p.v, p.sv, b, jc, kvh) + 32 * ks + 8 * lg);
    if (j >= Tk) vr[ks] = zero8<E>();
  }

  f32x4 adV[NDT], adK[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    adV[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    adK[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int q_first = p.causal ? max(0, kb - off) : 0;
  const int qb0 = q_first / BM;
  const int nqb = (Tq + BM - 1) / BM - qb0;       // query blocks per head that see this key block
  const int n_it = nqb > 0 ? G * nqb : 0;
  TileRegs<E, D, BM> q_regs, do_regs;
  float l_reg = 0.f, d_reg = 0.f;
  auto prefetch = [&](int h, int q0) {
    q_regs.load(p.q, p.sq, b, h, q0, Tq);
    do_regs.load(p.dout, p.sdo, b, h, q0, Tq);
    const int i = min(q0 + (tid & (BM - 1)), Tq - 1);   // in bounds for every thread
    const int64_t rb = ((int64_t)b * p.Hq + h) * Tq;
    if constexpr (!PGIVEN) l_reg = p.lse[rb + i];   // scaled by log2(e) when staged: a use
    d_reg = p.dlt[rb + i];                          // right after the load would wait for it
  };
  // (head, query block) of the current and next iteration, advanced without division
  int h = kvh * G, q0 = qb0 * BM;
  int hn = h, q0n = q0 + BM;
  if (q0n >= Tq) {
    q0n = qb0 * BM;
    ++hn;
  }
  if (n_it > 0) prefetch(h, q0);
  for (int it = 0; it < n_it; ++it) {
    const int64_t rowbase = ((int64_t)b * p.Hq + h) * Tq;
    __syncthreads();
    q_regs.template store<LQ>(sQ);
    do_regs.template store<LQ>(sdO);
    if (tid < BM) {
      sL[tid] = l_reg * kLog2e;
      sDl[tid] = d_reg;
    }
    __syncthreads();
    if (it + 1 < n_it) prefetch(hn, q0n);

    // S = Q K^T and dP = dO V^T for this wave's 16 keys (rows: 32 queries)
    f32x4 S[2], dP[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      frag_t<E> ado[NKS], aq[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        ado[ks] = row8<LQ>(sdO, 16 * t + lc, 32 * ks + 8 * lg);
        if constexpr (!PGIVEN) aq[ks] = row8<LQ>(sQ, 16 * t + lc, 32 * ks + 8 * lg);
      }
      dP[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        mma(dP[t], ado[ks], vr[ks]);
        if constexpr (!PGIVEN) mma(S[t], aq[ks], kr[ks]);
      }
    }

    // P and dS; element e of the packed operands is query 16*(e/4) + 4*lg + e%4.
    const f32x4 L0 = *reinterpret_cast<const f32x4*>(sL + 4 * lg);
    const f32x4 L1 = *reinterpret_cast<const f32x4*>(sL + 16 + 4 * lg);
    const f32x4 D0 = *reinterpret_cast<const f32x4*>(sDl + 4 * lg);
    const f32x4 D1 = *reinterpret_cast<const f32x4*>(sDl + 16 + 4 * lg);
    const bool full = q0 + BM <= Tq && kb + BN <= Tk && (!p.causal || kb + BN - 1 <= q0 + off);
    frag_t<E> pb, sb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = e >> 2, r = e & 3;
      const int i = q0 + 16 * t + 4 * lg + r;
      const float lrow = t ? L1[r] : L0[r];
      const float drow = t ? D1[r] : D0[r];
      float pr;
      if constexpr (PGIVEN) {
        const bool vis = (i < Tq) & (j < Tk) & (!p.causal | (j <= i + off));
        const float pv = p.P[(rowbase + min(i, Tq - 1)) * Tk + jc];
        pr = vis ? pv : 0.f;
      } else {
        pr = __builtin_amdgcn_exp2f(S[t][r] * sl2 - lrow);
        if (!full) {
          const bool vis = (i < Tq) & (j < Tk) & (!p.causal | (j <= i + off));
          pr = vis ? pr : 0.f;
        }
      }
      pb[e] = from_f32<E>(pr);
      sb[e] = from_f32<E>(pr * (dP[t][r] - drow));
    }

    // dV^T += dO^T P and dK^T += Q^T dS (scale applied at the end)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      mma(adV[dt], col8<LQ>(sdO, 4 * lg, 16 + 4 * lg, 16 * dt), pb);
      mma(adK[dt], col8<LQ>(sQ, 4 * lg, 16 + 4 * lg, 16 * dt), sb);
    }

    h = hn;
    q0 = q0n;
    q0n += BM;
    if (q0n >= Tq) {
      q0n = qb0 * BM;
      ++hn;
    }
  }

  // Epilogue: stage the wave's 16 keys through LDS (d-major accumulators to key-major
  // rows) and write dK = scale * acc, dV = acc with row stores.
  float* stage = reinterpret_cast<float*>(smem) + w * 16 * (D + 4);
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    __syncthreads();
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        stage[lc * (D + 4) + 16 * dt + 4 * lg + r] = which == 0 ? adK[dt][r] * p.scale : adV[dt][r];
    __syncthreads();
    const int kl = lane >> 2;
    const int key = kb + 16 * w + kl;
    void* base = which == 0 ? p.dk : p.dv;   // null: that gradient is not wanted
    if (key < Tk && base) {
      const int64_t* st = which == 0 ? p.sdk : p.sdv;
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
          *reinterpret_cast<float4*>(dst + c0 + c) = make_float4(src[c0 + c], src[c0 + c + 1], src[c0 + c + 2], src[c0 + c + 3]);
      }
    }
  }
}

template <typename E, int D>
hipError_t dq_dispatch(const AttnParams& p, int mode, hipStream_t s, KernelEvents ev) {
  const dim3 grid(p.B * p.Hq, (p.Tq + kWaves * 16 - 1) / (kWaves * 16));
  switch (mode) {
    case ROW_LSE_GIVEN: launch_kernel(flash_dq_kernel<E, D, ROW_LSE_GIVEN>, grid, dim3(kThreads), 0, s, ev, p); break;
    case ROW_LSE_COMPUTE: launch_kernel(flash_dq_kernel<E, D, ROW_LSE_COMPUTE>, grid, dim3(kThreads), 0, s, ev, p); break;
    case ROW_LSE_ONLY: launch_kernel(flash_dq_kernel<E, D, ROW_LSE_ONLY>, grid, dim3(kThreads), 0, s, ev, p); break;
    case ROW_FWD: launch_kernel(flash_dq_kernel<E, D, ROW_FWD>, grid, dim3(kThreads), 0, s, ev, p); break;
    case ROW_D_GIVEN: launch_kernel(flash_dq_kernel<E, D, ROW_D_GIVEN>, grid, dim3(kThreads), 0, s, ev, p); break;
    default: launch_kernel(flash_dq_kernel<E, D, ROW_P_GIVEN>, grid, dim3(kThreads), 0, s, ev, p); break;
  }
  return hipGetLastError();
}

template <typename E, int D>
hipError_t dkdv_dispatch(const AttnParams& p, hipStream_t s, KernelEvents ev) {
  constexpr int BN = kWaves * 16;
  // x = (batch, kv-head) so that every head's heaviest (earliest) key block is issued first.
  const dim3 grid(p.B * p.Hkv, (p.Tk + BN - 1) / BN);
  if (p.P)
    launch_kernel(flash_dkdv_kernel<E, D, true>, grid, dim3(kThreads), 0, s, ev, p);
  else
    launch_kernel(flash_dkdv_kernel<E, D, false>, grid, dim3(kThreads), 0, s, ev, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_flash_dq(const AttnParams& p, int mode, hipStream_t s, KernelEvents ev) {
  if (p.in_bf16) return p.D == 128 ? dq_dispatch<__bf16, 128>(p, mode, s, ev) : dq_dispatch<__bf16, 64>(p, mode, s, ev);
  return p.D == 128 ? dq_dispatch<float, 128>(p, mode, s, ev) : dq_dispatch<float, 64>(p, mode, s, ev);
}

hipError_t launch_flash_dkdv(const AttnParams& p, hipStream_t s, KernelEvents ev) {
  if (p.in_bf16) return p.D == 128 ? dkdv_dispatch<__bf16, 128>(p, s, ev) : dkdv_dispatch<__bf16, 64>(p, s, ev);
  return p.D == 128 ? dkdv_dispatch<float, 128>(p, s, ev) : dkdv_dispatch<float, 64>(p, s, ev);
}

}  // namespace vtb
