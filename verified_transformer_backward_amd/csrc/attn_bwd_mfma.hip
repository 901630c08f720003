// Attention backward for bf16 inputs with head dim 128: MFMA tiles fed by direct-to-LDS
// loads, double-buffered, one barrier per block.
//
// Same chain as attn_flash_bwd.hip ("Hesper.Training.VerifiedBackward", section
// "Attention (full single-head)", with the causal mask of the DaisyChain-Train
// transformer.js `backward`), laid out for gfx950's matrix cores:
//
//   dq    query-parallel, ONE sweep over the visible keys. With P = exp(S - lse) known
//         from the saved lse, dS = P o (dP - D) gives
//             dQ = scale (sum_j (P o dP)_ij k_j  -  D_i sum_j P_ij k_j),
//         so the sweep accumulates A = (P o dP) K, B = P K and D = rowsum(P o dP)
//         together and forms dQ = scale (A - D B) at the end: four contractions per
//         key block instead of two sweeps of five. Writes dQ and D.
//         The D used for dQ sums the same bf16-rounded (P o dP) values that enter A, so
//         the rounding of each term cancels against B: dQ_i carries errors
//         delta_ij (k_j - B_i) rather than delta_ij k_j, and a row whose dS vanishes
//         (a single visible key) gets dQ = 0 exactly. The D written for the dk/dv pass
//         is the fp32 sum, exact enough that dS = P o (dP - D) vanishes there too.
//         Also writes lse * log2(e) per row, so that the dk/dv pass forms P = exp2(...)
//         without a multiply per element.
//   dkdv  key-parallel over query blocks (of every q-head of the kv-head's group):
//         S, dP, then dV += P^T dO and dK += dS^T Q with dS = P o (dP - D), D from dq.
//
// A wave owns NT 16-row MFMA tiles of queries (dq) or keys (dkdv); every operand
// fragment it reads from LDS feeds NT MFMAs. K/V (dq) and Q/dO (dkdv) blocks of 64 rows
// are double buffered: the direct-to-LDS loads of the next block run under the current
// block's MFMAs, and one barrier per block both publishes the new block and retires the
// old one. Rows past the end of a tensor re-read its last row, so values stay finite and
// every use of them is masked; no load needs a bounds branch. Blocks that need no mask
// run a branch-free body. The LDS layout is the swizzled one of lds_tile.h, free of bank
// conflicts for the row reads, the transpose reads and the direct-to-LDS writes.
#include "device_common.h"
#include "launch.h"
#include "lds_tile.h"

#include <type_traits>

namespace vtb {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kHD = 128;        // head dim
constexpr int kNKS = kHD / 32;  // 32-deep k steps over the head dim
constexpr int kNDT = kHD / 16;  // 16-wide tiles over the head dim
constexpr int kRows = 64;       // rows per staged block
using LT = Lds<__bf16, kHD>;

#ifndef VTB_MFMA_TILES          // 16-row MFMA tiles per wave
#define VTB_MFMA_TILES 1
#endif
#ifndef VTB_MFMA_WAVES          // waves per workgroup
#define VTB_MFMA_WAVES 4
#endif
constexpr int kNT = VTB_MFMA_TILES;
constexpr int kW = VTB_MFMA_WAVES;
constexpr int kT = 64 * kW;
constexpr int kWavesPerEU = kNT == 1 ? 2 : 1;   // register budget: 256 or 512 per lane
// Two staged blocks: the loads of block j + 1 run under block j's MFMAs. The block loops
// are unrolled by two so that every LDS address is a per-lane base plus a constant.
template <int B>
using BufC = std::integral_constant<int, B>;

// Which (row, rank) a workgroup works on. Rows are gridDim.x (batch x head), ranks are the
// gridDim.y blocks of a row, rank 0 the heaviest under the causal mask. The hardware hands
// consecutive linear workgroup ids to the 8 XCDs in turn. With few blocks per row, every
// XCD takes its share of all rows, heaviest rank first across rows (the launch order).
// With many, each XCD takes a contiguous range of rows (items j = row * nb + rank), the
// heaviest rank first within a row, so that the few rows one XCD works on at a time share
// its L2: every workgroup of a row streams the same K/V (or Q/dO) blocks, and at long
// sequences the rows of all heads an XCD would otherwise interleave do not fit in it.
constexpr int kXcds = 8, kXcdOrderMinBlocks = 32;
__device__ __forceinline__ void grid_item(int& row, int& rank) {
  const int R = gridDim.x, nb = gridDim.y;
  if (nb < kXcdOrderMinBlocks) {
    row = blockIdx.x;
    rank = blockIdx.y;
    return;
  }
  const int L = (int)blockIdx.y * R + (int)blockIdx.x, N = R * nb;
  const int x = L % kXcds, k = L / kXcds, q = N / kXcds, r = N % kXcds;
  const int j = x * q + min(x, r) + k;   // XCD x owns items [x q + min(x, r), ... + q + (x < r))
  row = j / nb;
  rank = j % nb;
}
static_assert(kW == 4 || kW == 8, "64-row tiles are staged four rows per load by every wave");

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// s_waitcnt vmcnt(0): every vector-memory load of the wave, the direct-to-LDS ones
// included, has landed. A real waitcnt instruction, so the compiler also knows that its
// own earlier loads are complete and adds no waits for them inside the block loops.
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Scheduling fence: keeps the issue order of the operand-read groups written around it,
// so LDS reads run ahead of the MFMAs that consume them.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// Issue priority of the wave: raised over each run of MFMAs and lowered for the softmax
// arithmetic between them, so that of the two waves sharing a SIMD the one with matrix
// work ready issues it first and the other's vector work fills in around it.
// Transposed operand fragments read ahead of their MFMAs in the (P o dP)K / PK (dq) and
// dO^T P / Q^T dS (dk/dv) loops.
#ifndef VTB_DQ_AHEAD
#define VTB_DQ_AHEAD 4
#endif
#ifndef VTB_DKDV_AHEAD
#define VTB_DKDV_AHEAD 3
#endif
#ifndef VTB_MFMA_SETPRIO
#define VTB_MFMA_SETPRIO 1
#endif
__device__ __forceinline__ void prio_mfma() {
  if (VTB_MFMA_SETPRIO) __builtin_amdgcn_s_setprio(1);
}
__device__ __forceinline__ void prio_valu() {
  if (VTB_MFMA_SETPRIO) __builtin_amdgcn_s_setprio(0);
}

// Direct-to-LDS loads, issued through inline assembly. Each lane reads `bytes` bytes at
// sbase + voff (sbase wave-uniform) and writes them to LDS at m0 + lane * bytes. Written
// as assembly so that the compiler does not treat the asynchronous LDS write as aliasing
// every later LDS read (it would then wait for the load before each block's reads); the
// order is kept explicitly instead: wait_loads() + __syncthreads() before any read of a
// staged buffer, and a buffer is refilled only after the barrier that retires it. The
// s_nop covers the one wait state gfx9 needs between writing M0 and an LDS DMA.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)p);
}
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}

// Direct-to-LDS staging of 64 rows of one head into a swizzled 64 x 128 tile. Wave w
// writes rows RPW w .. RPW w + RPW - 1, four rows (1 KB) per load: lane l lands at
// physical chunk l % 16 of row 4i + l / 16 and so fetches the logical chunk the swizzle
// keeps there. The lane's byte offsets from the block's first row are fixed for the
// whole kernel (the row stride is), so a full block costs one 64-bit row address and,
// per load, a scalar add for M0.
struct RowStager {
  static constexpr int RPW = kRows / kW;
  static constexpr int NI = RPW / 4;
  uint32_t voff[NI];   // byte offset of the lane's 16 bytes for load i, from row t0
  int w;
  __device__ __forceinline__ void init(int wave, int64_t tstride) {
    w = wave;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = RPW * w + 4 * i + (lane >> 4);
      voff[i] = 2u * (uint32_t)(row * (int)tstride + 8 * ((lane & 15) ^ LT::chunk_xor(row)));
    }
  }
  // Rows [t0, t0 + 64) of `head` (row t at head + t * tstride) into the tile at LDS byte
  // address `tile`; rows >= tlimit read row tlimit - 1.
  __device__ __forceinline__ void stage(uint32_t tile, const __bf16* head, int64_t tstride, int t0, int tlimit) const {
    const __bf16* row0 = head + (int64_t)t0 * tstride;
    const uint32_t dst = tile + 2u * (uint32_t)(RPW * w * kHD);
    if (t0 + kRows <= tlimit) {
#pragma unroll
      for (int i = 0; i < NI; ++i) dma16(row0, voff[i], dst + 2u * (uint32_t)(4 * i * kHD));
    } else {
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int row = RPW * w + 4 * i + (lane >> 4);
        const int t = min(t0 + row, tlimit - 1) - t0;   // 0 .. 63
        const uint32_t vo = 2u * (uint32_t)(t * (int)tstride + 8 * ((lane & 15) ^ LT::chunk_xor(row)));
        dma16(row0, vo, dst + 2u * (uint32_t)(4 * i * kHD));
      }
    }
  }
};

// 64 consecutive fp32 values src[i0 .. i0 + 63] (indices clamped to n - 1) into LDS at
// byte address dst, one direct-to-LDS dword per lane; called by a single wave.
__device__ __forceinline__ void stage_vals64(uint32_t dst, const float* src, int i0, int n) {
  const int lane = threadIdx.x & 63;
  dma4(src + i0, 4u * (uint32_t)(min(i0 + lane, n - 1) - i0), dst);
}

// Four consecutive output elements (fp32 or bf16 RNE).
__device__ __forceinline__ void store4(void* base, int bf16, int64_t off, float a, float b, float c, float d) {
  if (bf16) {
    bf16x4 v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
    *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(base) + off) = v;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + off) = make_float4(a, b, c, d);
  }
}

// ------------------------------------------------------------------------------ dq
// Workgroup: kW * 16 * kNT query rows of one q-head; wave w owns kNT 16-row tiles
// starting at qw0. Per 64-key block the wave computes S^T = K Q^T and dP^T = V dO^T
// (keys as MFMA rows, so a lane owns one query column and its row sums stay in the
// lane), then A^T += K^T (P o dP)^T and B^T += K^T P^T with K^T from LDS transpose reads.
// DG (the forward's saved O given): D = dO . O from the rows loaded below, written to dlt
// for the dk/dv pass; the sweep accumulates A^T += K^T (P o (dP - D))^T only and dQ = scale A.
template <bool DG>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(kWavesPerEU, kWavesPerEU)))
void dq_mfma_kernel(AttnParams p) {
  constexpr int BN = kRows, QW = 16 * kNT, BM = kW * QW;
  __shared__ __attribute__((aligned(1024))) __bf16 sm[2][2][BN * kHD];   // [buffer][K, V]

  int row, rank;
  grid_item(row, rank);
  const int b = row / p.Hq, h = row % p.Hq;
  const int nqb = (p.Tq + BM - 1) / BM;
  const int qb = nqb - 1 - rank;   // causal: heaviest query block first
  const int G = p.Hq / p.Hkv, kvh = h / G;
  const int w = wave_id(), lane = threadIdx.x & 63, lg = lane >> 4, lc = lane & 15;
  const int Tq = p.Tq, Tk = p.Tk, off = Tk - Tq;
  const float sl2 = p.scale * kLog2e;
  const int64_t rowbase = ((int64_t)b * p.Hq + h) * Tq;
  const int qw0 = qb * BM + QW * w;

  const __bf16* Qh = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.sq[0] + (int64_t)h * p.sq[2];
  const __bf16* Oh = reinterpret_cast<const __bf16*>(p.dout) + (int64_t)b * p.sdo[0] + (int64_t)h * p.sdo[2];
  const __bf16* Kh = reinterpret_cast<const __bf16*>(p.k) + (int64_t)b * p.sk[0] + (int64_t)kvh * p.sk[2];
  const __bf16* Vh = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.sv[0] + (int64_t)kvh * p.sv[2];

  // Q and dO of the lane's queries: B operands (k = d, n = query) of S^T and dP^T.
  bf16x8 qa[kNT][kNKS], da[kNT][kNKS];
  float lse2[kNT], dg[kNT];
#pragma unroll
  for (int qt = 0; qt < kNT; ++qt) {
    const int i = min(qw0 + 16 * qt + lc, Tq - 1);
#pragma unroll
    for (int ks = 0; ks < kNKS; ++ks) {
      qa[qt][ks] = load8<__bf16>(Qh + (int64_t)i * p.sq[1] + 32 * ks + 8 * lg);
      da[qt][ks] = load8<__bf16>(Oh + (int64_t)i * p.sdo[1] + 32 * ks + 8 * lg);
    }
    lse2[qt] = p.lse[rowbase + i] * kLog2e;
    dg[qt] = 0.f;
    if constexpr (DG) {
      const __bf16* Oo = reinterpret_cast<const __bf16*>(p.o) + (int64_t)b * p.so[0] + (int64_t)i * p.so[1] +
                         (int64_t)h * p.so[2];
#pragma unroll
      for (int ks = 0; ks < kNKS; ++ks) {
        const bf16x8 o8 = load8<__bf16>(Oo + 32 * ks + 8 * lg);
#pragma unroll
        for (int e = 0; e < 8; ++e) dg[qt] = fmaf((float)da[qt][ks][e], (float)o8[e], dg[qt]);
      }
      dg[qt] += __shfl_xor(dg[qt], 16, 64);   // the four 16-lane groups hold the row's pieces
      dg[qt] += __shfl_xor(dg[qt], 32, 64);
    }
  }

  f32x4 acA[kNDT][kNT], acB[kNDT][kNT];
#pragma unroll
  for (int dt = 0; dt < kNDT; ++dt)
#pragma unroll
    for (int qt = 0; qt < kNT; ++qt) {
      acA[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
      acB[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  float dsum[kNT], dsum_r[kNT];   // D from fp32 P o dP, and from its bf16 rounding
#pragma unroll
  for (int qt = 0; qt < kNT; ++qt) dsum[qt] = dsum_r[qt] = 0.f;

  const int last_row = min(Tq, (qb + 1) * BM) - 1;
  const int kend = p.causal ? min(Tk, last_row + off + 1) : Tk;
  const int nblk = (kend + BN - 1) / BN;
  // keys this wave needs: none when its rows start past Tq
  const int wkend = qw0 >= Tq ? 0 : (p.causal ? min(Tk, min(Tq - 1, qw0 + QW - 1) + off + 1) : Tk);

  RowStager kst, vst;
  kst.init(w, p.sk[1]);
  vst.init(w, p.sv[1]);
  // The register loads above complete before any direct-to-LDS load is issued, so the
  // compiler needs no waits for them inside the loop (it does not see the LDS loads).
  wait_loads();
  const uint32_t sm_lds = lds_addr(&sm[0][0][0]);
  constexpr uint32_t kTileBytes = 2u * BN * kHD;
  if (nblk > 0) {
    kst.stage(sm_lds, Kh, p.sk[1], 0, Tk);
    vst.stage(sm_lds + kTileBytes, Vh, p.sv[1], 0, Tk);
  }

  auto block = [&](auto buf_c, int jb, bool full, auto&& dma) {
    const __bf16* sK = sm[decltype(buf_c)::value][0];
    const __bf16* sV = sm[decltype(buf_c)::value][1];
    // S^T, dP^T: tile kt holds keys jb + 16 kt + 4 lg + r (reg r) for query column lc.
    // The K and V row fragments of tile kt + 1 are read while tile kt's MFMAs run.
    f32x4 sT[4][kNT], dT[4][kNT];
    bf16x8 fk[2][kNKS], fv[2][kNKS];
    auto read_rows = [&](int kt, bf16x8(&ak)[kNKS], bf16x8(&av)[kNKS]) {
#pragma unroll
      for (int ks = 0; ks < kNKS; ++ks) {
        ak[ks] = row8<LT>(sK, 16 * kt + lc, 32 * ks + 8 * lg);
        av[ks] = row8<LT>(sV, 16 * kt + lc, 32 * ks + 8 * lg);
      }
    };
    prio_mfma();
    read_rows(0, fk[0], fv[0]);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      if (kt + 1 < 4) read_rows(kt + 1, fk[(kt + 1) & 1], fv[(kt + 1) & 1]);
      if (kt == 0 || kt == 2) dma(kt >> 1);
      fence();
#pragma unroll
      for (int qt = 0; qt < kNT; ++qt) {
        sT[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dT[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kNKS; ++ks) {
          mma(sT[kt][qt], fk[kt & 1][ks], qa[qt][ks]);
          mma(dT[kt][qt], fv[kt & 1][ks], da[qt][ks]);
        }
      }
      fence();
    }
    prio_valu();
    // K^T fragments of the first (dt, c) pairs are read under the softmax arithmetic.
    constexpr int NP = kNDT * 2, AHEAD = VTB_DQ_AHEAD;
    bf16x8 kT[AHEAD + 1];
    auto read_kT = [&](int pr) { return col8<LT>(sK, 32 * (pr & 1) + 4 * lg, 32 * (pr & 1) + 16 + 4 * lg, 16 * (pr >> 1)); };
#pragma unroll
    for (int pr = 0; pr < AHEAD; ++pr) kT[pr] = read_kT(pr);
    fence();
    // P and P o dP as bf16 B operands (k = 32 keys, n = query): element e of operand c
    // is key 32c + 4 lg + e (e < 4) or 32c + 16 + 4 lg + e - 4 (e >= 4).
    // Only blocks that cross the diagonal or the end of the keys are masked; the branch
    // covers just the masking, so both kinds of block share registers and MFMA code.
    float pe[4][kNT][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qt = 0; qt < kNT; ++qt)
#pragma unroll
        for (int r = 0; r < 4; ++r) pe[kt][qt][r] = __builtin_amdgcn_exp2f(sT[kt][qt][r] * sl2 - lse2[qt]);
    if (!full) {
      asm volatile("");   // keeps the masking inside the branch (no speculation into full blocks)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int qt = 0; qt < kNT; ++qt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int jj = jb + 16 * kt + 4 * lg + r, i = qw0 + 16 * qt + lc;
            pe[kt][qt][r] = ((jj < Tk) & (!p.causal | (jj <= i + off))) ? pe[kt][qt][r] : 0.f;
          }
    }
    bf16x8 pb[2][kNT], xb[2][kNT];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qt = 0; qt < kNT; ++qt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pr = pe[kt][qt][r];
          const float x = DG ? pr * (dT[kt][qt][r] - dg[qt]) : pr * dT[kt][qt][r];
          dsum[qt] += x;
          pb[kt >> 1][qt][4 * (kt & 1) + r] = (__bf16)pr;
          xb[kt >> 1][qt][4 * (kt & 1) + r] = (__bf16)x;
        }
    // The rounded sum, two terms per instruction: each bf16 pair dotted with (1, 1).
    if constexpr (!DG) {
      const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int qt = 0; qt < kNT; ++qt) {
          const bf16x8 x8 = xb[c][qt];
          float t = dsum_r[qt];
          t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x8, x8, 0, 1), one2, t, false);
          t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x8, x8, 2, 3), one2, t, false);
          t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x8, x8, 4, 5), one2, t, false);
          t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x8, x8, 6, 7), one2, t, false);
          dsum_r[qt] = t;
        }
    }
    fence();
    prio_mfma();
    // A^T += K^T (P o dP)^T,  B^T += K^T P^T over (dt, c) pairs, reads AHEAD pairs ahead
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
      if (pr + AHEAD < NP) kT[(pr + AHEAD) % (AHEAD + 1)] = read_kT(pr + AHEAD);
      if (pr == 0 || pr == NP / 2) dma(2 + (pr != 0));
      fence();
      const int dt = pr >> 1, c = pr & 1;
#pragma unroll
      for (int qt = 0; qt < kNT; ++qt) {
        mma(acA[dt][qt], kT[pr % (AHEAD + 1)], xb[c][qt]);
        if constexpr (!DG) mma(acB[dt][qt], kT[pr % (AHEAD + 1)], pb[c][qt]);
      }
      fence();
    }
    prio_valu();
  };

  // Block j sits in buffer j % 2. After the barrier every wave has finished block j - 1,
  // so the loads of block j + 1 go to its buffer right away, ahead of block j's MFMAs.
  auto iteration = [&](int j, auto buf_c) {
    constexpr int nxt = decltype(buf_c)::value ^ 1;
    const int jb = j * BN;
    wait_loads();
    __syncthreads();   // block j is in LDS; every wave is done with block j - 1
    const bool more = j + 1 < nblk;
    auto dma = [&](int part) {
      if (!more || part != 0) return;
      kst.stage(sm_lds + (2 * nxt) * kTileBytes, Kh, p.sk[1], jb + BN, Tk);
      vst.stage(sm_lds + (2 * nxt + 1) * kTileBytes, Vh, p.sv[1], jb + BN, Tk);
    };
    if (jb >= wkend) {
      dma(0);
      return;
    }
    const bool full = jb + BN <= Tk && (!p.causal || jb + BN - 1 <= qw0 + off);
    block(buf_c, jb, full, dma);
  };
  int j = 0;
  for (; j + 1 < nblk; j += 2) {
    iteration(j, BufC<0>{});
    iteration(j + 1, BufC<1>{});
  }
  if (j < nblk) iteration(j, BufC<0>{});

  // D of the lane's queries: the four 16-lane groups hold disjoint key subsets.
  float Dq[kNT];
#pragma unroll
  for (int qt = 0; qt < kNT; ++qt) {
    float d = dsum[qt], dr = dsum_r[qt];
    d += __shfl_xor(d, 16, 64);
    d += __shfl_xor(d, 32, 64);
    dr += __shfl_xor(dr, 16, 64);
    dr += __shfl_xor(dr, 32, 64);
    Dq[qt] = DG ? 0.f : dr;   // with D from O, A already holds (P o (dP - D)) K
    const int i = qw0 + 16 * qt + lc;
    if (lg == 0 && i < Tq) {
      p.dlt[rowbase + i] = DG ? dg[qt] : d;
      p.lse2[rowbase + i] = lse2[qt];   // the dk/dv pass reads lse in base-2 units
    }
  }
  // dQ = scale (A - D B): the lane holds d = 16 dt + 4 lg + r of query qw0 + 16 qt + lc.
#pragma unroll
  for (int qt = 0; qt < kNT; ++qt) {
    const int i = qw0 + 16 * qt + lc;
    if (i < Tq) {
      const int64_t o = (int64_t)b * p.sdq[0] + (int64_t)i * p.sdq[1] + (int64_t)h * p.sdq[2] + 4 * lg;
#pragma unroll
      for (int dt = 0; dt < kNDT; ++dt) {
        const f32x4 a = acA[dt][qt], bb = acB[dt][qt];
        const float s = p.scale, dd = Dq[qt];
        store4(p.dq, p.out_bf16, o + 16 * dt, s * (a[0] - dd * bb[0]), s * (a[1] - dd * bb[1]), s * (a[2] - dd * bb[2]),
               s * (a[3] - dd * bb[3]));
      }
    }
  }
}

// ------------------------------------------------------------------------------ forward
// Online-softmax forward on the dq pass's layout: per 64-key block the wave computes
// S^T = K Q^T (a lane owns one query column), takes the block's maximum over its four
// 16-lane groups, rescales its running sums and O^T by exp(m_old - m_new), then
// O^T += V^T P^T with V^T from LDS transpose reads. O is normalised by the sum of the
// bf16-rounded P that entered the MFMAs, so a query's weights sum to one as applied; lse
// comes from the fp32 sum.
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(kWavesPerEU, kWavesPerEU)))
void fwd_mfma_kernel(AttnParams p) {
  constexpr int BN = kRows, QW = 16 * kNT, BM = kW * QW;
  __shared__ __attribute__((aligned(1024))) __bf16 sm[2][2][BN * kHD];   // [buffer][K, V]

  int row, rank;
  grid_item(row, rank);
  const int b = row / p.Hq, h = row % p.Hq;
  const int nqb = (p.Tq + BM - 1) / BM;
  const int qb = nqb - 1 - rank;   // causal: heaviest query block first
  const int G = p.Hq / p.Hkv, kvh = h / G;
  const int w = wave_id(), lane = threadIdx.x & 63, lg = lane >> 4, lc = lane & 15;
  const int Tq = p.Tq, Tk = p.Tk, off = Tk - Tq;
  const float sl2 = p.scale * kLog2e;
  const int64_t rowbase = ((int64_t)b * p.Hq + h) * Tq;
  const int qw0 = qb * BM + QW * w;

  const __bf16* Qh = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.sq[0] + (int64_t)h * p.sq[2];
  const __bf16* Kh = reinterpret_cast<const __bf16*>(p.k) + (int64_t)b * p.sk[0] + (int64_t)kvh * p.sk[2];
  const __bf16* Vh = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.sv[0] + (int64_t)kvh * p.sv[2];

  bf16x8 qa[kNT][kNKS];   // Q of the lane's queries: B operand (k = d, n = query) of S^T
#pragma unroll
  for (int qt = 0; qt < kNT; ++qt) {
    const int i = min(qw0 + 16 * qt + lc, Tq - 1);
#pragma unroll
    for (int ks = 0; ks < kNKS; ++ks) qa[qt][ks] = load8<__bf16>(Qh + (int64_t)i * p.sq[1] + 32 * ks + 8 * lg);
  }
  f32x4 acO[kNDT][kNT];
#pragma unroll
  for (int dt = 0; dt < kNDT; ++dt)
#pragma unroll
    for (int qt = 0; qt < kNT; ++qt) acO[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // log2-domain running maximum (shared by the query's four lane groups), and this lane's
  // running sums of exp (fp32) and of the bf16-rounded exp
  float mrun[kNT], lrun[kNT], lrnd[kNT];
#pragma unroll
  for (int qt = 0; qt < kNT; ++qt) {
    mrun[qt] = -INFINITY;
    lrun[qt] = lrnd[qt] = 0.f;
  }

  const int last_row = min(Tq, (qb + 1) * BM) - 1;
  const int kend = p.causal ? min(Tk, last_row + off + 1) : Tk;
  const int nblk = (kend + BN - 1) / BN;
  const int wkend = qw0 >= Tq ? 0 : (p.causal ? min(Tk, min(Tq - 1, qw0 + QW - 1) + off + 1) : Tk);

  RowStager kst, vst;
  kst.init(w, p.sk[1]);
  vst.init(w, p.sv[1]);
  wait_loads();
  const uint32_t sm_lds = lds_addr(&sm[0][0][0]);
  constexpr uint32_t kTileBytes = 2u * BN * kHD;
  if (nblk > 0) {
    kst.stage(sm_lds, Kh, p.sk[1], 0, Tk);
    vst.stage(sm_lds + kTileBytes, Vh, p.sv[1], 0, Tk);
  }

  auto block = [&](auto buf_c, int jb, bool full, auto&& dma) {
    const __bf16* sK = sm[decltype(buf_c)::value][0];
    const __bf16* sV = sm[decltype(buf_c)::value][1];
    f32x4 sT[4][kNT];
    bf16x8 fk[2][kNKS];
    auto read_rows = [&](int kt, bf16x8(&ak)[kNKS]) {
#pragma unroll
      for (int ks = 0; ks < kNKS; ++ks) ak[ks] = row8<LT>(sK, 16 * kt + lc, 32 * ks + 8 * lg);
    };
    prio_mfma();
    read_rows(0, fk[0]);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      if (kt + 1 < 4) read_rows(kt + 1, fk[(kt + 1) & 1]);
      if (kt == 0 || kt == 2) dma(kt >> 1);
      fence();
#pragma unroll
      for (int qt = 0; qt < kNT; ++qt) {
        sT[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kNKS; ++ks) mma(sT[kt][qt], fk[kt & 1][ks], qa[qt][ks]);
      }
      fence();
    }
    prio_valu();
    // V^T fragments of the first (dt, c) pairs are read under the softmax arithmetic.
    constexpr int NP = kNDT * 2, AHEAD = 4;
    bf16x8 vT[AHEAD + 1];
    auto read_vT = [&](int pr) { return col8<LT>(sV, 32 * (pr & 1) + 4 * lg, 32 * (pr & 1) + 16 + 4 * lg, 16 * (pr >> 1)); };
#pragma unroll
    for (int pr = 0; pr < AHEAD; ++pr) vT[pr] = read_vT(pr);
    fence();
    // scaled scores, log2 domain; invisible keys -inf (only blocks that cross the
    // diagonal or the end of the keys are masked)
    float s2[4][kNT][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qt = 0; qt < kNT; ++qt)
#pragma unroll
        for (int r = 0; r < 4; ++r) s2[kt][qt][r] = sT[kt][qt][r] * sl2;
    if (!full) {
      asm volatile("");   // keeps the masking inside the branch (no speculation into full blocks)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int qt = 0; qt < kNT; ++qt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int jj = jb + 16 * kt + 4 * lg + r, i = qw0 + 16 * qt + lc;
            s2[kt][qt][r] = ((jj < Tk) & (!p.causal | (jj <= i + off))) ? s2[kt][qt][r] : -INFINITY;
          }
    }
    // P as bf16 B operands (k = 32 keys, n = query): element e of operand c is key
    // 32c + 4 lg + e (e < 4) or 32c + 16 + 4 lg + e - 4 (e >= 4).
    bf16x8 pb[2][kNT];
#pragma unroll
    for (int qt = 0; qt < kNT; ++qt) {
      float bm = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) bm = fmaxf(bm, s2[kt][qt][r]);
      bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
      const float mn = fmaxf(mrun[qt], bm);
      const float mref = mn == -INFINITY ? 0.f : mn;           // no visible key yet: every term is 0
      const float a = __builtin_amdgcn_exp2f(mrun[qt] - mref);  // 0 while the maximum is -inf
      // Rescale only when some query of the wave has a new maximum (a = 1 exactly
      // otherwise, so skipping the products changes nothing).
      if (__builtin_amdgcn_ballot_w64(a != 1.f)) {
        lrun[qt] *= a;
        lrnd[qt] *= a;
#pragma unroll
        for (int dt = 0; dt < kNDT; ++dt) acO[dt][qt] *= a;
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(s2[kt][qt][r] - mref);
          lrun[qt] += e;
          pb[kt >> 1][qt][4 * (kt & 1) + r] = (__bf16)e;
        }
      // the sum of the bf16-rounded weights, two per instruction (each pair dotted with (1, 1))
      const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
      float t = lrnd[qt];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 p8 = pb[c][qt];
        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 0, 1), one2, t, false);
        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 2, 3), one2, t, false);
        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 4, 5), one2, t, false);
        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 6, 7), one2, t, false);
      }
      lrnd[qt] = t;
      mrun[qt] = mn;
    }
    fence();
    prio_mfma();
    // O^T += V^T P^T over (dt, c) pairs, reads AHEAD pairs ahead
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
      if (pr + AHEAD < NP) vT[(pr + AHEAD) % (AHEAD + 1)] = read_vT(pr + AHEAD);
      if (pr == 0 || pr == NP / 2) dma(2 + (pr != 0));
      fence();
      const int dt = pr >> 1, c = pr & 1;
#pragma unroll
      for (int qt = 0; qt < kNT; ++qt) mma(acO[dt][qt], vT[pr % (AHEAD + 1)], pb[c][qt]);
      fence();
    }
    prio_valu();
  };

  auto iteration = [&](int j, auto buf_c) {
    constexpr int nxt = decltype(buf_c)::value ^ 1;
    const int jb = j * BN;
    wait_loads();
    __syncthreads();   // block j is in LDS; every wave is done with block j - 1
    const bool more = j + 1 < nblk;
    auto dma = [&](int part) {
      if (!more || part != 0) return;
      kst.stage(sm_lds + (2 * nxt) * kTileBytes, Kh, p.sk[1], jb + BN, Tk);
      vst.stage(sm_lds + (2 * nxt + 1) * kTileBytes, Vh, p.sv[1], jb + BN, Tk);
    };
    if (jb >= wkend) {
      dma(0);
      return;
    }
    const bool full = jb + BN <= Tk && (!p.causal || jb + BN - 1 <= qw0 + off);
    block(buf_c, jb, full, dma);
  };
  int j = 0;
  for (; j + 1 < nblk; j += 2) {
    iteration(j, BufC<0>{});
    iteration(j + 1, BufC<1>{});
  }
  if (j < nblk) iteration(j, BufC<0>{});

  // the four 16-lane groups hold disjoint key subsets of the same query
#pragma unroll
  for (int qt = 0; qt < kNT; ++qt) {
    float l = lrun[qt], lr = lrnd[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    lr += __shfl_xor(lr, 16, 64);
    lr += __shfl_xor(lr, 32, 64);
    const int i = qw0 + 16 * qt + lc;
    if (i < Tq) {
      if (lg == 0 && p.lse_out) p.lse_out[rowbase + i] = (mrun[qt] + log2f(l)) * kLn2;
      const float inv = lr > 0.f ? 1.f / lr : 0.f;
      // the lane holds d = 16 dt + 4 lg + r of query i
      const int64_t o = (int64_t)b * p.sdq[0] + (int64_t)i * p.sdq[1] + (int64_t)h * p.sdq[2] + 4 * lg;
#pragma unroll
      for (int dt = 0; dt < kNDT; ++dt) {
        const f32x4 v4 = acO[dt][qt];
        store4(p.dq, p.out_bf16, o + 16 * dt, v4[0] * inv, v4[1] * inv, v4[2] * inv, v4[3] * inv);
      }
    }
  }
}

// ------------------------------------------------------------------------------ dkdv
// Workgroup: kW * 16 * kNT keys of one kv-head; wave w owns kNT 16-key tiles starting
// at kw0, K and V in registers as B operands. For every (q-head of the group, 64-query
// block) that sees the keys: S = Q K^T, dP = dO V^T (queries as MFMA rows), P and dS
// with the block's lse and D, then dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T
// from LDS transpose reads. dK and dV are written once, in a fixed head order.
// L2: lse is read from p.lse2 (already times log2 e, written by the dq pass); otherwise
// from p.lse.
template <bool L2>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(kWavesPerEU, kWavesPerEU)))
void dkdv_mfma_kernel(AttnParams p) {
  constexpr int BM = kRows, KW = 16 * kNT, BN = kW * KW;
  __shared__ __attribute__((aligned(1024))) __bf16 sm[2][2][BM * kHD];   // [buffer][Q, dO]
  __shared__ __attribute__((aligned(16))) float sv[2][2][BM];            // [buffer][lse, D]

  int row, rank;
  grid_item(row, rank);
  const int b = row / p.Hkv, kvh = row % p.Hkv;
  const int kb = rank * BN;   // causal: rank 0 sees every query block
  const int G = p.Hq / p.Hkv;
  const int w = wave_id(), lane = threadIdx.x & 63, lg = lane >> 4, lc = lane & 15;
  const int Tq = p.Tq, Tk = p.Tk, off = Tk - Tq;
  const float sl2 = p.scale * kLog2e;
  const int kw0 = kb + KW * w;

  const __bf16* Kh = reinterpret_cast<const __bf16*>(p.k) + (int64_t)b * p.sk[0] + (int64_t)kvh * p.sk[2];
  const __bf16* Vh = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.sv[0] + (int64_t)kvh * p.sv[2];
  bf16x8 kr[kNT][kNKS], vr[kNT][kNKS];   // B operands (k = d, n = key kw0 + 16 kt + lc)
#pragma unroll
  for (int kt = 0; kt < kNT; ++kt) {
    const int jj = min(kw0 + 16 * kt + lc, Tk - 1);
#pragma unroll
    for (int ks = 0; ks < kNKS; ++ks) {
      kr[kt][ks] = load8<__bf16>(Kh + (int64_t)jj * p.sk[1] + 32 * ks + 8 * lg);
      vr[kt][ks] = load8<__bf16>(Vh + (int64_t)jj * p.sv[1] + 32 * ks + 8 * lg);
    }
  }
  f32x4 adK[kNDT][kNT], adV[kNDT][kNT];
#pragma unroll
  for (int dt = 0; dt < kNDT; ++dt)
#pragma unroll
    for (int kt = 0; kt < kNT; ++kt) {
      adK[dt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      adV[dt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const int q_first = p.causal ? max(0, kb - off) : 0;
  const int qb0 = q_first / BM;
  const int nqb = (Tq + BM - 1) / BM - qb0;
  const int n_it = nqb > 0 ? G * nqb : 0;
  const int wq_first = p.causal ? kw0 - off : 0;   // earlier queries see none of the wave's keys

  RowStager qst, ost;
  qst.init(w, p.sq[1]);
  ost.init(w, p.sdo[1]);
  const uint32_t sm_lds = lds_addr(&sm[0][0][0]);
  const uint32_t sv_lds = lds_addr(&sv[0][0][0]);
  constexpr uint32_t kTileBytes = 2u * BM * kHD, kValBytes = 4u * BM;
  auto stage = [&](int buf, int hh, int q0) {
    const __bf16* Qh = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.sq[0] + (int64_t)hh * p.sq[2];
    const __bf16* Oh = reinterpret_cast<const __bf16*>(p.dout) + (int64_t)b * p.sdo[0] + (int64_t)hh * p.sdo[2];
    qst.stage(sm_lds + (2 * buf) * kTileBytes, Qh, p.sq[1], q0, Tq);
    ost.stage(sm_lds + (2 * buf + 1) * kTileBytes, Oh, p.sdo[1], q0, Tq);
    const int64_t rb = ((int64_t)b * p.Hq + hh) * Tq;
    if (w == 0) stage_vals64(sv_lds + (2 * buf) * kValBytes, (L2 ? p.lse2 : p.lse) + rb, q0, Tq);
    if (w == 1) stage_vals64(sv_lds + (2 * buf + 1) * kValBytes, p.dlt + rb, q0, Tq);
  };

  auto block = [&](auto buf_c, int q0, bool full, auto&& dma) {
    constexpr int buf = decltype(buf_c)::value;
    const __bf16* sQ = sm[buf][0];
    const __bf16* sO = sm[buf][1];
    const f32x4* sL4 = reinterpret_cast<const f32x4*>(&sv[buf][0][0]);
    const f32x4* sD4 = reinterpret_cast<const f32x4*>(&sv[buf][1][0]);
    // S, dP: tile (qt, kt) reg r holds query q0 + 16 qt + 4 lg + r, key kw0 + 16 kt + lc.
    // The Q and dO row fragments of tile qt + 1 are read while tile qt's MFMAs run.
    f32x4 S[4][kNT], dP[4][kNT];
    bf16x8 fq[2][kNKS], fo[2][kNKS];
    auto read_rows = [&](int qt, bf16x8(&aq)[kNKS], bf16x8(&ao)[kNKS]) {
#pragma unroll
      for (int ks = 0; ks < kNKS; ++ks) {
        aq[ks] = row8<LT>(sQ, 16 * qt + lc, 32 * ks + 8 * lg);
        ao[ks] = row8<LT>(sO, 16 * qt + lc, 32 * ks + 8 * lg);
      }
    };
    prio_mfma();
    read_rows(0, fq[0], fo[0]);
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      if (qt + 1 < 4) read_rows(qt + 1, fq[(qt + 1) & 1], fo[(qt + 1) & 1]);
      if (qt == 0 || qt == 2) dma(qt >> 1);
      fence();
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt) {
        S[qt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dP[qt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kNKS; ++ks) {
          mma(S[qt][kt], fq[qt & 1][ks], kr[kt][ks]);
          mma(dP[qt][kt], fo[qt & 1][ks], vr[kt][ks]);
        }
      }
      fence();
    }
    prio_valu();
    // dO^T and Q^T fragments of the first (dt, c) pairs are read under the arithmetic.
    constexpr int NP = kNDT * 2, AHEAD = VTB_DKDV_AHEAD;
    bf16x8 oT[AHEAD + 1], qT[AHEAD + 1];
    auto read_T = [&](int pr, bf16x8& o, bf16x8& q) {
      const int c = pr & 1, dt = pr >> 1;
      o = col8<LT>(sO, 32 * c + 4 * lg, 32 * c + 16 + 4 * lg, 16 * dt);
      q = col8<LT>(sQ, 32 * c + 4 * lg, 32 * c + 16 + 4 * lg, 16 * dt);
    };
    f32x4 Lv[4], Dv[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      Lv[qt] = sL4[4 * qt + lg];
      Dv[qt] = sD4[4 * qt + lg];
    }
#pragma unroll
    for (int pr = 0; pr < AHEAD; ++pr) read_T(pr, oT[pr], qT[pr]);
    fence();
    // P and dS as bf16 B operands (k = 32 queries, n = key): element e of operand c is
    // query 32c + 4 lg + e (e < 4) or 32c + 16 + 4 lg + e - 4 (e >= 4).
    // Only blocks that cross the diagonal or a tensor's end are masked; the branch covers
    // just the masking, so both kinds of block share registers and MFMA code.
    float pe[4][kNT][4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt)
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) pe[qt][kt][r] = __builtin_amdgcn_exp2f(S[qt][kt][r] * sl2 - (L2 ? Lv[qt][r] : Lv[qt][r] * kLog2e));
    if (!full) {
      asm volatile("");   // keeps the masking inside the branch (no speculation into full blocks)
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int kt = 0; kt < kNT; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = q0 + 16 * qt + 4 * lg + r, jj = kw0 + 16 * kt + lc;
            pe[qt][kt][r] = ((i < Tq) & (jj < Tk) & (!p.causal | (jj <= i + off))) ? pe[qt][kt][r] : 0.f;
          }
    }
    bf16x8 pb[2][kNT], sb[2][kNT];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pr = pe[qt][kt][r];
          pb[qt >> 1][kt][4 * (qt & 1) + r] = (__bf16)pr;
          sb[qt >> 1][kt][4 * (qt & 1) + r] = (__bf16)(pr * (dP[qt][kt][r] - Dv[qt][r]));
        }
    }
    fence();
    prio_mfma();
    // dV^T += dO^T P,  dK^T += Q^T dS over (dt, c) pairs (scale applied at the end)
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
      if (pr + AHEAD < NP) read_T(pr + AHEAD, oT[(pr + AHEAD) % (AHEAD + 1)], qT[(pr + AHEAD) % (AHEAD + 1)]);
      if (pr == 0 || pr == NP / 2) dma(2 + (pr != 0));
      fence();
      const int dt = pr >> 1, c = pr & 1;
#pragma unroll
      for (int kt = 0; kt < kNT; ++kt) {
        mma(adV[dt][kt], oT[pr % (AHEAD + 1)], pb[c][kt]);
        mma(adK[dt][kt], qT[pr % (AHEAD + 1)], sb[c][kt]);
      }
      fence();
    }
    prio_valu();
  };

  // Iteration it works on (head h, query block q0); (hs, q0s) is the iteration whose
  // loads are in flight, one ahead. Both advance without division. The register loads
  // above complete first: the compiler then needs no waits for them in the loop (it does
  // not see the direct-to-LDS loads).
  int h = kvh * G, q0 = qb0 * BM;
  wait_loads();
  int hs = h, q0s = q0;
  if (n_it > 0) {
    stage(0, hs, q0s);
    q0s += BM;
    if (q0s >= Tq) {
      q0s = qb0 * BM;
      ++hs;
    }
  }
  // Iteration it sits in buffer it % 2. After the barrier every wave has finished
  // iteration it - 1, so the loads of it + 1 go to its buffer right away.
  auto iteration = [&](int it, auto buf_c) {
    constexpr int nxt = decltype(buf_c)::value ^ 1;
    wait_loads();
    __syncthreads();   // iteration it is in LDS; every wave is done with it - 1
    const bool more = it + 1 < n_it;
    const __bf16* Qn = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.sq[0] + (int64_t)hs * p.sq[2];
    const __bf16* On = reinterpret_cast<const __bf16*>(p.dout) + (int64_t)b * p.sdo[0] + (int64_t)hs * p.sdo[2];
    const int qn = q0s;
    auto dma = [&](int part) {
      if (!more || part != 0) return;
      const int64_t rb = ((int64_t)b * p.Hq + hs) * Tq;
      if (w == 0) stage_vals64(sv_lds + (2 * nxt) * kValBytes, (L2 ? p.lse2 : p.lse) + rb, qn, Tq);
      if (w == 1) stage_vals64(sv_lds + (2 * nxt + 1) * kValBytes, p.dlt + rb, qn, Tq);
      qst.stage(sm_lds + (2 * nxt) * kTileBytes, Qn, p.sq[1], qn, Tq);
      ost.stage(sm_lds + (2 * nxt + 1) * kTileBytes, On, p.sdo[1], qn, Tq);
    };
    if (q0 + BM - 1 >= wq_first && kw0 < Tk) {
      const bool full = q0 + BM <= Tq && kw0 + KW <= Tk && (!p.causal || kw0 + KW - 1 <= q0 + off);
      block(buf_c, q0, full, dma);
    } else {
      dma(0);
    }
    if (more) {
      q0s += BM;
      if (q0s >= Tq) {
        q0s = qb0 * BM;
        ++hs;
      }
    }
    q0 += BM;
    if (q0 >= Tq) q0 = qb0 * BM;
  };
  int it = 0;
  for (; it + 1 < n_it; it += 2) {
    iteration(it, BufC<0>{});
    iteration(it + 1, BufC<1>{});
  }
  if (it < n_it) iteration(it, BufC<0>{});

  // dK = scale acc, dV = acc: the lane holds d = 16 dt + 4 lg + r of key kw0 + 16 kt + lc.
#pragma unroll
  for (int kt = 0; kt < kNT; ++kt) {
    const int jj = kw0 + 16 * kt + lc;
    if (jj < Tk) {
      const int64_t ok = (int64_t)b * p.sdk[0] + (int64_t)jj * p.sdk[1] + (int64_t)kvh * p.sdk[2] + 4 * lg;
      const int64_t ov = (int64_t)b * p.sdv[0] + (int64_t)jj * p.sdv[1] + (int64_t)kvh * p.sdv[2] + 4 * lg;
#pragma unroll
      for (int dt = 0; dt < kNDT; ++dt) {
        const f32x4 k4 = adK[dt][kt], v4 = adV[dt][kt];
        const float s = p.scale;
        if (p.dk) store4(p.dk, p.out_bf16, ok + 16 * dt, s * k4[0], s * k4[1], s * k4[2], s * k4[3]);
        if (p.dv) store4(p.dv, p.out_bf16, ov + 16 * dt, v4[0], v4[1], v4[2], v4[3]);
      }
    }
  }
}

}  // namespace

bool mfma_path_applicable(const AttnParams& p) {
  // The staging loads address a 64-row block with 32-bit byte offsets from its first row.
  auto small = [](int64_t st) { return st >= 1 && st <= (int64_t)1 << 24; };
  return p.in_bf16 && p.D == kHD && small(p.sq[1]) && small(p.sk[1]) && small(p.sv[1]) && small(p.sdo[1]);
}

bool mfma_fwd_applicable(const AttnParams& p) {
  auto small = [](int64_t st) { return st >= 1 && st <= (int64_t)1 << 24; };
  return p.in_bf16 && p.D == kHD && small(p.sq[1]) && small(p.sk[1]) && small(p.sv[1]);
}

hipError_t launch_mfma_fwd(const AttnParams& p, hipStream_t s, KernelEvents ev) {
  constexpr int BM = kW * 16 * kNT;
  const dim3 grid(p.B * p.Hq, (p.Tq + BM - 1) / BM);
  launch_kernel(fwd_mfma_kernel, grid, dim3(kT), 0, s, ev, p);
  return hipGetLastError();
}

hipError_t launch_mfma_dq(const AttnParams& p, hipStream_t s, KernelEvents ev, bool d_given) {
  constexpr int BM = kW * 16 * kNT;
  const dim3 grid(p.B * p.Hq, (p.Tq + BM - 1) / BM);
  if (d_given)
    launch_kernel(dq_mfma_kernel<true>, grid, dim3(kT), 0, s, ev, p);
  else
    launch_kernel(dq_mfma_kernel<false>, grid, dim3(kT), 0, s, ev, p);
  return hipGetLastError();
}

hipError_t launch_mfma_dkdv(const AttnParams& p, hipStream_t s, KernelEvents ev) {
  constexpr int BN = kW * 16 * kNT;
  const dim3 grid(p.B * p.Hkv, (p.Tk + BN - 1) / BN);
  if (p.lse2)
    launch_kernel(dkdv_mfma_kernel<true>, grid, dim3(kT), 0, s, ev, p);
  else
    launch_kernel(dkdv_mfma_kernel<false>, grid, dim3(kT), 0, s, ev, p);
  return hipGetLastError();
}

}  // namespace vtb
