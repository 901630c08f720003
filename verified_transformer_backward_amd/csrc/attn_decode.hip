// Decode-shaped attention backward (few query rows per kv-head group, long KV cache).
//
// Same chain as the flash path ("Hesper.Training.VerifiedBackward", section "Attention
// (full single-head)": attentionBackwardQ / attentionBackwardV), organised for the
// case the single-query specs describe: R = (Hq/Hkv) * Tq <= 16 query rows share one
// kv-head, so the work is reading K and V once and writing dK and dV once.
//
// The KV cache is split into 64-key chunks (the tiled split-KV statistics idea the
// Hesper commit log uses for long caches: per-tile max, sum of exponentials, merged
// afterwards). Two launches, each touching the cache once:
//   chunk  per (chunk, kv-head, batch), K and V read once: for every row r and key j
//          s = scale q.k and dP = dO.v; per-row chunk statistics m_c = max s,
//          l_c = sum e, u_c = sum e dP with e = exp(s - m_c); and the chunk's two dQ
//          pieces A_c = sum_j e dP k_j and B_c = sum_j e k_j.
//   grads  per (chunk, kv-head, batch), no K/V reads: merges the statistics into lse
//          (unless given) and D = rowsum(P o dP) = sum_c exp(m_c - lse) u_c, forms P and
//          dS = P o (dP - D) for the chunk from the stored s and dP, and writes
//          dV_j = sum_rows P dO and dK_j = scale sum_rows dS q (rows in fixed
//          head-then-query order). Since dS = P o (dP - D),
//              dQ_r = scale sum_c exp(m_c - lse_r) (A_c - D_r B_c),
//          summed over chunks in fixed order; the (row, column) outputs of dQ are split
//          evenly over the chunk workgroups of the kv-head.
// When the keys fit one chunk, the chunk workgroup does the gradient pass's work itself
// (one launch, the same arithmetic, no workspace traffic).
#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace vtb {
namespace {

constexpr int kCH = 64;        // keys per chunk
constexpr int kMaxRows = 16;   // query rows per kv-head group
constexpr int kThreads = 256;
constexpr int kPreCh = 16;     // chunks whose dQ terms are prefetched into registers

struct DecodeWs {
  float* s;      // [rows, Tk] scaled scores (-inf where invisible); row = (b Hq + h) Tq + i
  float* dp;     // [rows, Tk]
  float* stats;  // [rows, nch, 3] = (m_c, l_c, u_c)
  float* a;      // [nch, rows, D] sum_j exp(s - m_c) dP k_j over the chunk
  float* bk;     // [nch, rows, D] sum_j exp(s - m_c) k_j over the chunk
};

__host__ __device__ inline int64_t align_up(int64_t x) { return (x + 63) / 64 * 64; }

DecodeWs carve(const AttnParams& p, void* base) {
  const int nch = (p.Tk + kCH - 1) / kCH;
  const int64_t rows = (int64_t)p.B * p.Hq * p.Tq;
  float* f = reinterpret_cast<float*>(base);
  DecodeWs w;
  w.s = f;
  f += align_up(rows * p.Tk);
  w.dp = f;
  f += align_up(rows * p.Tk);
  w.stats = f;
  f += align_up(rows * nch * 3);
  w.a = f;
  f += align_up(nch * rows * p.D);
  w.bk = f;
  return w;
}

template <typename E>
__device__ __forceinline__ const E* rp(const void* base, const int64_t* st, int b, int t, int h) {
  return reinterpret_cast<const E*>(base) + (int64_t)b * st[0] + (int64_t)t * st[1] + (int64_t)h * st[2];
}

// Rows r of the group: q-head kvh G + r / Tq, query r % Tq. The R rows of q and dO go to
// LDS as fp32 (row stride ld), eight elements per load.
template <typename E, int D>
__device__ __forceinline__ void stage_rows(const AttnParams& p, int b, int kvh, int R, float* sq, float* sdo,
                                           int ld) {
  constexpr int C8 = D / 8;
  const int G = p.Hq / p.Hkv, Tq = p.Tq;
  for (int idx = threadIdx.x; idx < R * C8; idx += kThreads) {
    const int r = idx / C8, c8 = idx % C8;
    const int h = kvh * G + r / Tq, i = r % Tq;
    const frag_t<E> q8 = load8<E>(rp<E>(p.q, p.sq, b, i, h) + 8 * c8);
    const frag_t<E> o8 = load8<E>(rp<E>(p.dout, p.sdo, b, i, h) + 8 * c8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sq[r * ld + 8 * c8 + e] = to_f32(q8[e]);
      sdo[r * ld + 8 * c8 + e] = to_f32(o8[e]);
    }
  }
}

// FUSED (the keys fit one chunk, nch == 1): the chunk's statistics are the row's, so the
// same workgroup goes on to the gradient pass's work (P, dS, dK, dV, dQ) with the
// arithmetic of decode_grads_kernel for one chunk, bit for bit, and nothing goes through
// the workspace.
template <typename E, typename EO, int D, bool FUSED>
__global__ __launch_bounds__(kThreads) void decode_chunk_kernel(AttnParams p, DecodeWs ws, int nch) {
  // LDS rows padded to D + 4 floats: the 16 lanes of an MFMA operand read, each taking 16
  // bytes of its own row, cover all 64 banks once.
  constexpr int LD = D + 4;
  constexpr int V = 16 / sizeof(E), CV = D / V, NL = kCH * CV / kThreads;   // 16-byte loads
  static_assert(NL * kThreads == kCH * CV, "chunk loads must tile the workgroup");
  static_assert(kCH == 64 && kThreads == 256, "four waves of 16 keys cover the chunk");
  typedef E vec_t __attribute__((ext_vector_type(V)));
  const int ch = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = p.Hq / p.Hkv, R = G * p.Tq, Tq = p.Tq, Tk = p.Tk, off = Tk - Tq;
  const int j0 = ch * kCH;
  // Dynamic LDS sized for the group's R rows at launch: q and dO (rows of LD), the chunk
  // (V, then K), then s and dP per row and key. Once the statistics of a row have read its
  // s and dP, the same places take e and e dP (the lane that reads is the lane that writes).
  extern __shared__ float4 dyn4[];
  float* sq = reinterpret_cast<float*>(dyn4);
  float* sdo = sq + R * LD;
  float* skv = sdo + R * LD;
  float* ss = skv + kCH * LD;
  float* sdp = ss + R * kCH;
  float* sw = ss;
  float* sx = sdp;
  const int tid = threadIdx.x;

  // K and V of the chunk: every load issued up front, 16 contiguous bytes per lane; rows
  // past Tk re-read row Tk - 1.
  vec_t kreg[NL], vreg[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int f = tid + kThreads * i, row = f / CV, cv = f % CV;
    const int j = min(j0 + row, Tk - 1);
    kreg[i] = *reinterpret_cast<const vec_t*>(rp<E>(p.k, p.sk, b, j, kvh) + V * cv);
    vreg[i] = *reinterpret_cast<const vec_t*>(rp<E>(p.v, p.sv, b, j, kvh) + V * cv);
  }
  stage_rows<E, D>(p, b, kvh, R, sq, sdo, LD);
  auto to_lds = [&](const vec_t(&reg)[NL]) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int f = tid + kThreads * i, row = f / CV, cv = f % CV;
#pragma unroll
      for (int e4 = 0; e4 < V; e4 += 4)
        *reinterpret_cast<float4*>(skv + row * LD + V * cv + e4) =
            make_float4(to_f32(reg[i][e4]), to_f32(reg[i][e4 + 1]), to_f32(reg[i][e4 + 2]), to_f32(reg[i][e4 + 3]));
    }
  };
  // The chunk's products with every row on the fp32 matrix cores (16x16x4): wave w takes
  // keys 16 w .. 16 w + 15 as the rows of A (the staged chunk) and the group's rows as the
  // columns of B (x; columns past R re-read row R - 1 and are not stored), contracting over
  // the head dim. Lane (c, g) = (lane % 16, lane / 16) holds d = d0 + 4 g .. 4 g + 3 of its
  // A row and B column, and step e of each group of four contracts element e, so A and B
  // agree on every k. Result register r is key 16 w + 4 g + r of row c: out[c][key] = mul * dot.
  const int lane = tid & 63, w = tid >> 6, mc = lane & 15, mg = lane >> 4;
  auto mfma_dots = [&](const float* x, float* out, float mul) {
    const float* arow = skv + (16 * w + mc) * LD + 4 * mg;
    const float* brow = x + min(mc, R - 1) * LD + 4 * mg;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int d0 = 0; d0 < D; d0 += 16) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(arow + d0);
      const f32x4 bx = *reinterpret_cast<const f32x4*>(brow + d0);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], bx[e], acc, 0, 0, 0);
    }
    if (mc < R)
      *reinterpret_cast<float4*>(out + mc * kCH + 16 * w + 4 * mg) =
          make_float4(acc[0] * mul, acc[1] * mul, acc[2] * mul, acc[3] * mul);
  };
  to_lds(vreg);
  __syncthreads();
  mfma_dots(sdo, sdp, 1.f);
  __syncthreads();   // every read of V is done
  to_lds(kreg);
  __syncthreads();
  mfma_dots(sq, ss, p.scale);
  __syncthreads();

  // statistics: lane = key jj, wave = rows rg, rg + 4, ...
  const int jj = lane, rg = w, j = j0 + jj;
  constexpr int kRPW = kMaxRows / (kThreads / 64);   // rows per wave at most
  float fP[kRPW], fdS[kRPW];                         // FUSED: P and dS of (row rg + 4 t, key jj)
  __shared__ float sM[kMaxRows], sLse[kMaxRows], sDl[kMaxRows];
  if constexpr (FUSED) {
#pragma unroll
    for (int t = 0; t < kRPW; ++t) {
      const int r = rg + 4 * t;
      fP[t] = fdS[t] = 0.f;
      if (r < R) {   // wave-uniform
        const int h = kvh * G + r / Tq, i = r % Tq;
        const int64_t row = ((int64_t)b * p.Hq + h) * Tq + i;
        const float s = ss[r * kCH + jj];
        const float dp = sdp[r * kCH + jj];
        const bool vis = j < Tk && (!p.causal || j <= i + off);
        const float m = wave_max(vis ? s : -INFINITY);
        const float e = (vis && m != -INFINITY) ? expf(s - m) : 0.f;
        const float l = wave_sum(e);
        const float u = wave_sum(e * dp);
        sw[r * kCH + jj] = e;
        sx[r * kCH + jj] = e * dp;
        // one chunk's statistics merged as the gradient pass merges them: M = m, L = l, U = u,
        // taken from lane 0 as the stored statistics are (the compiler may fuse a lane's own
        // e dP into the first step of the sum, so lanes can differ in the last bit). D is
        // rounded on its own (the gradient pass reads it back from LDS), so that it is not
        // contracted into dP - D below.
        const float lse = __shfl(p.lse ? p.lse[row] : m + logf(l), 0, 64);
        const float Dl = __shfl(__fmul_rn(u, expf(m - lse)), 0, 64);
        const float rs = vis ? s : -INFINITY;
        const float pr = rs == -INFINITY ? 0.f : expf(rs - lse);
        fP[t] = pr;
        fdS[t] = pr * ((j < Tk ? dp : 0.f) - Dl);
        if (jj == 0) {
          sM[r] = m;
          sLse[r] = lse;
          sDl[r] = Dl;
        }
      }
    }
  }
  for (int r = rg; r < (FUSED ? 0 : R); r += 4) {
    const int h = kvh * G + r / Tq, i = r % Tq;
    const int64_t row = ((int64_t)b * p.Hq + h) * Tq + i;
    const float s = ss[r * kCH + jj];
    const float dp = sdp[r * kCH + jj];
    const bool vis = j < Tk && (!p.causal || j <= i + off);
    if (j < Tk) {
      ws.s[row * Tk + j] = vis ? s : -INFINITY;
      ws.dp[row * Tk + j] = dp;
    }
    const float m = wave_max(vis ? s : -INFINITY);
    const float e = (vis && m != -INFINITY) ? expf(s - m) : 0.f;
    const float l = wave_sum(e);
    const float u = wave_sum(e * dp);
    sw[r * kCH + jj] = e;
    sx[r * kCH + jj] = e * dp;
    if (jj == 0) {
      float* st = ws.stats + (row * nch + ch) * 3;
      st[0] = m;
      st[1] = l;
      st[2] = u;
    }
  }
  __syncthreads();

  // A_c, B_c: wave w takes rows w, w + 4, ...; lane = (key part ks, four columns c4), the
  // KS parts of the chunk's keys summed over lanes in a fixed order (part 0 + part 1, then
  // + the sum of parts 2 and 3), so every wave works when R < 8.
  constexpr int C4 = D / 4, KS = 64 / C4, KL = kCH / KS;
  static_assert(C4 * KS == 64 && KS * KL == kCH, "one wave covers the row");
  const int c4 = lane % C4, ks = lane / C4;
  const int64_t rows = (int64_t)p.B * p.Hq * Tq;
  if constexpr (FUSED) {
    float4 fa[kRPW], fb[kRPW];
#pragma unroll
    for (int t = 0; t < kRPW; ++t) {
      const int r = w + 4 * t;
      fa[t] = fb[t] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < R) {
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), bb = a;
#pragma unroll 8
        for (int k = ks * KL; k < ks * KL + KL; ++k) {
          const float4 kv = *reinterpret_cast<const float4*>(skv + k * LD + 4 * c4);
          const float x = sx[r * kCH + k], we = sw[r * kCH + k];
          a.x = fmaf(x, kv.x, a.x); a.y = fmaf(x, kv.y, a.y); a.z = fmaf(x, kv.z, a.z); a.w = fmaf(x, kv.w, a.w);
          bb.x = fmaf(we, kv.x, bb.x); bb.y = fmaf(we, kv.y, bb.y); bb.z = fmaf(we, kv.z, bb.z); bb.w = fmaf(we, kv.w, bb.w);
        }
#pragma unroll
        for (int o = C4; o < 64; o <<= 1) {
          a.x += __shfl_xor(a.x, o, 64); a.y += __shfl_xor(a.y, o, 64); a.z += __shfl_xor(a.z, o, 64); a.w += __shfl_xor(a.w, o, 64);
          bb.x += __shfl_xor(bb.x, o, 64); bb.y += __shfl_xor(bb.y, o, 64); bb.z += __shfl_xor(bb.z, o, 64); bb.w += __shfl_xor(bb.w, o, 64);
        }
        fa[t] = a;
        fb[t] = bb;
      }
    }
    __syncthreads();   // every read of K, e and e dP is done: their places take A, B, P and dS
    float* sA = skv;            // [R][D]
    float* sB = skv + R * D;    // [R][D]; 2 R D <= kCH (D + 4)
#pragma unroll
    for (int t = 0; t < kRPW; ++t) {
      const int r = w + 4 * t;
      if (r < R) {
        if (ks == 0) {
          *reinterpret_cast<float4*>(sA + r * D + 4 * c4) = fa[t];
          *reinterpret_cast<float4*>(sB + r * D + 4 * c4) = fb[t];
        }
        ss[r * kCH + jj] = fP[t];
        sdp[r * kCH + jj] = fdS[t];
      }
    }
    __syncthreads();
    // dK, dV rows of the chunk: thread owns four columns of one key per pass
    const int jn = min(kCH, Tk - j0);
    {
      constexpr int KP = kThreads / C4;
      const int tc = tid % C4;
      for (int kk = tid / C4; kk < jn; kk += KP) {
        const int jk = j0 + kk;
        float4 ak = make_float4(0.f, 0.f, 0.f, 0.f), av = ak;
        for (int r = 0; r < R; ++r) {
          const float4 qv = *reinterpret_cast<const float4*>(sq + r * LD + 4 * tc);
          const float4 ov = *reinterpret_cast<const float4*>(sdo + r * LD + 4 * tc);
          const float ps = ss[r * kCH + kk], ds = sdp[r * kCH + kk];
          av.x = fmaf(ps, ov.x, av.x); av.y = fmaf(ps, ov.y, av.y); av.z = fmaf(ps, ov.z, av.z); av.w = fmaf(ps, ov.w, av.w);
          ak.x = fmaf(ds, qv.x, ak.x); ak.y = fmaf(ds, qv.y, ak.y); ak.z = fmaf(ds, qv.z, ak.z); ak.w = fmaf(ds, qv.w, ak.w);
        }
        EO* dkp = reinterpret_cast<EO*>(p.dk) + (int64_t)b * p.sdk[0] + (int64_t)jk * p.sdk[1] + (int64_t)kvh * p.sdk[2] + 4 * tc;
        EO* dvp = reinterpret_cast<EO*>(p.dv) + (int64_t)b * p.sdv[0] + (int64_t)jk * p.sdv[1] + (int64_t)kvh * p.sdv[2] + 4 * tc;
        const float sc = p.scale;
        if constexpr (std::is_same<EO, float>::value) {
          if (p.dk) __builtin_nontemporal_store(f32x4{ak.x * sc, ak.y * sc, ak.z * sc, ak.w * sc}, reinterpret_cast<f32x4*>(dkp));
          if (p.dv) __builtin_nontemporal_store(f32x4{av.x, av.y, av.z, av.w}, reinterpret_cast<f32x4*>(dvp));
        } else {
          if (p.dk)
            __builtin_nontemporal_store(bf16x4{(__bf16)(ak.x * sc), (__bf16)(ak.y * sc), (__bf16)(ak.z * sc), (__bf16)(ak.w * sc)},
                                        reinterpret_cast<bf16x4*>(dkp));
          if (p.dv)
            __builtin_nontemporal_store(bf16x4{(__bf16)av.x, (__bf16)av.y, (__bf16)av.z, (__bf16)av.w},
                                        reinterpret_cast<bf16x4*>(dvp));
        }
      }
    }
    // dQ_r = scale exp(m - lse_r) (A - D_r B), D_r B rounded on its own (as in the gradient pass)
    for (int o = tid; o < R * D; o += kThreads) {
      const int r = o / D, d = o % D;
      const int h = kvh * G + r / Tq, i = r % Tq;
      const float lse = sLse[r], Dr = sDl[r], mr = sM[r];
      const float wq = mr == -INFINITY ? 0.f : expf(mr - lse);
      float acc = 0.f;
      acc += wq * (sA[r * D + d] - __fmul_rn(Dr, sB[r * D + d]));
      EO* dqp = reinterpret_cast<EO*>(p.dq) + (int64_t)b * p.sdq[0] + (int64_t)i * p.sdq[1] + (int64_t)h * p.sdq[2];
      dqp[d] = from_f32<EO>(acc * p.scale);
    }
    return;
  }
  for (int r = w; r < R; r += kThreads / 64) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), bb = a;
#pragma unroll 8
    for (int k = ks * KL; k < ks * KL + KL; ++k) {
      const float4 kv = *reinterpret_cast<const float4*>(skv + k * LD + 4 * c4);
      const float x = sx[r * kCH + k], w = sw[r * kCH + k];
      a.x = fmaf(x, kv.x, a.x); a.y = fmaf(x, kv.y, a.y); a.z = fmaf(x, kv.z, a.z); a.w = fmaf(x, kv.w, a.w);
      bb.x = fmaf(w, kv.x, bb.x); bb.y = fmaf(w, kv.y, bb.y); bb.z = fmaf(w, kv.z, bb.z); bb.w = fmaf(w, kv.w, bb.w);
    }
#pragma unroll
    for (int o = C4; o < 64; o <<= 1) {
      a.x += __shfl_xor(a.x, o, 64); a.y += __shfl_xor(a.y, o, 64); a.z += __shfl_xor(a.z, o, 64); a.w += __shfl_xor(a.w, o, 64);
      bb.x += __shfl_xor(bb.x, o, 64); bb.y += __shfl_xor(bb.y, o, 64); bb.z += __shfl_xor(bb.z, o, 64); bb.w += __shfl_xor(bb.w, o, 64);
    }
    if (ks == 0) {
      const int h = kvh * G + r / Tq, i = r % Tq;
      const int64_t o = ((int64_t)ch * rows + ((int64_t)b * p.Hq + h) * Tq + i) * D + 4 * c4;
      *reinterpret_cast<float4*>(ws.a + o) = a;
      *reinterpret_cast<float4*>(ws.bk + o) = bb;
    }
  }
}

template <typename E, typename EO, int D>
__global__ __launch_bounds__(kThreads) void decode_grads_kernel(AttnParams p, DecodeWs ws, int nch) {
  const int ch = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = p.Hq / p.Hkv, R = G * p.Tq, Tq = p.Tq, Tk = p.Tk;
  const int j0 = ch * kCH, jn = min(kCH, Tk - j0);
  __shared__ __attribute__((aligned(16))) float sq[kMaxRows][D];
  __shared__ __attribute__((aligned(16))) float sdo[kMaxRows][D];
  __shared__ float sP[kMaxRows][kCH], sdS[kMaxRows][kCH];
  __shared__ float sLse[kMaxRows], sDl[kMaxRows];
  const int tid = threadIdx.x;

  // dQ: this workgroup's share of the group's R * D outputs (one per thread when it fits),
  // summed over chunks in order. Its chunk terms are loaded first, so they arrive while
  // the statistics merge and dK/dV run.
  const int total = R * D, per = (total + nch - 1) / nch;
  const int o0 = ch * per, o1 = min(total, o0 + per);
  const int64_t rows = (int64_t)p.B * p.Hq * Tq;
  const bool pre = per <= kThreads && nch <= kPreCh;
  const int o = o0 + tid;
  int64_t orow = 0;
  float pm[kPreCh], pa[kPreCh], pb[kPreCh];
  if (pre && o < o1) {
    const int r = o / D, h = kvh * G + r / Tq, i = r % Tq;
    orow = ((int64_t)b * p.Hq + h) * Tq + i;
#pragma unroll
    for (int c = 0; c < kPreCh; ++c) {
      const int cc = min(c, nch - 1);
      const int64_t e = ((int64_t)cc * rows + orow) * D + o % D;
      pm[c] = c < nch ? ws.stats[(orow * nch + cc) * 3] : -INFINITY;
      pa[c] = ws.a[e];
      pb[c] = ws.bk[e];
    }
  }

  // the chunk's stored scores and dP, one (row, key) pair per thread and pass
  constexpr int kPairs = kMaxRows * kCH / kThreads;
  float rs[kPairs], rd[kPairs];
#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
    const int idx = tid + kThreads * k, r = idx / kCH, j = j0 + idx % kCH;
    rs[k] = -INFINITY;
    rd[k] = 0.f;
    if (r < R && j < Tk) {
      const int64_t row = ((int64_t)b * p.Hq + kvh * G + r / Tq) * Tq + r % Tq;
      rs[k] = ws.s[row * Tk + j];
      rd[k] = ws.dp[row * Tk + j];
    }
  }

  // q and dO of the group's rows (one 8-element piece of each per thread), loaded with the
  // rest so that every input of the pass is in flight before the first wait
  constexpr int C8 = D / 8;
  static_assert(kMaxRows * C8 <= kThreads, "one q and dO piece per thread");
  const bool has_row = tid < R * C8;
  frag_t<E> q8, o8;
  if (has_row) {
    const int r = tid / C8, c8 = tid % C8;
    q8 = load8<E>(rp<E>(p.q, p.sq, b, r % Tq, kvh * G + r / Tq) + 8 * c8);
    o8 = load8<E>(rp<E>(p.dout, p.sdo, b, r % Tq, kvh * G + r / Tq) + 8 * c8);
  }

  // merge every chunk's statistics for each row (16 lanes per row)
  {
    const int r = tid >> 4, cl = tid & 15;
    if (r < R) {  // uniform within each 16-lane group
      const int h = kvh * G + r / Tq, i = r % Tq;
      const int64_t row = ((int64_t)b * p.Hq + h) * Tq + i;
      const float* st = ws.stats + row * nch * 3;
      // one pass per lane (running max with rescaled sums), then across the 16 lanes
      float M = -INFINITY, L = 0.f, U = 0.f;
      for (int c = cl; c < nch; c += 16) {
        const float mc = st[3 * c], lc = st[3 * c + 1], uc = st[3 * c + 2];
        if (mc == -INFINITY) continue;
        const float Mn = fmaxf(M, mc);
        const float wo = expf(M - Mn), wn = expf(mc - Mn);   // M = -inf gives wo = 0
        L = L * wo + lc * wn;
        U = U * wo + uc * wn;
        M = Mn;
      }
      const float Mall = group16_max(M);
      const float wl = M == -INFINITY ? 0.f : expf(M - Mall);
      L = group16_sum(L * wl);
      U = group16_sum(U * wl);
      M = Mall;
      const float lse = p.lse ? p.lse[row] : M + logf(L);
      if (cl == 0) {
        sLse[r] = lse;
        sDl[r] = U * expf(M - lse);
      }
    }
  }
  if (has_row) {
    const int r = tid / C8, c8 = tid % C8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sq[r][8 * c8 + e] = to_f32(q8[e]);
      sdo[r][8 * c8 + e] = to_f32(o8[e]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
    const int idx = tid + kThreads * k, r = idx / kCH, jj = idx % kCH;
    if (r < R) {
      const float pr = rs[k] == -INFINITY ? 0.f : expf(rs[k] - sLse[r]);
      sP[r][jj] = pr;
      sdS[r][jj] = pr * (rd[k] - sDl[r]);
    }
  }
  __syncthreads();

  // dK, dV rows of this chunk: thread owns four columns of one key per pass
  {
    constexpr int C4 = D / 4, KP = kThreads / C4;
    const int c4 = tid % C4;
    for (int jj = tid / C4; jj < jn; jj += KP) {
      const int j = j0 + jj;
      float4 ak = make_float4(0.f, 0.f, 0.f, 0.f), av = ak;
      for (int r = 0; r < R; ++r) {
        const float4 qv = *reinterpret_cast<const float4*>(&sq[r][4 * c4]);
        const float4 ov = *reinterpret_cast<const float4*>(&sdo[r][4 * c4]);
        const float ps = sP[r][jj], ds = sdS[r][jj];
        av.x = fmaf(ps, ov.x, av.x); av.y = fmaf(ps, ov.y, av.y); av.z = fmaf(ps, ov.z, av.z); av.w = fmaf(ps, ov.w, av.w);
        ak.x = fmaf(ds, qv.x, ak.x); ak.y = fmaf(ds, qv.y, ak.y); ak.z = fmaf(ds, qv.z, ak.z); ak.w = fmaf(ds, qv.w, ak.w);
      }
      EO* dkp = reinterpret_cast<EO*>(p.dk) + (int64_t)b * p.sdk[0] + (int64_t)j * p.sdk[1] + (int64_t)kvh * p.sdk[2] + 4 * c4;
      EO* dvp = reinterpret_cast<EO*>(p.dv) + (int64_t)b * p.sdv[0] + (int64_t)j * p.sdv[1] + (int64_t)kvh * p.sdv[2] + 4 * c4;
      const float sc = p.scale;
      // dK and dV are written once and never read here: nontemporal stores
      // (a null dK or dV is not wanted and not written)
      if constexpr (std::is_same<EO, float>::value) {
        if (p.dk) __builtin_nontemporal_store(f32x4{ak.x * sc, ak.y * sc, ak.z * sc, ak.w * sc}, reinterpret_cast<f32x4*>(dkp));
        if (p.dv) __builtin_nontemporal_store(f32x4{av.x, av.y, av.z, av.w}, reinterpret_cast<f32x4*>(dvp));
      } else {
        if (p.dk)
          __builtin_nontemporal_store(bf16x4{(__bf16)(ak.x * sc), (__bf16)(ak.y * sc), (__bf16)(ak.z * sc), (__bf16)(ak.w * sc)},
                                      reinterpret_cast<bf16x4*>(dkp));
        if (p.dv)
          __builtin_nontemporal_store(bf16x4{(__bf16)av.x, (__bf16)av.y, (__bf16)av.z, (__bf16)av.w},
                                      reinterpret_cast<bf16x4*>(dvp));
      }
    }
  }

  // dQ_r = scale sum_c exp(m_c - lse_r) (A_c - D_r B_c); D_r B_c is rounded on its own,
  // so for a single visible key A_c and D_r B_c are the same rounded product and cancel.
  if (pre) {
    if (o < o1) {
      const int r = o / D, h = kvh * G + r / Tq, i = r % Tq;
      const float lse = sLse[r], Dr = sDl[r];
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < kPreCh; ++c) {
        const float w = pm[c] == -INFINITY ? 0.f : expf(pm[c] - lse);
        acc += w * (pa[c] - __fmul_rn(Dr, pb[c]));
      }
      EO* dqp = reinterpret_cast<EO*>(p.dq) + (int64_t)b * p.sdq[0] + (int64_t)i * p.sdq[1] + (int64_t)h * p.sdq[2];
      dqp[o % D] = from_f32<EO>(acc * p.scale);
    }
  } else {
    for (int oo = o0 + tid; oo < o1; oo += kThreads) {
      const int r = oo / D, d = oo % D;
      const int h = kvh * G + r / Tq, i = r % Tq;
      const int64_t row = ((int64_t)b * p.Hq + h) * Tq + i;
      const float lse = sLse[r], Dr = sDl[r];
      const float* st = ws.stats + row * nch * 3;
      float acc = 0.f;
#pragma unroll 8
      for (int c = 0; c < nch; ++c) {
        const float mc = st[3 * c];
        const int64_t e = ((int64_t)c * rows + row) * D + d;
        const float w = mc == -INFINITY ? 0.f : expf(mc - lse);
        acc += w * (ws.a[e] - __fmul_rn(Dr, ws.bk[e]));
      }
      EO* dqp = reinterpret_cast<EO*>(p.dq) + (int64_t)b * p.sdq[0] + (int64_t)i * p.sdq[1] + (int64_t)h * p.sdq[2];
      dqp[d] = from_f32<EO>(acc * p.scale);
    }
  }
}

template <typename E, typename EO, int D>
hipError_t decode_dispatch(const AttnParams& p, void* wsp, hipStream_t s, KernelEvents e1, KernelEvents e2) {
  const int nch = (p.Tk + kCH - 1) / kCH;
  DecodeWs ws = carve(p, wsp);
  const dim3 grid(nch, p.Hkv, p.B);
  const int R = (p.Hq / p.Hkv) * p.Tq;
  const size_t lds = (size_t)((2 * R + kCH) * (D + 4) + 2 * R * kCH) * sizeof(float);   // <= 59 KB at R = 16
  // Keys in one chunk: one fused launch, bitwise equal to the two below. A timed call (caller
  // events given) keeps its two kernels.
  const bool timed = e1.start || e1.stop || e2.start || e2.stop;
  if (nch == 1 && !timed) {
    launch_kernel(decode_chunk_kernel<E, EO, D, true>, grid, dim3(kThreads), (uint32_t)lds, s, e1, p, ws, nch);
    return hipGetLastError();
  }
  launch_kernel(decode_chunk_kernel<E, float, D, false>, grid, dim3(kThreads), (uint32_t)lds, s, e1, p, ws, nch);
  launch_kernel(decode_grads_kernel<E, EO, D>, grid, dim3(kThreads), 0, s, e2, p, ws, nch);
  return hipGetLastError();
}

}  // namespace

bool decode_applicable(const AttnParams& p) {
  return p.Tq >= 1 && (int64_t)(p.Hq / p.Hkv) * p.Tq <= kMaxRows && (p.D == 64 || p.D == 128);
}

size_t decode_workspace_bytes(const AttnParams& p) {
  const int64_t nch = (p.Tk + kCH - 1) / kCH;
  const int64_t rows = (int64_t)p.B * p.Hq * p.Tq;
  const int64_t floats = 2 * align_up(rows * p.Tk) + align_up(rows * nch * 3) + 2 * align_up(nch * rows * p.D);
  return (size_t)floats * sizeof(float);
}

hipError_t launch_decode(const AttnParams& p, void* ws, hipStream_t s, KernelEvents e1, KernelEvents e2) {
  if (p.in_bf16) {
    if (p.out_bf16) return p.D == 128 ? decode_dispatch<__bf16, __bf16, 128>(p, ws, s, e1, e2) : decode_dispatch<__bf16, __bf16, 64>(p, ws, s, e1, e2);
    return p.D == 128 ? decode_dispatch<__bf16, float, 128>(p, ws, s, e1, e2) : decode_dispatch<__bf16, float, 64>(p, ws, s, e1, e2);
  }
  if (p.out_bf16) return p.D == 128 ? decode_dispatch<float, __bf16, 128>(p, ws, s, e1, e2) : decode_dispatch<float, __bf16, 64>(p, ws, s, e1, e2);
  return p.D == 128 ? decode_dispatch<float, float, 128>(p, ws, s, e1, e2) : decode_dispatch<float, float, 64>(p, ws, s, e1, e2);
}

}  // namespace vtb
