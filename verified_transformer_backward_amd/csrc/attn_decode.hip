// Decode-shaped attention backward (few query rows per kv-head group, long KV cache).
//
// Same chain as the flash path ("Hesper.Training.VerifiedBackward", section "Attention
// (full single-head)": attentionBackwardQ / attentionBackwardV), organised for the
// case the single-query specs describe: R = (Hq/Hkv) * Tq <= 16 query rows share one
// kv-head, so the work is reading K and V once and writing dK and dV once.
//
// The KV cache is split into 64-key chunks (the tiled split-KV statistics idea the
// Hesper commit log uses for long caches: per-tile max, sum of exponentials, merged
// afterwards). Three launches:
//   scores  per (chunk, kv-head, batch): s = scale q.k and dP = dO.v for every row and
//           key of the chunk, plus per-row chunk statistics m_c = max s,
//           l_c = sum exp(s - m_c), u_c = sum exp(s - m_c) dP.
//   grads   per (chunk, kv-head, batch): merges all chunks' statistics into lse (unless
//           given) and D = rowsum(P o dP) = sum_c exp(m_c - lse) u_c, forms P and dS for
//           the chunk, writes dV_j = sum_rows P dO and dK_j = scale sum_rows dS q (rows
//           in fixed head-then-query order) and a per-chunk dQ partial scale dS K.
//   reduce  dQ = sum over chunks of the partials (fixed order, no atomics).
#include "device_common.h"
#include "launch.h"

namespace vtb {
namespace {

constexpr int kCH = 64;        // keys per chunk
constexpr int kMaxRows = 16;   // query rows per kv-head group
constexpr int kThreads = 256;

struct DecodeWs {
  float* s;        // [B, Hq, Tq, Tk] scaled scores (-inf where invisible)
  float* dp;       // [B, Hq, Tq, Tk]
  float* stats;    // [B, Hq, Tq, nch, 3] = (m_c, l_c, u_c)
  float* dq_part;  // [nch, B, Hq, Tq, D]
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
  w.dq_part = f;
  return w;
}

template <typename E>
__device__ __forceinline__ const E* rp(const void* base, const int64_t* st, int b, int t, int h) {
  return reinterpret_cast<const E*>(base) + (int64_t)b * st[0] + (int64_t)t * st[1] + (int64_t)h * st[2];
}

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void decode_scores_kernel(AttnParams p, DecodeWs ws, int nch) {
  const int ch = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = p.Hq / p.Hkv, R = G * p.Tq, Tq = p.Tq, Tk = p.Tk;
  const int j0 = ch * kCH;
  __shared__ float sq[kMaxRows][D], sdo[kMaxRows][D];
  __shared__ float sk[kCH][D + 1], sv[kCH][D + 1];
  const int tid = threadIdx.x;
  for (int idx = tid; idx < R * D; idx += kThreads) {
    const int r = idx / D, d = idx % D;
    const int h = kvh * G + r / Tq, i = r % Tq;
    sq[r][d] = to_f32(rp<E>(p.q, p.sq, b, i, h)[d]);
    sdo[r][d] = to_f32(rp<E>(p.dout, p.sdo, b, i, h)[d]);
  }
  for (int idx = tid; idx < kCH * D; idx += kThreads) {
    const int jj = idx / D, d = idx % D;
    const int j = j0 + jj;
    sk[jj][d] = j < Tk ? to_f32(rp<E>(p.k, p.sk, b, j, kvh)[d]) : 0.f;
    sv[jj][d] = j < Tk ? to_f32(rp<E>(p.v, p.sv, b, j, kvh)[d]) : 0.f;
  }
  __syncthreads();
  const int jj = tid & 63, rg = tid >> 6;
  const int j = j0 + jj;
  for (int r = rg; r < R; r += kThreads / 64) {  // r is uniform across the wave
    const int h = kvh * G + r / Tq, i = r % Tq;
    float s = 0.f, dp = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) {
      s = fmaf(sq[r][d], sk[jj][d], s);
      dp = fmaf(sdo[r][d], sv[jj][d], dp);
    }
    s *= p.scale;
    const bool vis = j < Tk && (!p.causal || j <= i + Tk - Tq);
    const int64_t row = ((int64_t)b * p.Hq + h) * Tq + i;
    if (j < Tk) {
      ws.s[row * Tk + j] = vis ? s : -INFINITY;
      ws.dp[row * Tk + j] = dp;
    }
    const float m = wave_max(vis ? s : -INFINITY);
    const float e = (vis && m != -INFINITY) ? expf(s - m) : 0.f;
    const float l = wave_sum(e);
    const float u = wave_sum(e * dp);
    if (jj == 0) {
      float* st = ws.stats + (row * nch + ch) * 3;
      st[0] = m;
      st[1] = l;
      st[2] = u;
    }
  }
}

template <typename E, typename EO, int D>
__global__ __launch_bounds__(kThreads) void decode_grads_kernel(AttnParams p, DecodeWs ws, int nch) {
  const int ch = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = p.Hq / p.Hkv, R = G * p.Tq, Tq = p.Tq, Tk = p.Tk;
  const int j0 = ch * kCH;
  __shared__ float sq[kMaxRows][D], sdo[kMaxRows][D];
  __shared__ float sP[kMaxRows][kCH], sdS[kMaxRows][kCH];
  __shared__ float sLse[kMaxRows], sDl[kMaxRows];
  const int tid = threadIdx.x;

  // merge every chunk's statistics for each row (16 lanes per row)
  {
    const int r = tid >> 4, cl = tid & 15;
    if (r < R) {  // uniform within each 16-lane group
      const int h = kvh * G + r / Tq, i = r % Tq;
      const int64_t row = ((int64_t)b * p.Hq + h) * Tq + i;
      const float* st = ws.stats + row * nch * 3;
      float M = -INFINITY;
      for (int c = cl; c < nch; c += 16) M = fmaxf(M, st[3 * c]);
      M = group16_max(M);
      float L = 0.f, U = 0.f;
      for (int c = cl; c < nch; c += 16) {
        const float mc = st[3 * c];
        const float wgt = mc == -INFINITY ? 0.f : expf(mc - M);
        L += st[3 * c + 1] * wgt;
        U += st[3 * c + 2] * wgt;
      }
      L = group16_sum(L);
      U = group16_sum(U);
      const float lse = p.lse ? p.lse[row] : M + logf(L);
      if (cl == 0) {
        sLse[r] = lse;
        sDl[r] = U * expf(M - lse);
      }
    }
  }
  for (int idx = tid; idx < R * D; idx += kThreads) {
    const int r = idx / D, d = idx % D;
    const int h = kvh * G + r / Tq, i = r % Tq;
    sq[r][d] = to_f32(rp<E>(p.q, p.sq, b, i, h)[d]);
    sdo[r][d] = to_f32(rp<E>(p.dout, p.sdo, b, i, h)[d]);
  }
  __syncthreads();
  for (int idx = tid; idx < R * kCH; idx += kThreads) {
    const int r = idx / kCH, jj = idx % kCH;
    const int j = j0 + jj;
    const int h = kvh * G + r / Tq, i = r % Tq;
    const int64_t row = ((int64_t)b * p.Hq + h) * Tq + i;
    float pr = 0.f, ds = 0.f;
    if (j < Tk) {
      const float s = ws.s[row * Tk + j];
      pr = s == -INFINITY ? 0.f : expf(s - sLse[r]);
      ds = pr * (ws.dp[row * Tk + j] - sDl[r]);
    }
    sP[r][jj] = pr;
    sdS[r][jj] = ds;
  }
  __syncthreads();

  // dK, dV rows of this chunk: thread owns column d, keys jj = tid / D + k * (256 / D)
  {
    const int d = tid % D;
    for (int jj = tid / D; jj < kCH; jj += kThreads / D) {
      const int j = j0 + jj;
      if (j >= Tk) break;
      float ak = 0.f, av = 0.f;
      for (int r = 0; r < R; ++r) {
        av = fmaf(sP[r][jj], sdo[r][d], av);
        ak = fmaf(sdS[r][jj], sq[r][d], ak);
      }
      EO* dkp = reinterpret_cast<EO*>(p.dk) + (int64_t)b * p.sdk[0] + (int64_t)j * p.sdk[1] + (int64_t)kvh * p.sdk[2];
      EO* dvp = reinterpret_cast<EO*>(p.dv) + (int64_t)b * p.sdv[0] + (int64_t)j * p.sdv[1] + (int64_t)kvh * p.sdv[2];
      dkp[d] = from_f32<EO>(ak * p.scale);
      dvp[d] = from_f32<EO>(av);
    }
  }
  // dQ partial of this chunk: thread owns column d, rows r = tid / D + k * (256 / D)
  {
    const int d = tid % D;
    const int jn = min(kCH, Tk - j0);
    for (int r = tid / D; r < R; r += kThreads / D) {
      const int h = kvh * G + r / Tq, i = r % Tq;
      float a = 0.f;
      for (int jj = 0; jj < jn; ++jj) a = fmaf(sdS[r][jj], to_f32(rp<E>(p.k, p.sk, b, j0 + jj, kvh)[d]), a);
      ws.dq_part[((((int64_t)ch * p.B + b) * p.Hq + h) * Tq + i) * D + d] = a * p.scale;
    }
  }
}

template <typename EO>
__global__ __launch_bounds__(256) void decode_dq_reduce_kernel(const float* __restrict__ part, int nch, EO* dq,
                                                               int B, int Hq, int Tq, int D, int64_t s0, int64_t s1,
                                                               int64_t s2) {
  const int64_t n = (int64_t)B * Hq * Tq * D;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
    float a = 0.f;
    for (int c = 0; c < nch; ++c) a += part[(int64_t)c * n + idx];
    const int d = idx % D;
    int64_t rest = idx / D;
    const int i = rest % Tq;
    rest /= Tq;
    const int h = rest % Hq;
    const int b = rest / Hq;
    dq[b * s0 + i * s1 + h * s2 + d] = from_f32<EO>(a);
  }
}

template <typename E, typename EO, int D>
hipError_t decode_dispatch(const AttnParams& p, void* wsp, hipStream_t s) {
  const int nch = (p.Tk + kCH - 1) / kCH;
  DecodeWs ws = carve(p, wsp);
  const dim3 grid(nch, p.Hkv, p.B);
  hipLaunchKernelGGL((decode_scores_kernel<E, D>), grid, dim3(kThreads), 0, s, p, ws, nch);
  hipLaunchKernelGGL((decode_grads_kernel<E, EO, D>), grid, dim3(kThreads), 0, s, p, ws, nch);
  const int64_t n = (int64_t)p.B * p.Hq * p.Tq * D;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL((decode_dq_reduce_kernel<EO>), dim3(blocks), dim3(256), 0, s, ws.dq_part, nch,
                     reinterpret_cast<EO*>(p.dq), p.B, p.Hq, p.Tq, D, p.sdq[0], p.sdq[1], p.sdq[2]);
  return hipGetLastError();
}

}  // namespace

bool decode_applicable(const AttnParams& p) {
  return p.Tq >= 1 && (int64_t)(p.Hq / p.Hkv) * p.Tq <= kMaxRows && (p.D == 64 || p.D == 128);
}

size_t decode_workspace_bytes(const AttnParams& p) {
  const int64_t nch = (p.Tk + kCH - 1) / kCH;
  const int64_t rows = (int64_t)p.B * p.Hq * p.Tq;
  const int64_t floats = 2 * align_up(rows * p.Tk) + align_up(rows * nch * 3) + align_up(nch * rows * p.D);
  return (size_t)floats * sizeof(float);
}

hipError_t launch_decode(const AttnParams& p, void* ws, hipStream_t s) {
  if (p.in_bf16) {
    if (p.out_bf16) return p.D == 128 ? decode_dispatch<__bf16, __bf16, 128>(p, ws, s) : decode_dispatch<__bf16, __bf16, 64>(p, ws, s);
    return p.D == 128 ? decode_dispatch<__bf16, float, 128>(p, ws, s) : decode_dispatch<__bf16, float, 64>(p, ws, s);
  }
  if (p.out_bf16) return p.D == 128 ? decode_dispatch<float, __bf16, 128>(p, ws, s) : decode_dispatch<float, __bf16, 64>(p, ws, s);
  return p.D == 128 ? decode_dispatch<float, float, 128>(p, ws, s) : decode_dispatch<float, float, 64>(p, ws, s);
}

}  // namespace vtb
