// Decode-shaped attention forward by split-KV: O and lse for few query rows per kv-head
// group over a long KV cache, reading K and V once.
//
// The Hesper commit log's tiled flash-attention entry describes it: Phase 1 computes, per
// KV tile in parallel, a partial output with the tile's running maximum and sum of
// exponentials; Phase 2 merges the tiles' partials. The result equals the standard
// scores -> softmax -> apply form ("Hesper.Training.VerifiedBackward", section "Scaled
// Dot-Product": scores scale q.k; softmax; weighted sum of values).
//
//   chunk  per (64-key chunk, kv-head, batch): K and V read once. For every row r of the
//          group (R = (Hq/Hkv) Tq <= 16 rows: q-head kvh G + r / Tq, query r % Tq) and key
//          j: s = scale q.k on the fp32 matrix cores; m_c = max over the visible keys,
//          e = exp(s - m_c), l_c = sum e, o_c = sum_j e v_j (a D-vector per row).
//   merge  per query row: m = max_c m_c, w_c = exp(m_c - m), l = sum w_c l_c,
//          O = (sum w_c o_c) / l and lse = m + ln l.
// Every reduction runs in a fixed order (O's sum chunk by chunk, l's over a fixed wave
// tree): results are bitwise reproducible.
#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace vtb {
namespace {

constexpr int kCH = 64;         // keys per chunk
constexpr int kMaxRows = 16;    // query rows per kv-head group
constexpr int kThreads = 256;

struct FwdWs {
  float* o;       // [nch, rows, D] partial sum_j e v_j
  float* stats;   // [nch, rows, 2] = (m_c, l_c); m_c = -inf when no key of the chunk is visible
};

__host__ __device__ inline int64_t align64(int64_t x) { return (x + 63) / 64 * 64; }

FwdWs carve(const AttnParams& p, void* base) {
  const int64_t nch = (p.Tk + kCH - 1) / kCH, rows = (int64_t)p.B * p.Hq * p.Tq;
  float* f = reinterpret_cast<float*>(base);
  FwdWs w;
  w.o = f;
  w.stats = f + align64(nch * rows * p.D);
  return w;
}

template <typename E>
__device__ __forceinline__ const E* rp(const void* base, const int64_t* st, int b, int t, int h) {
  return reinterpret_cast<const E*>(base) + (int64_t)b * st[0] + (int64_t)t * st[1] + (int64_t)h * st[2];
}

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void decode_fwd_chunk_kernel(AttnParams p, FwdWs ws, int nch) {
  constexpr int LD = D + 4;   // padded fp32 rows: a 16-lane operand read covers every bank once
  constexpr int V = 16 / sizeof(E), CV = D / V, NL = kCH * CV / kThreads;
  static_assert(NL * kThreads == kCH * CV, "chunk loads must tile the workgroup");
  static_assert(kMaxRows * D / 8 <= kThreads, "one q piece per thread");
  typedef E vec_t __attribute__((ext_vector_type(V)));
  const int ch = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = p.Hq / p.Hkv, R = G * p.Tq, Tq = p.Tq, Tk = p.Tk, off = Tk - Tq;
  const int j0 = ch * kCH, tid = threadIdx.x;
  __shared__ __attribute__((aligned(16))) float skv[kCH * LD];     // K, then V
  __shared__ __attribute__((aligned(16))) float sq[kMaxRows * LD];
  __shared__ float se[kMaxRows][kCH];                              // s, then e

  // q first (one 8-element piece per thread: R * D / 8 <= 256), then every K and V load
  // of the chunk; rows past Tk re-read row Tk - 1. Loads complete in issue order, so q
  // and K are waited for while V is still in flight.
  constexpr int C8 = D / 8;
  const bool has_q = tid < R * C8;
  frag_t<E> q8;
  if (has_q) q8 = load8<E>(rp<E>(p.q, p.sq, b, (tid / C8) % Tq, kvh * G + (tid / C8) / Tq) + 8 * (tid % C8));
  vec_t kreg[NL], vreg[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int f = tid + kThreads * i, row = f / CV, cv = f % CV;
    const int j = min(j0 + row, Tk - 1);
    kreg[i] = *reinterpret_cast<const vec_t*>(rp<E>(p.k, p.sk, b, j, kvh) + V * cv);
  }
  __builtin_amdgcn_sched_barrier(0);   // keep every K load ahead of the V loads
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int f = tid + kThreads * i, row = f / CV, cv = f % CV;
    const int j = min(j0 + row, Tk - 1);
    vreg[i] = *reinterpret_cast<const vec_t*>(rp<E>(p.v, p.sv, b, j, kvh) + V * cv);
  }
  if (has_q) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sq[(tid / C8) * LD + 8 * (tid % C8) + e] = to_f32(q8[e]);
  }
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
  to_lds(kreg);
  __syncthreads();
  // s = scale q.k on the fp32 matrix cores (16x16x4): wave w takes keys 16 w .. 16 w + 15
  // as the rows of A and the group's rows as the columns of B (columns past R re-read row
  // R - 1 and are not stored). Lane (c, g) holds d = d0 + 4 g .. 4 g + 3 of its A row and
  // B column; register r of the result is key 16 w + 4 g + r of row c.
  {
    const int lane = tid & 63, w = tid >> 6, mc = lane & 15, mg = lane >> 4;
    const float* arow = skv + (16 * w + mc) * LD + 4 * mg;
    const float* brow = sq + min(mc, R - 1) * LD + 4 * mg;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int d0 = 0; d0 < D; d0 += 16) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(arow + d0);
      const f32x4 bx = *reinterpret_cast<const f32x4*>(brow + d0);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], bx[e], acc, 0, 0, 0);
    }
    if (mc < R) {
#pragma unroll
      for (int r = 0; r < 4; ++r) se[mc][16 * w + 4 * mg + r] = acc[r] * p.scale;
    }
  }
  __syncthreads();   // every read of K is done
  to_lds(vreg);
  // chunk statistics: lane = key, wave = rows w, w + 4, ...
  const int lane = tid & 63, w = tid >> 6, j = j0 + lane;
  const int64_t rows = (int64_t)p.B * p.Hq * Tq;
  for (int r = w; r < R; r += 4) {
    const int i = r % Tq;
    const float s = se[r][lane];
    const bool vis = j < Tk && (!p.causal || j <= i + off);
    const float m = wave_max(vis ? s : -INFINITY);
    const float e = (vis && m != -INFINITY) ? expf(s - m) : 0.f;
    const float l = wave_sum(e);
    se[r][lane] = e;
    if (lane == 0) {
      const int64_t row = ((int64_t)b * p.Hq + kvh * G + r / Tq) * Tq + i;
      float* st = ws.stats + ((int64_t)ch * rows + row) * 2;
      st[0] = m;
      st[1] = l;
    }
  }
  __syncthreads();
  // o_c = sum_j e v_j on the fp32 matrix cores: the rows of A are the group's rows (rows
  // past R re-read row R - 1 and are not stored), k runs over the chunk's keys, and wave w
  // takes the 16-column tiles w, w + 4, ... of V. Register r of lane (c, g) is row 4 g + r,
  // column c of the tile.
  {
    const float* erow = &se[min(lane & 15, R - 1)][lane >> 4];
    const int mc = lane & 15, mg = lane >> 4;
    for (int ct = w; ct < D / 16; ct += 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < kCH; k0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(erow[k0], skv[(k0 + mg) * LD + 16 * ct + mc], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = 4 * mg + r;
        if (rr < R) {
          const int64_t row = ((int64_t)b * p.Hq + kvh * G + rr / Tq) * Tq + rr % Tq;
          ws.o[((int64_t)ch * rows + row) * D + 16 * ct + mc] = acc[r];
        }
      }
    }
  }
}

// One wave per query row. The partial sums of the first kPF chunks are loaded before the
// statistics (one chunk per lane, chunks c, c + 64, ... per lane) are reduced across the
// wave, so both reads are in flight together; lane l then accumulates columns 2 l, 2 l + 1
// (D = 128) or l (D = 64) over the chunks in order. A chunk with no visible key has
// m_c = -inf, weight 0 and o_c = 0.
constexpr int kPF = 16;

template <typename EO, int D>
__global__ __launch_bounds__(kThreads) void decode_fwd_merge_kernel(AttnParams p, FwdWs ws, int nch) {
  constexpr int PER = D / 64;
  typedef float vec_t __attribute__((ext_vector_type(PER)));
  const int64_t rows = (int64_t)p.B * p.Hq * p.Tq;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const float* obase = ws.o + row * D + PER * lane;
  const int64_t ostride = rows * D;   // from one chunk's partial to the next
  vec_t pre[kPF];
#pragma unroll
  for (int i = 0; i < kPF; ++i)
    if (i < nch) pre[i] = *reinterpret_cast<const vec_t*>(obase + i * ostride);
  auto stat = [&](int c) { return *reinterpret_cast<const float2*>(ws.stats + ((int64_t)c * rows + row) * 2); };
  const float2 s0 = lane < nch ? stat(lane) : make_float2(-INFINITY, 0.f);
  float m = s0.x;
  for (int c = lane + 64; c < nch; c += 64) m = fmaxf(m, stat(c).x);
  m = wave_max(m);
  const float w0 = s0.x == -INFINITY ? 0.f : expf(s0.x - m);
  float l = w0 * s0.y;
  for (int c = lane + 64; c < nch; c += 64) {
    const float2 st = stat(c);
    l += st.x == -INFINITY ? 0.f : expf(st.x - m) * st.y;
  }
  l = wave_sum(l);
  vec_t acc = {};
#pragma unroll
  for (int i = 0; i < kPF; ++i) {
    const float wc = __shfl(w0, i);
    if (i < nch) {
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(wc, pre[i][e], acc[e]);
    }
  }
  for (int c0 = 0; c0 < nch; c0 += 64) {
    float wl = w0;
    if (c0 > 0) {
      const float mc = c0 + lane < nch ? stat(c0 + lane).x : -INFINITY;
      wl = mc == -INFINITY ? 0.f : expf(mc - m);
    }
    const int n = min(64, nch - c0);
    for (int i = c0 == 0 ? kPF : 0; i < n; i += 8) {   // eight chunks' loads in flight
      vec_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i + u < n) v[u] = *reinterpret_cast<const vec_t*>(obase + (int64_t)(c0 + i + u) * ostride);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wc = __shfl(wl, (i + u) & 63);
        if (i + u < n) {
#pragma unroll
          for (int e = 0; e < PER; ++e) acc[e] = fmaf(wc, v[u][e], acc[e]);
        }
      }
    }
  }
  const int i = (int)(row % p.Tq), h = (int)((row / p.Tq) % p.Hq), b = (int)(row / ((int64_t)p.Tq * p.Hq));
  EO* o = reinterpret_cast<EO*>(p.dq) + (int64_t)b * p.sdq[0] + (int64_t)i * p.sdq[1] + (int64_t)h * p.sdq[2] + PER * lane;
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = from_f32<EO>(acc[e] * inv);
  if (p.lse_out && lane == 0) p.lse_out[row] = m + logf(l);
}

template <typename E, typename EO, int D>
hipError_t dispatch(const AttnParams& p, void* ws, hipStream_t s) {
  const int nch = (p.Tk + kCH - 1) / kCH;
  const FwdWs w = carve(p, ws);
  hipLaunchKernelGGL((decode_fwd_chunk_kernel<E, D>), dim3(nch, p.Hkv, p.B), dim3(kThreads), 0, s, p, w, nch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)p.B * p.Hq * p.Tq;
  const int per = kThreads / 64;
  hipLaunchKernelGGL((decode_fwd_merge_kernel<EO, D>), dim3((unsigned)((rows + per - 1) / per)), dim3(kThreads), 0, s,
                     p, w, nch);
  return hipGetLastError();
}

}  // namespace

bool decode_fwd_applicable(const AttnParams& p) {
  return (p.Hq / p.Hkv) * p.Tq <= kMaxRows && (p.D == 64 || p.D == 128) && p.Tk >= 1 && p.Tq >= 1;
}

size_t decode_fwd_workspace_bytes(const AttnParams& p) {
  const int64_t nch = (p.Tk + kCH - 1) / kCH, rows = (int64_t)p.B * p.Hq * p.Tq;
  return (size_t)(align64(nch * rows * p.D) + align64(nch * rows * 2)) * sizeof(float);
}

hipError_t launch_decode_fwd(const AttnParams& p, void* ws, hipStream_t s) {
  if (p.in_bf16) {
    if (p.out_bf16) return p.D == 128 ? dispatch<__bf16, __bf16, 128>(p, ws, s) : dispatch<__bf16, __bf16, 64>(p, ws, s);
    return p.D == 128 ? dispatch<__bf16, float, 128>(p, ws, s) : dispatch<__bf16, float, 64>(p, ws, s);
  }
  if (p.out_bf16) return p.D == 128 ? dispatch<float, __bf16, 128>(p, ws, s) : dispatch<float, __bf16, 64>(p, ws, s);
  return p.D == 128 ? dispatch<float, float, 128>(p, ws, s) : dispatch<float, float, 64>(p, ws, s);
}

}  // namespace vtb
