// Internal interface between the C-ABI layer (api.cpp) and the kernel translation units.
// Everything here is already validated by the caller; launchers only compute grids.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vtb {

// Attention backward problem after validation. Element pointers are typed by in_bf16 /
// out_bf16; strides are (batch, token, head) in elements with the head dim contiguous.
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;   // row log-sum-exp read by the backward (given or workspace)
  const float* P;     // saved softmax [B, Hq, Tq, Tk] or nullptr
  const void* o;      // the forward's saved output [B, Tq, Hq, D] (ROW_D_GIVEN), strides so
  float* lse_out;     // where a pass that computes lse writes it
  float* dlt;         // workspace [B, Hq, Tq]: D_i = rowsum(P o dP)
  float* lse2;        // workspace [B, Hq, Tq]: lse_i * log2(e), written by the MFMA dq pass for its dk/dv pass
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, Tq, Tk, D;
  float scale;
  int causal;
  int in_bf16, out_bf16;
  int64_t sq[3], sk[3], sv[3], sdo[3], sdq[3], sdk[3], sdv[3], so[3];
};

// Optional timing of one kernel: HIP events that the dispatch itself records at the
// kernel's start and end (hipExtLaunchKernelGGL), so no separate event packet lies
// between them. Empty: an ordinary launch.
struct KernelEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
                          KernelEvents ev, Args... args) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
}

// How the query-parallel pass obtains P: from the given lse, by computing lse itself
// (online max/sum), lse only (no backward), or from a saved softmax P. ROW_FWD is the
// forward: O = softmax(scale Q K^T) V by online softmax, written through dq / sdq, and
// lse written to lse_out when that is not null.
// ROW_D_GIVEN takes the given lse and the forward's saved output o: the row term is
// D_i = dO_i . O_i (fp32 sum of in-dtype products, formed from the rows the pass loads
// anyway and written to dlt), then one sweep forms dQ.
enum RowMode { ROW_LSE_GIVEN = 0, ROW_LSE_COMPUTE = 1, ROW_LSE_ONLY = 2, ROW_P_GIVEN = 3, ROW_FWD = 4, ROW_D_GIVEN = 5 };

// Flash-style path (any Tq): query-parallel pass (row term D, lse when computed, dQ),
// then key-parallel pass (dK, dV). The second reads D (and lse) written by the first.
hipError_t launch_flash_dq(const AttnParams& p, int mode, hipStream_t s, KernelEvents ev = {});
hipError_t launch_flash_dkdv(const AttnParams& p, hipStream_t s, KernelEvents ev = {});

// bf16, head dim 128: MFMA tiles fed by double-buffered direct-to-LDS loads of 64-row
// blocks. The dq pass takes a given lse (single sweep; writes dQ and D); the dk/dv pass
// takes lse and D from the workspace or the caller, like launch_flash_dkdv.
bool mfma_path_applicable(const AttnParams& p);
// MFMA forward (bf16, D = 128): O and lse by online softmax, O written through dq / sdq.
bool mfma_fwd_applicable(const AttnParams& p);
hipError_t launch_mfma_fwd(const AttnParams& p, hipStream_t s, KernelEvents ev = {});
// d_given: D = dO . O from the saved output o (written to dlt) and dQ = scale (P o (dP - D)) K
// takes three contractions per key block instead of four.
hipError_t launch_mfma_dq(const AttnParams& p, hipStream_t s, KernelEvents ev = {}, bool d_given = false);
hipError_t launch_mfma_dkdv(const AttnParams& p, hipStream_t s, KernelEvents ev = {});

// Decode path (Hq/Hkv * Tq <= 16): a chunk pass (scores, dP, split-KV statistics, dQ
// pieces; reads K and V once) and a gradient pass (dK, dV, dQ; no K/V reads). Workspace
// layout is owned by attn_decode.hip.
size_t decode_workspace_bytes(const AttnParams& p);
bool decode_applicable(const AttnParams& p);
hipError_t launch_decode(const AttnParams& p, void* ws, hipStream_t s, KernelEvents ev_chunk = {},
                         KernelEvents ev_grads = {});

// Split-KV decode forward (Hq/Hkv * Tq <= 16): per 64-key chunk the rows' partial
// (max, sum of exponentials, weighted value sum) in the workspace, then a merge into O
// (written through dq / sdq) and lse (lse_out, when not null).
bool decode_fwd_applicable(const AttnParams& p);
size_t decode_fwd_workspace_bytes(const AttnParams& p);
hipError_t launch_decode_fwd(const AttnParams& p, void* ws, hipStream_t s);

// Fill `n` floats with zero (graph-capture safe, no hipMemsetAsync).
hipError_t launch_zero_f32(float* x, int64_t n, hipStream_t s);
// Zero a strided [B, T, H, D] tensor of fp32 or bf16 elements.
hipError_t launch_zero_bthd(void* x, int bf16, int B, int T, int H, int D, const int64_t st[3], hipStream_t s,
                            KernelEvents ev = {});

// Elementwise tail.
// RoPE and RMSNorm backward in fp32 or bf16 storage (bf16 != 0), fp32 arithmetic; gamma
// stays fp32.
hipError_t launch_rope_bwd(int bf16, const void* dy, void* dx, int n_tok, int n_heads, int head_dim,
                           int64_t tok_stride, const int32_t* pos, int pos0, double base, int layout, hipStream_t s);
hipError_t launch_rmsnorm_bwd(int bf16, const void* x, const float* gamma, const void* dy, void* dx, int rows, int n,
                              float eps, hipStream_t s);
hipError_t launch_rope_rmsnorm_res_bwd(const float* dq, float dq_scale, const float* x,
                                       const float* gamma, const float* dh_out, float* dh_in, int T,
                                       int n_heads, int head_dim, int pos0, double base, int layout,
                                       float eps, hipStream_t s);

// LayerNorm (no affine) backward from the forward's y and sigma, rows of n values, fp32 or
// bf16 storage (bf16 != 0) with fp32 arithmetic; sigma is fp32. dres (may be null) is a
// residual gradient added to the result; dx == dres is allowed.
hipError_t launch_layernorm_bwd(int bf16, const void* dy, const void* y, const float* sig, const void* dres, void* dx,
                                int rows, int n, hipStream_t s);
// ReLU^2 x Mul backward over n elements, fp32 or bf16 storage.
hipError_t launch_relu2_mul_bwd(int bf16, const void* gate, const void* up, const void* dh, void* dgate, void* dup,
                                int64_t n, hipStream_t s);

// FFN block pieces (fp32): the sub-norm backward fused with ReLU^2 x Mul backward over
// [T, 2F] gate|up rows (dgu gets dgate|dup), and RMSNorm backward plus a residual
// (dx = dres + RMSNormBackward(x, gamma, dy); dx == dres allowed).
hipError_t launch_subnorm_relu2_bwd(const float* gu, const float* dhn, const float* gamma2, float* dgu, int T, int F,
                                    float eps, hipStream_t s);
hipError_t launch_rmsnorm_res_bwd(const float* x, const float* gamma, const float* dy, const float* dres, float* dx,
                                  int T, int n, float eps, hipStream_t s, float* rinv = nullptr);
// RMSNorm gain gradient: dgamma[c] = sum_t dy[t, c] x[t, c] rinv[t] over rows t (rinv from
// launch_rmsnorm_res_bwd), summed in a fixed order.
hipError_t launch_rmsnorm_gamma(const float* x, const float* dy, const float* rinv, float* dgamma, int rows, int n,
                                hipStream_t s);

// fp32 MFMA GEMMs of the linear backward (one launch computes both products).
hipError_t launch_linear_bwd(const float* x, const float* w, const float* dy, float* dx, float* dw,
                             int T, int K, int N, hipStream_t s);
// The same products with dX's contraction cut into linear_bwd_splits(T, K, N) chunks that
// run as separate tiles (their fp32 partials in `part`, splits * T * K floats, 16-byte
// aligned), then summed into dx in chunk order. For the layer chain, where dX's 2560-deep
// contraction would otherwise be the critical path. dx and dw are both required.
int linear_bwd_splits(int T, int K, int N);
// Attention backward with a saved softmax, as batched fp32 MFMA GEMMs over H heads of a
// [T, ld] activation layout (head h at column h * D; B = 1, Tq = Tk = T): dP = dO V^T into
// ds [H, T, T], dS = P o (dP - D) in place, then dQ = scale dS K, dK = scale dS^T Q and
// dV = P^T dO in one launch. Causal tiles and contraction ranges skip invisible pairs.
hipError_t launch_linear_bwd_split(const float* x, const float* w, const float* dy, float* dx, float* dw, int T, int K,
                                   int N, float* part, hipStream_t s);
hipError_t launch_attn_saved_p_bwd(const float* q, const float* k, const float* v, const float* dout, const float* P,
                                   float* ds, float* dq, float* dk, float* dv, int T, int H, int D, int ld, float scale,
                                   int causal, hipStream_t s);
// The same with separate row strides: ld_in for q, k, v; ld_do for dout; ld_out for dq,
// dk, dv (q, k, v and their gradients can then sit in one [T, 3C] row).
hipError_t launch_attn_saved_p_bwd_ld(const float* q, const float* k, const float* v, const float* dout, const float* P,
                                      float* ds, float* dq, float* dk, float* dv, int T, int H, int D, int ld_in,
                                      int ld_do, int ld_out, float scale, int causal, hipStream_t s);
// The linear backward with dX's split-K partials left in part (ns_out = their count; 1
// means dX went straight to dx and part is unused), for a consumer that sums them itself.
hipError_t launch_linear_bwd_parts(const float* x, const float* w, const float* dy, float* dx, float* dw, int T, int K,
                                   int N, float* part, int* ns_out, hipStream_t s);
// Attention backward with a saved P whose dO arrives as ns split-K partials (part + s
// part_stride, rows of ld_do; ns = 1: part is dO itself). For T <= 512 and D in {32, 64,
// 128} one kernel sums the partials, writes dO to dout (for dV), forms dP on the matrix
// cores and D and dS in its epilogue; otherwise the partials are summed into dout and the
// dP product and the dS rows run as two launches. Then the dQ/dK/dV launch.
hipError_t launch_attn_saved_p_bwd_parts(const float* q, const float* k, const float* v, const float* part, int ns,
                                         int64_t part_stride, float* dout, const float* P, float* ds, float* dq,
                                         float* dk, float* dv, int T, int H, int D, int ld_in, int ld_do, int ld_out,
                                         float scale, int causal, hipStream_t s);

}  // namespace vtb
