/*
 * vtb.h -- C ABI of the MI355X (gfx950) attention-layer backward library (libvtb.so).
 *
 * The operations are the vector-Jacobian products stated on the
 * "Hesper.Training.VerifiedBackward" API page (sections "Softmax", "RoPE (Rotary Position
 * Embedding)", "RMSNorm", "Scaled Dot-Product", "Attention (full single-head)"), the
 * linear backward and per-layer reverse chain of the Hesper pull-request commit log,
 * and the batched causal multi-head form of the DaisyChain-Train transformer.js page
 * (function `backward`).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller. The library never
 *     allocates, frees or keeps caller memory; scratch space comes in through an
 *     explicit `workspace` argument sized by the matching *_workspace_size() query.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream). They
 *     never synchronise; the caller records events or synchronises.
 *   - Every call returns a vtb_status. Arguments are validated before anything is
 *     launched, so a call that fails validation has launched nothing. Outputs are
 *     undefined after any error. vtb_last_error() gives a thread-local detail string.
 *   - Outputs are overwritten, never accumulated into.
 *   - Accumulation is always fp32, whatever the storage type.
 *   - Calls are stateless and may run concurrently on different streams, each with its
 *     own workspace.
 */
#ifndef VTB_H
#define VTB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* vtb_stream_t; /* a hipStream_t */

typedef enum {
  VTB_OK = 0,
  VTB_ERR_ARG = 1,          /* bad shape, stride, NULL pointer or value */
  VTB_ERR_UNSUPPORTED = 2,  /* valid request the library does not implement (e.g. head_dim 96) */
  VTB_ERR_ALIAS = 3,        /* an output overlaps an input or another output */
  VTB_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than the size query returns */
  VTB_ERR_HIP = 5           /* the HIP runtime reported an error at launch */
} vtb_status;

typedef enum { VTB_F32 = 0, VTB_BF16 = 1 } vtb_dtype;

/* Static name of a status code. */
const char* vtb_status_string(int status);
/* Detail of the last failure on the calling thread ("" if none). */
const char* vtb_last_error(void);
/* ABI version: increases when a signature or struct layout changes. */
int vtb_abi_version(void);

/* ---------------------------------------------------------------------------------------
 * Attention backward.
 *
 * "Hesper.Training.VerifiedBackward", section "Attention (full single-head)":
 * attentionBackwardQ (dAttn = dOut . V^T, dScores = softmaxBackward, dQ = scale dScores K)
 * and attentionBackwardV (dV = attn^T dOut), with scaledDotBackwardK for dK, applied to
 * every query row of every head:
 *     P  = exp(scale Q K^T - lse)          (or the saved softmax P when given)
 *     dP = dO V^T;   D = rowsum(P o dP);   dS = P o (dP - D)
 *     dQ = scale dS K;   dK = scale dS^T Q;   dV = P^T dO
 * Causal visibility follows transformer.js (key tj visible to query ti iff tj <= ti),
 * aligned bottom-right when Tq != Tk: key j is visible to query i iff j <= i + Tk - Tq.
 * Grouped queries: q-head h reads kv-head h / (Hq / Hkv); dK and dV sum the group's heads.
 *
 * Layout: q, dout, dq are [B, Tq, Hq, D]; k, v, dk, dv are [B, Tk, Hkv, D], each with its
 * own (batch, token, head) strides in ELEMENTS and D contiguous (stride 1).
 * lse is [B, Hq, Tq] fp32 contiguous: natural-log sum over visible keys of
 * exp(scale q.k). P is [B, Hq, Tq, Tk] fp32 contiguous; entries at invisible
 * positions are ignored. D must be 64 or 128.
 * -------------------------------------------------------------------------------------*/
typedef struct {
  int32_t B, Hq, Hkv, Tq, Tk, D;
  float scale;
  int32_t causal;      /* 0 or 1; causal requires Tk >= Tq */
  int32_t in_dtype;    /* vtb_dtype of q, k, v, dout */
  int32_t out_dtype;   /* vtb_dtype of dq, dk, dv */
  int64_t s_q[3], s_k[3], s_v[3], s_do[3], s_dq[3], s_dk[3], s_dv[3]; /* (b, t, h) strides */
} attn_bwd_desc;

/* Bytes of workspace attn_bwd needs for this descriptor (0 on an invalid descriptor). */
size_t attn_bwd_workspace_size(const attn_bwd_desc* desc);

/* lse: NULL => computed internally from q, k. P: non-NULL => used as the softmax, and
 * lse is ignored. dq must be non-NULL; dk and dv may each be NULL, meaning that gradient
 * is not wanted: it is not written (with both NULL the key-parallel pass is skipped).
 * Outputs must not overlap each other or any input. Tk == 0 is an error; Tq == 0 (or
 * B == 0) writes zero dk, dv (those that are non-NULL). */
int attn_bwd(const attn_bwd_desc* desc, const void* q, const void* k, const void* v,
             const void* dout, const float* lse, const float* P, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes, vtb_stream_t stream);

/* attn_bwd for callers that saved the forward's output O. "Hesper.Training.VerifiedBackward",
 * section "Attention (full single-head)": the apply step gives O_i = sum_j P_ij v_j and
 * dP_ij = dO_i . v_j, so the softmax backward's row term rowsum(P o dP) equals dO_i . O_i.
 * That dot product (one fp32 sum per query row) replaces the pass over every visible key
 * that attn_bwd needs for it: the query-parallel pass then forms dS = P o (dP - D)
 * directly (three contractions per key block instead of four) and the key-parallel pass
 * reads the same D. Results are attn_bwd's up to the rounding of O.
 * o: [B, Tq, Hq, D] in desc->in_dtype, device memory, 16-byte aligned, with element
 * strides s_o[3] (batch, token, head; multiples of 8), read only. lse is required and
 * there is no saved P; every other argument is attn_bwd's (same workspace size).
 * Decode-shaped problems (the decode path of attn_bwd) do not read o: their row term
 * comes from the chunk statistics, which cost no extra K/V read. */
int attn_bwd_o(const attn_bwd_desc* desc, const void* q, const void* k, const void* v,
               const void* dout, const void* o, const int64_t* s_o, const float* lse, void* dq,
               void* dk, void* dv, void* workspace, size_t workspace_bytes, vtb_stream_t stream);

/* attn_bwd for callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops, harnesses that forbid hipMalloc): identical arguments and results except
 * that there is no workspace argument. The workspace is a device array inside the library,
 * one per GPU, attn_bwd_noalloc_max_workspace() bytes (16 MiB), resolved on the first call
 * on each device and held until the process ends; the call itself allocates nothing. The
 * stream must belong to the current device. Calls whose attn_bwd_workspace_size exceeds
 * the array return VTB_ERR_WORKSPACE (use attn_bwd with a caller workspace). Every call on
 * a GPU uses that GPU's one array: calls that overlap in time on one GPU (different
 * streams, or graphs replayed concurrently) race and give undefined results. No part of
 * the array needs clearing between calls: each call writes every value it reads first. */
size_t attn_bwd_noalloc_max_workspace(void);
int attn_bwd_noalloc(const attn_bwd_desc* desc, const void* q, const void* k, const void* v,
                     const void* dout, const float* lse, const float* P, void* dq, void* dk, void* dv,
                     vtb_stream_t stream);

/* attn_bwd with per-kernel timing, for measurement: identical results. Every call runs
 * two kernels on `stream` (flash and MFMA paths: the query-parallel dq pass, then the
 * key-parallel dk/dv pass; decode path: the chunk pass, then the gradient pass, also when
 * the keys fit one 64-key chunk, where attn_bwd runs one fused kernel instead;
 * Tq == 0: the zero fills of dk and dv), and the caller's HIP events (hipEvent_t,
 * created by the caller) are recorded by the dispatches themselves: events[0] and
 * events[1] at the start and end of the first kernel, events[2] and events[3] at the
 * start and end of the second. A call that launches nothing records none. n_events must
 * be >= 4. */
int attn_bwd_timed(const attn_bwd_desc* desc, const void* q, const void* k, const void* v,
                   const void* dout, const float* lse, const float* P, void* dq, void* dk,
                   void* dv, void* workspace, size_t workspace_bytes, vtb_stream_t stream,
                   void* const* events, int32_t n_events);

/* Forward statistics the backward consumes: lse [B, Hq, Tq] fp32 (written), the row
 * log-sum-exp of the scaled scores over visible keys ("Attention (full single-head)",
 * attentionForward's softmax normaliser). Uses desc's q/k strides, dtypes and mask. */
int attn_fwd_lse(const attn_bwd_desc* desc, const void* q, const void* k, float* lse,
                 vtb_stream_t stream);

/* Attention forward by online softmax: the FlashAttention.lean entry of the Hesper pull
 * request's commit log (flashAttentionSpec: K and V consumed one position at a time with a
 * running maximum and sum of exponentials, equal to scores -> softmax -> apply), over the
 * softmax and apply of "Attention (full single-head)" (attentionForward), batched with
 * the same heads, grouping and causal mask as attn_bwd:
 *     O_i = sum_j P_ij v_j,  P_ij = exp(scale q_i . k_j - lse_i) over visible j,
 *     lse_i = ln sum_{visible j} exp(scale q_i . k_j).
 * q: [B, Tq, Hq, D], k, v: [B, Tk, Hkv, D] in desc->in_dtype with strides s_q, s_k, s_v.
 * o (written): [B, Tq, Hq, D] in desc->out_dtype with strides s_dq (o has dq's shape).
 * lse (written, may be NULL): [B, Hq, Tq] fp32, the input attn_bwd takes.
 * All pointers device memory owned by the caller, 16-byte aligned; o and lse must not
 * overlap the inputs or each other (VTB_ERR_ALIAS). One kernel on `stream`; nothing is
 * written on an error. bf16 inputs use bf16 P in the P V product, fp32 accumulation. */
int attn_fwd(const attn_bwd_desc* desc, const void* q, const void* k, const void* v, void* o,
             float* lse, vtb_stream_t stream);

/* Workspace bytes attn_fwd_ws needs for desc (>= 256); 0 when desc is invalid
 * (vtb_last_error says why). */
size_t attn_fwd_workspace_size(const attn_bwd_desc* desc);

/* attn_fwd with a workspace, which lets decode-shaped problems ((Hq/Hkv) * Tq <= 16 rows
 * per kv head) run split-KV: the tiled flash attention entry of the Hesper pull request's
 * commit log computes, per KV tile in parallel, a partial output together with the
 * tile's running maximum and sum of exponentials (Phase 1), then merges the tiles
 * (Phase 2). Here one workgroup per (64-key chunk, kv head, batch) reads that chunk's K
 * and V once for all rows of the group and writes (m_c, l_c, sum_j exp(s_j - m_c) v_j);
 * a second kernel merges the chunks in order into O and lse. Results are those of
 * attn_fwd (same definitions, same arguments) up to rounding order; other shapes take
 * attn_fwd's own kernels and leave the workspace unused.
 * workspace: device memory, 16-byte aligned, at least attn_fwd_workspace_size(desc)
 * bytes (else VTB_ERR_WORKSPACE), owned by the caller, overwritten, not overlapping any
 * tensor (VTB_ERR_ALIAS); NULL is VTB_ERR_WORKSPACE. Two kernels on `stream`. */
int attn_fwd_ws(const attn_bwd_desc* desc, const void* q, const void* k, const void* v, void* o,
                float* lse, void* workspace, size_t workspace_bytes, vtb_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * RoPE backward: "Hesper.Training.VerifiedBackward", section "RoPE (Rotary Position
 * Embedding)", ropeBackward = rotation by -theta:
 *     (dx0, dx1) = (dy0 cos t + dy1 sin t, -dy0 sin t + dy1 cos t)
 * with theta(pos, i) = pos * base^(-2i / head_dim), i = 0 .. head_dim/2 - 1.
 * dy, dx: [n_tok, n_heads, head_dim] fp32, token stride tok_stride (elements), heads
 * packed (head stride = head_dim). pos: device int32 [n_tok] or NULL for pos0 + t.
 * layout 0 pairs (2i, 2i+1); layout 1 pairs (i, i + head_dim/2). head_dim must be even.
 * dx == dy (exactly in place) is allowed; any other overlap is VTB_ERR_ALIAS.
 * -------------------------------------------------------------------------------------*/
int rope_bwd(const float* dy, float* dx, int32_t n_tok, int32_t n_heads, int32_t head_dim,
             int64_t tok_stride, const int32_t* pos, int32_t pos0, double base, int32_t layout,
             vtb_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * RMSNorm backward: "Hesper.Training.VerifiedBackward", section "RMSNorm",
 * rmsNormBackward, per row of n values:
 *     rms = sqrt(mean(x^2) + eps);  c = sum_j dy_j gamma_j x_j
 *     dx_i = (dy_i gamma_i - x_i c / (n rms^2)) / rms
 * x, dy, dx: [rows, n] fp32 contiguous; gamma: [n] fp32. dx must not overlap inputs.
 * -------------------------------------------------------------------------------------*/
int rmsnorm_bwd(const float* x, const float* gamma, const float* dy, float* dx, int32_t rows,
                int32_t n, float eps, vtb_stream_t stream);

/* The same two operations with the storage type as an argument: dtype VTB_F32 or VTB_BF16
 * for dy, dx (RoPE) and x, dy, dx (RMSNorm), fp32 arithmetic, outputs rounded once (RNE
 * for bf16); gamma stays fp32. Layouts, aliasing rules and errors as above. */
int rope_bwd_ex(int32_t dtype, const void* dy, void* dx, int32_t n_tok, int32_t n_heads, int32_t head_dim,
                int64_t tok_stride, const int32_t* pos, int32_t pos0, double base, int32_t layout,
                vtb_stream_t stream);
int rmsnorm_bwd_ex(int32_t dtype, const void* x, const float* gamma, const void* dy, void* dx, int32_t rows,
                   int32_t n, float eps, vtb_stream_t stream);

/* Fused tail of one layer's backward (RoPE backward, RMSNorm backward, residual):
 *     dh_in = dh_out + rmsNormBackward(x, gamma, ropeBackward(dq))
 * per token row of C = n_heads * head_dim values, positions pos0 + t. dq: [T, C] fp32
 * scaled by dq_scale on read; x, dh_out, dh_in: [T, C]; gamma: [C]. dh_in == dh_out is
 * allowed (in place); other overlaps are VTB_ERR_ALIAS. */
int rope_rmsnorm_res_bwd(const float* dq, float dq_scale, const float* x, const float* gamma,
                         const float* dh_out, float* dh_in, int32_t T, int32_t n_heads,
                         int32_t head_dim, int32_t pos0, double base, int32_t layout, float eps,
                         vtb_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * LayerNorm (no affine) backward: DaisyChain-Train transformer.js page, functions lnFwd /
 * lnBwd ("layernorm (no affine)"). The forward keeps, per row of n values,
 *     sigma = sqrt(mean((x - mean x)^2) + 1e-5),   y = (x - mean x) / sigma,
 * and the backward is, from dy, y and sigma alone,
 *     dx = (dy - mean(dy) - y * mean(dy * y)) / sigma.
 * dtype VTB_F32 or VTB_BF16 is the storage type of dy, y and dx ([rows, n] contiguous);
 * sig is fp32 [rows]. Arithmetic is fp32. dx must not overlap any input.
 * -------------------------------------------------------------------------------------*/
int layernorm_bwd(int32_t dtype, const void* dy, const void* y, const float* sig, void* dx, int32_t rows,
                  int32_t n, vtb_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * ReLU^2 x Mul backward (the FFN gate): Hesper pull-request commit log, "FFN backward"
 * (FFNBackward.lean). For h = ReLU(gate)^2 * up elementwise,
 *     dgate = dh * up * 2 * ReLU(gate),   dup = dh * ReLU(gate)^2.
 * gate, up, dh, dgate, dup: n contiguous elements of dtype (VTB_F32 or VTB_BF16);
 * arithmetic is fp32. Outputs must not overlap inputs or each other.
 * -------------------------------------------------------------------------------------*/
int relu2_mul_bwd(int32_t dtype, const void* gate, const void* up, const void* dh, void* dgate, void* dup,
                  int64_t n, vtb_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Linear backward of Y = X W (Hesper commit log: outer-product dW and transposed dX;
 * transformer.js `backward`, Wo: gWo = ctxOut^T dx2, dctx = dx2 Wo^T):
 *     dX = dY W^T   [T, K]        dW = X^T dY = sum_t x_t (outer) dy_t   [K, N]
 * x: [T, K], w: [K, N], dy: [T, N], all fp32 row-major contiguous. dx or dw may be NULL
 * (that product is skipped), not both. Outputs must not overlap inputs or each other.
 * -------------------------------------------------------------------------------------*/
int linear_bwd(const float* x, const float* w, const float* dy, float* dx, float* dw, int32_t T,
               int32_t K, int32_t N, vtb_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * One layer's backward, the Hesper commit log's reverse chain over saved activations
 * (linear backward, attention backward with the saved softmax, RoPE backward, RMSNorm
 * backward, residual passing the hidden gradient through unchanged):
 *     dO, dW   = dh_out W^T,  o^T dh_out
 *     dq, dK, dV = attention backward (saved P, causal per cfg)
 *     dh_in    = dh_out + rmsNormBackward(x, gamma, ropeBackward(dq))    (positions 0..T-1)
 * Saved tensors (fp32): x [T, C] RMSNorm input, gamma [C], w [C, C], o [T, C] attention
 * output, q [T, H, D] rotated queries, k, v [T, H, D] caches, P [H, T, T] softmax.
 * Outputs: dh_in [T, C], dw [C, C], dk, dv [T, H, D]. C = H * D; D must be 64 or 128.
 * dh_in == dh_out is allowed. A 30-layer stack calls this from the last layer down.
 * -------------------------------------------------------------------------------------*/
typedef struct {
  int32_t T, H, D;
  float scale, eps;
  double rope_base;
  int32_t rope_layout, causal;
} layer_bwd_cfg;

typedef struct {
  const float *x, *gamma, *w, *o, *q, *k, *v, *P;
} layer_saved;

size_t layer_bwd_workspace_size(const layer_bwd_cfg* cfg);

int layer_bwd(const layer_bwd_cfg* cfg, const layer_saved* saved, const float* dh_out,
              float* dh_in, float* dw, float* dk, float* dv, void* workspace,
              size_t workspace_bytes, vtb_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * One FFN block's backward: the Hesper pull-request commit log, "FFN backward"
 * (FFNBackward.lean), ops in its order: ffnDown transpose, ffnSubNorm (RMSNorm) backward,
 * ReLU^2 x Mul backward, ffnGate/Up transposes, ffnNorm (RMSNorm) backward; the residual
 * passes dout through. The block's forward is read as
 *     xn = RMSNorm(x; gamma1),  gu = xn Wgu  (Wgu = [Wgate | Wup], [C, 2F]),
 *     h = ReLU(gu[:, :F])^2 * gu[:, F:],  hn = RMSNorm(h; gamma2),  out = x + hn Wdown,
 * and the backward computes
 *     dhn, dWdown = dout Wdown^T, hn^T dout
 *     dgate, dup  = ReLU^2 x Mul backward(gate, up, RMSNormBackward(h, gamma2, dhn))
 *     dxn, dWgu   = [dgate | dup] Wgu^T, xn^T [dgate | dup]
 *     dx          = dout + RMSNormBackward(x, gamma1, dxn)
 * with h formed again from the saved gate and up. Saved tensors (fp32, row-major,
 * 16-byte aligned): x, xn [T, C]; gamma1 [C]; w_gu [C, 2F]; gu [T, 2F]; gamma2 [F];
 * hn [T, F]; w_down [F, C]. Outputs: dx [T, C], dw_gu [C, 2F], dw_down [F, C]. dx == dout
 * is allowed; no other overlap. Workspace from ffn_bwd_workspace_size().
 * -------------------------------------------------------------------------------------*/
typedef struct {
  int32_t T, C, F;
  float eps;
} ffn_bwd_cfg;

typedef struct {
  const float *x, *gamma1, *xn, *w_gu, *gu, *gamma2, *hn, *w_down;
} ffn_saved;

size_t ffn_bwd_workspace_size(const ffn_bwd_cfg* cfg);

int ffn_bwd(const ffn_bwd_cfg* cfg, const ffn_saved* saved, const float* dout, float* dx, float* dw_gu,
            float* dw_down, void* workspace, size_t workspace_bytes, vtb_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * One transformer attention block's backward, as the DaisyChain-Train transformer.js page
 * builds the block (forward layer loop and `backward`): over B sequences of T tokens,
 * hidden C = H * D,
 *     ln = LayerNorm(xin) (no affine; y, sigma kept),  [q | k | v] = ln.y Wqkv  (Wqkv =
 *     [Wq | Wk | Wv], [C, 3C]),  P = causal softmax(scale q_h k_h^T) per sequence and head,
 *     ctx = P v_h,  x2 = xin + ctx Wo,
 * and the backward from dx2:
 *     gWo, dctx  = ctx^T dx2, dx2 Wo^T
 *     dq, dk, dv = attention backward with the saved P (dS = P o (dP - rowsum(P o dP)))
 *     gWqkv, dln = ln.y^T [dq | dk | dv], [dq | dk | dv] Wqkv^T
 *     dx         = dx2 + lnBwd(dln, ln.y, sigma)
 * Saved tensors (fp32, row-major, 16-byte aligned): ln_y [B T, C], ln_sig [B T],
 * w_qkv [C, 3C], qkv [B T, 3C] (q, k, v side by side, head h at columns h D of each
 * third), P [B H, T, T], ctx [B T, C], w_o [C, C]. Outputs: dx [B T, C], dw_qkv [C, 3C],
 * dw_o [C, C]. dx == dx2 is allowed; no other overlap. Workspace from
 * attn_block_bwd_workspace_size().
 * -------------------------------------------------------------------------------------*/
typedef struct {
  int32_t B, T, H, D;
  float scale;
  int32_t causal;
} attn_block_cfg;

typedef struct {
  const float *ln_y, *ln_sig, *w_qkv, *qkv, *P, *ctx, *w_o;
} attn_block_saved;

size_t attn_block_bwd_workspace_size(const attn_block_cfg* cfg);

int attn_block_bwd(const attn_block_cfg* cfg, const attn_block_saved* saved, const float* dx2, float* dx,
                   float* dw_qkv, float* dw_o, void* workspace, size_t workspace_bytes, vtb_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * One attention layer of the Hesper form, backward: RMSNorm with a learned gain, Q/K/V
 * projections, RoPE on the projected queries and keys, causal attention, output projection
 * and residual. The pieces are "Hesper.Training.VerifiedBackward"'s rmsNormForward /
 * rmsNormBackward (section "RMSNorm"), ropeForward / ropeBackward (section "RoPE (Rotary
 * Position Embedding)") and its attention chain (section "Attention (full single-head)"),
 * with the causal mask and the fused Q/K/V weight gradient of the DaisyChain-Train
 * transformer.js `backward`. Over B sequences of T tokens, hidden C = H * D, positions
 * t = 0 .. T-1 within each sequence, the forward
 *     n = gamma o x / r_t (r_t = sqrt(mean(x_t^2) + eps)),  [a | b | v] = n Wqkv,
 *     q = RoPE(a), k = RoPE(b) per head,  P = causal softmax(scale q_h k_h^T),
 *     ctx = P v_h,  x2 = x + ctx Wo
 * has the backward from dx2
 *     gWo, dctx  = ctx^T dx2, dx2 Wo^T
 *     dq, dk, dv = attention backward with the saved P
 *     da, db     = RoPEBackward(dq), RoPEBackward(dk)          (rotation by -theta)
 *     gWqkv, dn  = n^T [da | db | dv], [da | db | dv] Wqkv^T
 *     dx         = dx2 + RMSNormBackward(x, gamma, dn),  dgamma = sum_t dn_t o x_t / r_t
 * (dgamma: the derivative of the same RMSNorm map in gamma). RoPE angles are
 * t * rope_base^(-2i / D); rope_layout 0 pairs (2i, 2i+1), 1 pairs (i, i + D/2).
 * Saved tensors (fp32, row-major, 16-byte aligned): x [B T, C], gamma [C], n [B T, C] (the
 * RMSNorm output), w_qkv [C, 3C], qkv [B T, 3C] (the rotated q and k, then v; head h at
 * columns h D of each third), P [B H, T, T], ctx [B T, C], w_o [C, C]. Outputs: dx [B T, C],
 * dgamma [C], dw_qkv [C, 3C], dw_o [C, C]. dx == dx2 is allowed; no other overlap. Every
 * reduction runs in a fixed order: results are bitwise reproducible. Workspace from
 * rms_attn_block_bwd_workspace_size().
 * -------------------------------------------------------------------------------------*/
typedef struct {
  int32_t B, T, H, D;
  float scale;
  int32_t causal;
  float eps;
  double rope_base;
  int32_t rope_layout;
} rms_attn_block_cfg;

typedef struct {
  const float *x, *gamma, *n, *w_qkv, *qkv, *P, *ctx, *w_o;
} rms_attn_block_saved;

size_t rms_attn_block_bwd_workspace_size(const rms_attn_block_cfg* cfg);

int rms_attn_block_bwd(const rms_attn_block_cfg* cfg, const rms_attn_block_saved* saved, const float* dx2,
                       float* dx, float* dgamma, float* dw_qkv, float* dw_o, void* workspace,
                       size_t workspace_bytes, vtb_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VTB_H */
