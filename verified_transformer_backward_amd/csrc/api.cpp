// C ABI of libvtb: argument validation, alias and workspace checks, path selection and
// launches on the caller's stream. Nothing here allocates device memory or synchronises.
#include "vtb.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return VTB_OK;
  return fail(VTB_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi) in bytes; empty when lo == hi
};

Span span_of(const void* p, size_t bytes) {
  Span s;
  s.lo = reinterpret_cast<uintptr_t>(p);
  s.hi = s.lo + bytes;
  return s;
}

bool overlap(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

// Bytes spanned by a [B, T, H, D] tensor with (b, t, h) strides and D contiguous.
size_t bthd_bytes(int B, int T, int H, int D, const int64_t st[3], size_t esize) {
  if (B <= 0 || T <= 0 || H <= 0 || D <= 0) return 0;
  const int64_t last = (int64_t)(B - 1) * st[0] + (int64_t)(T - 1) * st[1] + (int64_t)(H - 1) * st[2] + D;
  return (size_t)last * esize;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

bool valid_dtype(int32_t d) { return d == VTB_F32 || d == VTB_BF16; }
size_t esize(int32_t d) { return d == VTB_BF16 ? 2 : 4; }

// Workspace carve-up of the flash path: row term D, computed lse (or, on the MFMA path
// where lse is given, lse in base-2 units for the dk/dv pass).
struct FlashWs {
  size_t dlt, lse, total;
};

FlashWs flash_ws(const attn_bwd_desc* d) {
  FlashWs w;
  const size_t rows = (size_t)d->B * d->Hq * d->Tq;
  w.dlt = 0;
  w.lse = align256(rows * sizeof(float));
  w.total = w.lse + align256(rows * sizeof(float));
  return w;
}

vtb::AttnParams make_params(const attn_bwd_desc* d) {
  vtb::AttnParams p{};
  p.B = d->B;
  p.Hq = d->Hq;
  p.Hkv = d->Hkv;
  p.Tq = d->Tq;
  p.Tk = d->Tk;
  p.D = d->D;
  p.scale = d->scale;
  p.causal = d->causal;
  p.in_bf16 = d->in_dtype == VTB_BF16;
  p.out_bf16 = d->out_dtype == VTB_BF16;
  for (int i = 0; i < 3; ++i) {
    p.sq[i] = d->s_q[i];
    p.sk[i] = d->s_k[i];
    p.sv[i] = d->s_v[i];
    p.sdo[i] = d->s_do[i];
    p.sdq[i] = d->s_dq[i];
    p.sdk[i] = d->s_dk[i];
    p.sdv[i] = d->s_dv[i];
  }
  return p;
}

// Shape, dtype and stride checks shared by attn_bwd, its workspace query and attn_fwd_lse.
int check_desc(const attn_bwd_desc* d, bool need_grads) {
  if (!d) return fail(VTB_ERR_ARG, "desc is NULL");
  if (d->B < 0 || d->Tq < 0 || d->Tk < 0) return fail(VTB_ERR_ARG, "negative size (B=%d Tq=%d Tk=%d)", d->B, d->Tq, d->Tk);
  if (d->Hq < 1 || d->Hkv < 1) return fail(VTB_ERR_ARG, "Hq=%d and Hkv=%d must be >= 1", d->Hq, d->Hkv);
  if (d->Hq % d->Hkv) return fail(VTB_ERR_ARG, "Hq=%d is not a multiple of Hkv=%d", d->Hq, d->Hkv);
  if (d->D != 64 && d->D != 128) return fail(VTB_ERR_UNSUPPORTED, "head dim D=%d (supported: 64, 128)", d->D);
  if (!valid_dtype(d->in_dtype)) return fail(VTB_ERR_ARG, "in_dtype=%d", d->in_dtype);
  if (need_grads && !valid_dtype(d->out_dtype)) return fail(VTB_ERR_ARG, "out_dtype=%d", d->out_dtype);
  if (!std::isfinite(d->scale)) return fail(VTB_ERR_ARG, "scale is not finite");
  if (d->causal != 0 && d->causal != 1) return fail(VTB_ERR_ARG, "causal=%d must be 0 or 1", d->causal);
  if (d->causal && d->Tk < d->Tq) return fail(VTB_ERR_ARG, "causal needs Tk >= Tq (Tq=%d Tk=%d)", d->Tq, d->Tk);
  if (d->Tk == 0 && d->Tq > 0 && d->B > 0) return fail(VTB_ERR_ARG, "Tk == 0: softmax over no keys is undefined");
  const int64_t* all[7] = {d->s_q, d->s_k, d->s_v, d->s_do, d->s_dq, d->s_dk, d->s_dv};
  const char* names[7] = {"q", "k", "v", "dout", "dq", "dk", "dv"};
  for (int t = 0; t < (need_grads ? 7 : 2); ++t)
    for (int i = 0; i < 3; ++i) {
      if (all[t][i] < 0) return fail(VTB_ERR_ARG, "%s stride %d is negative", names[t], i);
      if (all[t][i] % 8) return fail(VTB_ERR_UNSUPPORTED, "%s stride %d = %lld is not a multiple of 8 elements", names[t], i, (long long)all[t][i]);
    }
  return VTB_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" {

const char* vtb_status_string(int status) {
  switch (status) {
    case VTB_OK: return "VTB_OK";
    case VTB_ERR_ARG: return "VTB_ERR_ARG";
    case VTB_ERR_UNSUPPORTED: return "VTB_ERR_UNSUPPORTED";
    case VTB_ERR_ALIAS: return "VTB_ERR_ALIAS";
    case VTB_ERR_WORKSPACE: return "VTB_ERR_WORKSPACE";
    case VTB_ERR_HIP: return "VTB_ERR_HIP";
    default: return "VTB_UNKNOWN_STATUS";
  }
}

const char* vtb_last_error(void) { return g_last_error.c_str(); }

int vtb_abi_version(void) { return 1; }

size_t attn_bwd_workspace_size(const attn_bwd_desc* d) {
  if (check_desc(d, true) != VTB_OK) return 0;
  const vtb::AttnParams p = make_params(d);
  size_t bytes = flash_ws(d).total;
  if (vtb::decode_applicable(p)) bytes = std::max(bytes, vtb::decode_workspace_bytes(p));
  return std::max<size_t>(bytes, 256);
}

}  // extern "C"

namespace {

// Caller events of attn_bwd_timed: launch i (0 or 1) of a call is timed by events[2i]
// (its start) and events[2i + 1] (its end).
struct PhaseEvents {
  void* const* ev;
  int n;
  vtb::KernelEvents pass(int i) const {
    vtb::KernelEvents k;
    if (ev && n >= 2 * i + 2) {
      k.start = reinterpret_cast<hipEvent_t>(ev[2 * i]);
      k.stop = reinterpret_cast<hipEvent_t>(ev[2 * i + 1]);
    }
    return k;
  }
};

// o (with strides so): the forward's saved output, or NULL. When given, lse is required,
// P must be NULL, and the row term D comes from dO . O.
int attn_bwd_impl(const attn_bwd_desc* d, const void* q, const void* k, const void* v, const void* dout, const float* lse,
                  const float* P, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, hipStream_t s,
                  PhaseEvents ev, const void* o = nullptr, const int64_t* so = nullptr) {
  g_last_error.clear();
  int rc = check_desc(d, true);
  if (rc) return rc;
  if (o) {
    if (!so) return fail(VTB_ERR_ARG, "s_o is NULL");
    if (P) return fail(VTB_ERR_ARG, "a saved O is used with lse, not with a saved P");
    if (!lse && d->B > 0 && d->Tq > 0) return fail(VTB_ERR_ARG, "a saved O needs the saved lse");
    for (int i = 0; i < 3; ++i) {
      if (so[i] < 0) return fail(VTB_ERR_ARG, "o stride %d is negative", i);
      if (so[i] % 8) return fail(VTB_ERR_UNSUPPORTED, "o stride %d = %lld is not a multiple of 8 elements", i, (long long)so[i]);
    }
  }
  const size_t ein = esize(d->in_dtype), eout = esize(d->out_dtype);
  const Span sq = span_of(q, bthd_bytes(d->B, d->Tq, d->Hq, d->D, d->s_q, ein));
  const Span sk = span_of(k, bthd_bytes(d->B, d->Tk, d->Hkv, d->D, d->s_k, ein));
  const Span sv = span_of(v, bthd_bytes(d->B, d->Tk, d->Hkv, d->D, d->s_v, ein));
  const Span sdo = span_of(dout, bthd_bytes(d->B, d->Tq, d->Hq, d->D, d->s_do, ein));
  const Span sdq = span_of(dq, bthd_bytes(d->B, d->Tq, d->Hq, d->D, d->s_dq, eout));
  const Span sdk = span_of(dk, dk ? bthd_bytes(d->B, d->Tk, d->Hkv, d->D, d->s_dk, eout) : 0);
  const Span sdv = span_of(dv, dv ? bthd_bytes(d->B, d->Tk, d->Hkv, d->D, d->s_dv, eout) : 0);
  const size_t rows = (size_t)d->B * d->Hq * d->Tq;
  const Span slse = span_of(lse, P ? 0 : (lse ? rows * 4 : 0));
  const Span sP = span_of(P, P ? rows * (size_t)d->Tk * 4 : 0);
  const Span sws = span_of(workspace, workspace_bytes);
  const Span so_ = span_of(o, o ? bthd_bytes(d->B, d->Tq, d->Hq, d->D, so, ein) : 0);
  const bool has_q = d->B > 0 && d->Tq > 0, has_k = d->B > 0 && d->Tk > 0;
  if (has_q && (!q || !dout || !dq)) return fail(VTB_ERR_ARG, "q, dout and dq must be non-NULL");
  if (o && !aligned16(o)) return fail(VTB_ERR_UNSUPPORTED, "tensor pointers must be 16-byte aligned");
  if (has_k && (!k || !v)) return fail(VTB_ERR_ARG, "k and v must be non-NULL");   // dk, dv: NULL = not wanted
  const void* ptrs[8] = {q, k, v, dout, dq, dk, dv, workspace};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(VTB_ERR_UNSUPPORTED, "tensor pointers must be 16-byte aligned");
  const Span outs[3] = {sdq, sdk, sdv};
  const Span ins[8] = {sq, sk, sv, sdo, slse, sP, so_, sws};
  for (int t = 0; t < 3; ++t) {
    for (int i = 0; i < 8; ++i)
      if (overlap(outs[t], ins[i])) return fail(VTB_ERR_ALIAS, "output %d overlaps an input or the workspace", t);
    for (int t2 = t + 1; t2 < 3; ++t2)
      if (overlap(outs[t], outs[t2])) return fail(VTB_ERR_ALIAS, "outputs %d and %d overlap", t, t2);
  }
  for (int i = 0; i < 7; ++i)
    if (overlap(sws, ins[i])) return fail(VTB_ERR_ALIAS, "workspace overlaps an input");

  vtb::AttnParams p = make_params(d);
  p.q = q;
  p.k = k;
  p.v = v;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.P = P;

  if (!has_q) {  // no queries: dK = dV = 0
    if (!has_k) return VTB_OK;
    if (dk) {
      rc = hip_status(vtb::launch_zero_bthd(dk, p.out_bf16, d->B, d->Tk, d->Hkv, d->D, d->s_dk, s, ev.pass(0)), "zero dk");
      if (rc) return rc;
    }
    if (dv) return hip_status(vtb::launch_zero_bthd(dv, p.out_bf16, d->B, d->Tk, d->Hkv, d->D, d->s_dv, s, ev.pass(1)), "zero dv");
    return VTB_OK;
  }

  const size_t need = attn_bwd_workspace_size(d);
  if (!workspace || workspace_bytes < need)
    return fail(VTB_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0, need);

  if (!P && vtb::decode_applicable(p)) {   // a saved O is not read: D comes from the chunk statistics
    p.lse = lse;
    return hip_status(vtb::launch_decode(p, workspace, s, ev.pass(0), ev.pass(1)), "decode path");
  }
  const FlashWs w = flash_ws(d);
  char* base = reinterpret_cast<char*>(workspace);
  p.dlt = reinterpret_cast<float*>(base + w.dlt);
  int mode;
  if (P) {
    mode = vtb::ROW_P_GIVEN;
  } else if (o) {
    p.lse = lse;
    p.o = o;
    for (int i = 0; i < 3; ++i) p.so[i] = so[i];
    mode = vtb::ROW_D_GIVEN;
  } else if (lse) {
    p.lse = lse;
    mode = vtb::ROW_LSE_GIVEN;
  } else {
    p.lse_out = reinterpret_cast<float*>(base + w.lse);
    p.lse = p.lse_out;
    mode = vtb::ROW_LSE_COMPUTE;
  }
  const bool mfma = vtb::mfma_path_applicable(p);
  if (mfma && (mode == vtb::ROW_LSE_GIVEN || mode == vtb::ROW_D_GIVEN)) {
    p.lse2 = reinterpret_cast<float*>(base + w.lse);   // free when lse is given
    rc = hip_status(vtb::launch_mfma_dq(p, s, ev.pass(0), mode == vtb::ROW_D_GIVEN), "dq pass");
  } else {
    rc = hip_status(vtb::launch_flash_dq(p, mode, s, ev.pass(0)), "flash dq pass");
  }
  if (rc) return rc;
  if (!dk && !dv) return VTB_OK;   // only dQ wanted: the key-parallel pass is skipped
  if (mfma && !P) return hip_status(vtb::launch_mfma_dkdv(p, s, ev.pass(1)), "dk/dv pass");
  return hip_status(vtb::launch_flash_dkdv(p, s, ev.pass(1)), "flash dk/dv pass");
}

}  // namespace

extern "C" {

int attn_bwd(const attn_bwd_desc* d, const void* q, const void* k, const void* v, const void* dout, const float* lse,
             const float* P, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, vtb_stream_t stream) {
  return attn_bwd_impl(d, q, k, v, dout, lse, P, dq, dk, dv, workspace, workspace_bytes,
                       reinterpret_cast<hipStream_t>(stream), PhaseEvents{nullptr, 0});
}

int attn_bwd_o(const attn_bwd_desc* d, const void* q, const void* k, const void* v, const void* dout, const void* o,
               const int64_t* s_o, const float* lse, void* dq, void* dk, void* dv, void* workspace,
               size_t workspace_bytes, vtb_stream_t stream) {
  if (!o) return fail(VTB_ERR_ARG, "o is NULL (use attn_bwd without a saved O)");
  return attn_bwd_impl(d, q, k, v, dout, lse, nullptr, dq, dk, dv, workspace, workspace_bytes,
                       reinterpret_cast<hipStream_t>(stream), PhaseEvents{nullptr, 0}, o, s_o);
}

}  // extern "C"

namespace {

// ---------------------------------------------------------------------------- no-allocation variant
// attn_bwd_noalloc's workspace: a file-scope device array, one copy per GPU, held until the
// process ends. In host code `scratch` only names the symbol; its device address on the
// current GPU comes from hipGetSymbolAddress, taken once per device and kept in scratch_ptr.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`, resolved on the first call on that device.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(VTB_ERR_UNSUPPORTED, "device %d is beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(VTB_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return VTB_OK;
}

}  // namespace

extern "C" {

size_t attn_bwd_noalloc_max_workspace(void) { return kScratchBytes; }

int attn_bwd_noalloc(const attn_bwd_desc* d, const void* q, const void* k, const void* v, const void* dout,
                     const float* lse, const float* P, void* dq, void* dk, void* dv, vtb_stream_t stream) {
  g_last_error.clear();
  int rc = check_desc(d, true);
  if (rc) return rc;
  const size_t need = attn_bwd_workspace_size(d);
  if (need > kScratchBytes)
    return fail(VTB_ERR_WORKSPACE, "this problem needs %zu bytes of workspace; attn_bwd_noalloc holds at most %zu "
                "(use attn_bwd with a caller workspace)", need, kScratchBytes);
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  return attn_bwd_impl(d, q, k, v, dout, lse, P, dq, dk, dv, ws, kScratchBytes, reinterpret_cast<hipStream_t>(stream),
                       PhaseEvents{nullptr, 0});
}

int attn_bwd_timed(const attn_bwd_desc* d, const void* q, const void* k, const void* v, const void* dout,
                   const float* lse, const float* P, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, vtb_stream_t stream, void* const* events, int32_t n_events) {
  if (!events || n_events < 4) return fail(VTB_ERR_ARG, "attn_bwd_timed needs 4 events");
  for (int i = 0; i < 4; ++i)
    if (!events[i]) return fail(VTB_ERR_ARG, "event %d is NULL", i);
  return attn_bwd_impl(d, q, k, v, dout, lse, P, dq, dk, dv, workspace, workspace_bytes,
                       reinterpret_cast<hipStream_t>(stream), PhaseEvents{events, 4});
}

int attn_fwd_lse(const attn_bwd_desc* d, const void* q, const void* k, float* lse, vtb_stream_t stream) {
  g_last_error.clear();
  int rc = check_desc(d, false);
  if (rc) return rc;
  const size_t ein = esize(d->in_dtype);
  const size_t rows = (size_t)d->B * d->Hq * d->Tq;
  if (rows == 0) return VTB_OK;
  if (!q || !k || !lse) return fail(VTB_ERR_ARG, "q, k and lse must be non-NULL");
  if (!aligned16(q) || !aligned16(k)) return fail(VTB_ERR_UNSUPPORTED, "q and k must be 16-byte aligned");
  const Span sl = span_of(lse, rows * 4);
  if (overlap(sl, span_of(q, bthd_bytes(d->B, d->Tq, d->Hq, d->D, d->s_q, ein))) ||
      overlap(sl, span_of(k, bthd_bytes(d->B, d->Tk, d->Hkv, d->D, d->s_k, ein))))
    return fail(VTB_ERR_ALIAS, "lse overlaps q or k");
  vtb::AttnParams p = make_params(d);
  p.q = q;
  p.k = k;
  p.lse_out = lse;
  return hip_status(vtb::launch_flash_dq(p, vtb::ROW_LSE_ONLY, reinterpret_cast<hipStream_t>(stream)), "lse pass");
}

}  // extern "C"

namespace {

int attn_fwd_impl(const attn_bwd_desc* d, const void* q, const void* k, const void* v, void* o, float* lse,
                  void* workspace, size_t workspace_bytes, hipStream_t s) {
  g_last_error.clear();
  int rc = check_desc(d, false);
  if (rc) return rc;
  if (!valid_dtype(d->out_dtype)) return fail(VTB_ERR_ARG, "out_dtype=%d", d->out_dtype);
  const int64_t* st[2] = {d->s_v, d->s_dq};
  const char* names[2] = {"v", "o (s_dq)"};
  for (int t = 0; t < 2; ++t)
    for (int i = 0; i < 3; ++i) {
      if (st[t][i] < 0) return fail(VTB_ERR_ARG, "%s stride %d is negative", names[t], i);
      if (st[t][i] % 8) return fail(VTB_ERR_UNSUPPORTED, "%s stride %d = %lld is not a multiple of 8 elements", names[t], i, (long long)st[t][i]);
    }
  const size_t ein = esize(d->in_dtype), eout = esize(d->out_dtype);
  const size_t rows = (size_t)d->B * d->Hq * d->Tq;
  if (rows == 0) return VTB_OK;
  if (!q || !k || !v || !o) return fail(VTB_ERR_ARG, "q, k, v and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (workspace && !aligned16(workspace)))
    return fail(VTB_ERR_UNSUPPORTED, "q, k, v, o and the workspace must be 16-byte aligned");
  const Span so = span_of(o, bthd_bytes(d->B, d->Tq, d->Hq, d->D, d->s_dq, eout));
  const Span sq = span_of(q, bthd_bytes(d->B, d->Tq, d->Hq, d->D, d->s_q, ein));
  const Span sk = span_of(k, bthd_bytes(d->B, d->Tk, d->Hkv, d->D, d->s_k, ein));
  const Span sv = span_of(v, bthd_bytes(d->B, d->Tk, d->Hkv, d->D, d->s_v, ein));
  const Span sws = span_of(workspace, workspace_bytes);
  if (overlap(so, sq) || overlap(so, sk) || overlap(so, sv) || overlap(so, sws))
    return fail(VTB_ERR_ALIAS, "o overlaps q, k, v or the workspace");
  if (lse) {
    const Span sl = span_of(lse, rows * 4);
    if (overlap(sl, sq) || overlap(sl, sk) || overlap(sl, sv) || overlap(sl, so) || overlap(sl, sws))
      return fail(VTB_ERR_ALIAS, "lse overlaps q, k, v, o or the workspace");
  }
  vtb::AttnParams p = make_params(d);
  p.q = q;
  p.k = k;
  p.v = v;
  p.dq = o;
  p.lse_out = lse;
  if (workspace && vtb::decode_fwd_applicable(p)) {
    const size_t need = vtb::decode_fwd_workspace_bytes(p);
    if (workspace_bytes < need)
      return fail(VTB_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
    if (overlap(sws, sq) || overlap(sws, sk) || overlap(sws, sv))
      return fail(VTB_ERR_ALIAS, "the workspace overlaps q, k or v");
    return hip_status(vtb::launch_decode_fwd(p, workspace, s), "split-KV decode forward");
  }
  if (vtb::mfma_fwd_applicable(p)) return hip_status(vtb::launch_mfma_fwd(p, s), "forward pass (MFMA)");
  return hip_status(vtb::launch_flash_dq(p, vtb::ROW_FWD, s), "forward pass");
}

}  // namespace

extern "C" {

int attn_fwd(const attn_bwd_desc* d, const void* q, const void* k, const void* v, void* o, float* lse,
             vtb_stream_t stream) {
  return attn_fwd_impl(d, q, k, v, o, lse, nullptr, 0, reinterpret_cast<hipStream_t>(stream));
}

size_t attn_fwd_workspace_size(const attn_bwd_desc* d) {
  if (check_desc(d, false) != VTB_OK) return 0;
  const vtb::AttnParams p = make_params(d);
  size_t bytes = vtb::decode_fwd_applicable(p) ? vtb::decode_fwd_workspace_bytes(p) : 0;
  return std::max<size_t>(bytes, 256);
}

int attn_fwd_ws(const attn_bwd_desc* d, const void* q, const void* k, const void* v, void* o, float* lse,
                void* workspace, size_t workspace_bytes, vtb_stream_t stream) {
  if (!workspace) return fail(VTB_ERR_WORKSPACE, "attn_fwd_ws needs a workspace (attn_fwd_workspace_size)");
  return attn_fwd_impl(d, q, k, v, o, lse, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream));
}

int rope_bwd_ex(int32_t dtype, const void* dy, void* dx, int32_t n_tok, int32_t n_heads, int32_t head_dim,
                int64_t tok_stride, const int32_t* pos, int32_t pos0, double base, int32_t layout, vtb_stream_t stream) {
  g_last_error.clear();
  if (!valid_dtype(dtype)) return fail(VTB_ERR_ARG, "dtype=%d", dtype);
  if (n_tok < 0 || n_heads < 1 || head_dim < 2 || (head_dim & 1))
    return fail(VTB_ERR_ARG, "bad shape n_tok=%d n_heads=%d head_dim=%d (head_dim must be even)", n_tok, n_heads, head_dim);
  if (tok_stride < (int64_t)n_heads * head_dim) return fail(VTB_ERR_ARG, "tok_stride < n_heads * head_dim");
  if (layout != 0 && layout != 1) return fail(VTB_ERR_ARG, "layout=%d must be 0 or 1", layout);
  if (!(base > 0.0) || !std::isfinite(base)) return fail(VTB_ERR_ARG, "base must be positive and finite");
  if (n_tok == 0) return VTB_OK;
  if (!dy || !dx) return fail(VTB_ERR_ARG, "dy and dx must be non-NULL");
  const size_t bytes = ((size_t)(n_tok - 1) * tok_stride + (size_t)n_heads * head_dim) * esize(dtype);
  if (dx != dy && overlap(span_of(dx, bytes), span_of(dy, bytes))) return fail(VTB_ERR_ALIAS, "dx partially overlaps dy");
  if (pos && (overlap(span_of(pos, n_tok * 4u), span_of(dx, bytes))))
    return fail(VTB_ERR_ALIAS, "pos overlaps dx");
  return hip_status(vtb::launch_rope_bwd(dtype == VTB_BF16, dy, dx, n_tok, n_heads, head_dim, tok_stride, pos, pos0, base,
                                         layout, reinterpret_cast<hipStream_t>(stream)),
                    "rope_bwd");
}

int rope_bwd(const float* dy, float* dx, int32_t n_tok, int32_t n_heads, int32_t head_dim, int64_t tok_stride,
             const int32_t* pos, int32_t pos0, double base, int32_t layout, vtb_stream_t stream) {
  return rope_bwd_ex(VTB_F32, dy, dx, n_tok, n_heads, head_dim, tok_stride, pos, pos0, base, layout, stream);
}

int rmsnorm_bwd_ex(int32_t dtype, const void* x, const float* gamma, const void* dy, void* dx, int32_t rows, int32_t n,
                   float eps, vtb_stream_t stream) {
  g_last_error.clear();
  if (!valid_dtype(dtype)) return fail(VTB_ERR_ARG, "dtype=%d", dtype);
  if (rows < 0 || n < 1) return fail(VTB_ERR_ARG, "bad shape rows=%d n=%d", rows, n);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(VTB_ERR_ARG, "eps must be finite and >= 0");
  if (rows == 0) return VTB_OK;
  if (!x || !gamma || !dy || !dx) return fail(VTB_ERR_ARG, "x, gamma, dy and dx must be non-NULL");
  const size_t bytes = (size_t)rows * n * esize(dtype);
  const Span o = span_of(dx, bytes);
  if (overlap(o, span_of(x, bytes)) || overlap(o, span_of(dy, bytes)) || overlap(o, span_of(gamma, (size_t)n * 4)))
    return fail(VTB_ERR_ALIAS, "dx overlaps an input");
  return hip_status(vtb::launch_rmsnorm_bwd(dtype == VTB_BF16, x, gamma, dy, dx, rows, n, eps,
                                            reinterpret_cast<hipStream_t>(stream)),
                    "rmsnorm_bwd");
}

int rmsnorm_bwd(const float* x, const float* gamma, const float* dy, float* dx, int32_t rows, int32_t n, float eps,
                vtb_stream_t stream) {
  return rmsnorm_bwd_ex(VTB_F32, x, gamma, dy, dx, rows, n, eps, stream);
}

int rope_rmsnorm_res_bwd(const float* dq, float dq_scale, const float* x, const float* gamma, const float* dh_out,
                         float* dh_in, int32_t T, int32_t n_heads, int32_t head_dim, int32_t pos0, double base,
                         int32_t layout, float eps, vtb_stream_t stream) {
  g_last_error.clear();
  if (T < 0 || n_heads < 1 || head_dim < 2 || (head_dim & 1)) return fail(VTB_ERR_ARG, "bad shape");
  if ((int64_t)n_heads * head_dim > 4096) return fail(VTB_ERR_UNSUPPORTED, "row width n_heads*head_dim > 4096");
  if (layout != 0 && layout != 1) return fail(VTB_ERR_ARG, "layout must be 0 or 1");
  if (!(base > 0.0) || !std::isfinite(base)) return fail(VTB_ERR_ARG, "base must be positive and finite");
  if (!(eps >= 0.f) || !std::isfinite(eps) || !std::isfinite(dq_scale)) return fail(VTB_ERR_ARG, "eps/dq_scale");
  if (T == 0) return VTB_OK;
  if (!dq || !x || !gamma || !dh_out || !dh_in) return fail(VTB_ERR_ARG, "NULL pointer");
  const size_t C = (size_t)n_heads * head_dim, bytes = (size_t)T * C * 4;
  const Span o = span_of(dh_in, bytes);
  if (overlap(o, span_of(dq, bytes)) || overlap(o, span_of(x, bytes)) || overlap(o, span_of(gamma, C * 4)))
    return fail(VTB_ERR_ALIAS, "dh_in overlaps an input");
  if (dh_in != dh_out && overlap(o, span_of(dh_out, bytes))) return fail(VTB_ERR_ALIAS, "dh_in partially overlaps dh_out");
  return hip_status(vtb::launch_rope_rmsnorm_res_bwd(dq, dq_scale, x, gamma, dh_out, dh_in, T, n_heads, head_dim, pos0,
                                                     base, layout, eps, reinterpret_cast<hipStream_t>(stream)),
                    "rope_rmsnorm_res_bwd");
}

int layernorm_bwd(int32_t dtype, const void* dy, const void* y, const float* sig, void* dx, int32_t rows, int32_t n,
                  vtb_stream_t stream) {
  g_last_error.clear();
  if (!valid_dtype(dtype)) return fail(VTB_ERR_ARG, "dtype=%d", dtype);
  if (rows < 0 || n < 1) return fail(VTB_ERR_ARG, "bad shape rows=%d n=%d", rows, n);
  if (rows == 0) return VTB_OK;
  if (!dy || !y || !sig || !dx) return fail(VTB_ERR_ARG, "dy, y, sig and dx must be non-NULL");
  const size_t bytes = (size_t)rows * n * esize(dtype);
  const Span o = span_of(dx, bytes);
  if (overlap(o, span_of(dy, bytes)) || overlap(o, span_of(y, bytes)) || overlap(o, span_of(sig, (size_t)rows * 4)))
    return fail(VTB_ERR_ALIAS, "dx overlaps an input");
  return hip_status(vtb::launch_layernorm_bwd(dtype == VTB_BF16, dy, y, sig, nullptr, dx, rows, n,
                                              reinterpret_cast<hipStream_t>(stream)),
                    "layernorm_bwd");
}

int relu2_mul_bwd(int32_t dtype, const void* gate, const void* up, const void* dh, void* dgate, void* dup, int64_t n,
                  vtb_stream_t stream) {
  g_last_error.clear();
  if (!valid_dtype(dtype)) return fail(VTB_ERR_ARG, "dtype=%d", dtype);
  if (n < 0) return fail(VTB_ERR_ARG, "n=%lld is negative", (long long)n);
  if (n == 0) return VTB_OK;
  if (!gate || !up || !dh || !dgate || !dup) return fail(VTB_ERR_ARG, "gate, up, dh, dgate and dup must be non-NULL");
  const size_t bytes = (size_t)n * esize(dtype);
  const Span sg = span_of(gate, bytes), su = span_of(up, bytes), sd = span_of(dh, bytes);
  const Span og = span_of(dgate, bytes), ou = span_of(dup, bytes);
  for (const Span& o : {og, ou})
    if (overlap(o, sg) || overlap(o, su) || overlap(o, sd)) return fail(VTB_ERR_ALIAS, "an output overlaps an input");
  if (overlap(og, ou)) return fail(VTB_ERR_ALIAS, "dgate overlaps dup");
  return hip_status(vtb::launch_relu2_mul_bwd(dtype == VTB_BF16, gate, up, dh, dgate, dup, n,
                                              reinterpret_cast<hipStream_t>(stream)),
                    "relu2_mul_bwd");
}

int linear_bwd(const float* x, const float* w, const float* dy, float* dx, float* dw, int32_t T, int32_t K, int32_t N,
               vtb_stream_t stream) {
  g_last_error.clear();
  if (T < 0 || K < 1 || N < 1) return fail(VTB_ERR_ARG, "bad shape T=%d K=%d N=%d", T, K, N);
  if (!dx && !dw) return fail(VTB_ERR_ARG, "dx and dw are both NULL");
  if (!w || !dy || (dw && !x && T > 0)) return fail(VTB_ERR_ARG, "NULL input");
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const Span sx = span_of(x, (size_t)T * K * 4), sw = span_of(w, (size_t)K * N * 4), sdy = span_of(dy, (size_t)T * N * 4);
  const Span sdx = span_of(dx, dx ? (size_t)T * K * 4 : 0), sdw = span_of(dw, dw ? (size_t)K * N * 4 : 0);
  for (const Span& o : {sdx, sdw})
    if (overlap(o, sx) || overlap(o, sw) || overlap(o, sdy)) return fail(VTB_ERR_ALIAS, "output overlaps an input");
  if (overlap(sdx, sdw)) return fail(VTB_ERR_ALIAS, "dx overlaps dw");
  for (const void* ptr : {(const void*)x, (const void*)w, (const void*)dy, (const void*)dx, (const void*)dw})
    if (ptr && !aligned16(ptr)) return fail(VTB_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  if (T == 0) return dw ? hip_status(vtb::launch_zero_f32(dw, (int64_t)K * N, s), "zero dw") : VTB_OK;
  return hip_status(vtb::launch_linear_bwd(x, w, dy, dx, dw, T, K, N, s), "linear_bwd");
}

size_t layer_bwd_workspace_size(const layer_bwd_cfg* c) {
  if (!c || c->T < 1 || c->H < 1 || (c->D != 64 && c->D != 128)) return 0;
  const size_t TC = (size_t)c->T * c->H * c->D;
  const int C = c->H * c->D;
  // dO, dq, the [H, T, T] dP / dS grid, dX partials of the split contraction
  return align256(TC * 4) * 2 + align256((size_t)c->H * c->T * c->T * 4) +
         align256((size_t)vtb::linear_bwd_splits(c->T, C, C) * TC * 4);
}

int layer_bwd(const layer_bwd_cfg* c, const layer_saved* sv, const float* dh_out, float* dh_in, float* dw, float* dk,
              float* dv, void* workspace, size_t workspace_bytes, vtb_stream_t stream) {
  g_last_error.clear();
  if (!c || !sv) return fail(VTB_ERR_ARG, "cfg and saved must be non-NULL");
  if (c->T < 1 || c->H < 1) return fail(VTB_ERR_ARG, "T=%d H=%d must be >= 1", c->T, c->H);
  if (c->D != 64 && c->D != 128) return fail(VTB_ERR_UNSUPPORTED, "head dim D=%d (supported: 64, 128)", c->D);
  if ((int64_t)c->H * c->D > 4096) return fail(VTB_ERR_UNSUPPORTED, "hidden size H*D > 4096");
  if (c->causal != 0 && c->causal != 1) return fail(VTB_ERR_ARG, "causal must be 0 or 1");
  if (c->rope_layout != 0 && c->rope_layout != 1) return fail(VTB_ERR_ARG, "rope_layout must be 0 or 1");
  if (!std::isfinite(c->scale) || !(c->eps >= 0.f) || !(c->rope_base > 0.0)) return fail(VTB_ERR_ARG, "scale/eps/rope_base");
  const float* in_ptrs[9] = {sv->x, sv->gamma, sv->w, sv->o, sv->q, sv->k, sv->v, sv->P, dh_out};
  for (const float* ptr : in_ptrs)
    if (!ptr) return fail(VTB_ERR_ARG, "a saved tensor or dh_out is NULL");
  if (!dh_in || !dw || !dk || !dv) return fail(VTB_ERR_ARG, "outputs must be non-NULL");
  for (const float* ptr : in_ptrs)
    if (!aligned16(ptr)) return fail(VTB_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  // the outputs and the workspace are written (and the workspace read back) with 16-byte vectors
  const void* out_ptrs[5] = {dh_in, dw, dk, dv, workspace};
  for (const void* ptr : out_ptrs)
    if (ptr && !aligned16(ptr)) return fail(VTB_ERR_UNSUPPORTED, "outputs and workspace must be 16-byte aligned");
  const int T = c->T, H = c->H, D = c->D, C = H * D;
  const size_t TC = (size_t)T * C * 4;
  const Span ins[9] = {span_of(sv->x, TC), span_of(sv->gamma, (size_t)C * 4), span_of(sv->w, (size_t)C * C * 4),
                       span_of(sv->o, TC), span_of(sv->q, TC), span_of(sv->k, TC), span_of(sv->v, TC),
                       span_of(sv->P, (size_t)H * T * T * 4), span_of(dh_out, TC)};
  const Span outs[4] = {span_of(dh_in, TC), span_of(dw, (size_t)C * C * 4), span_of(dk, TC), span_of(dv, TC)};
  const Span sws = span_of(workspace, workspace_bytes);
  for (int o = 0; o < 4; ++o) {
    for (int i = 0; i < 9; ++i) {
      if (o == 0 && i == 8 && dh_in == dh_out) continue;  // in place allowed
      if (overlap(outs[o], ins[i])) return fail(VTB_ERR_ALIAS, "output %d overlaps input %d", o, i);
    }
    for (int o2 = o + 1; o2 < 4; ++o2)
      if (overlap(outs[o], outs[o2])) return fail(VTB_ERR_ALIAS, "outputs %d and %d overlap", o, o2);
    if (overlap(outs[o], sws)) return fail(VTB_ERR_ALIAS, "output %d overlaps the workspace", o);
  }
  const size_t need = layer_bwd_workspace_size(c);
  if (!workspace || workspace_bytes < need)
    return fail(VTB_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0, need);
  for (int i = 0; i < 9; ++i)
    if (overlap(sws, ins[i])) return fail(VTB_ERR_ALIAS, "workspace overlaps input %d", i);

  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = reinterpret_cast<char*>(workspace);
  float* d_o = reinterpret_cast<float*>(base);
  float* dq = reinterpret_cast<float*>(base + align256(TC));
  float* ds = reinterpret_cast<float*>(base + 2 * align256(TC));
  float* part = reinterpret_cast<float*>(base + 2 * align256(TC) + align256((size_t)H * T * T * 4));

  // 1. linear backward: dO = dh_out W^T (as split-K partials), dW = o^T dh_out
  int ns = 1;
  int rc = hip_status(vtb::launch_linear_bwd_parts(sv->o, sv->w, dh_out, d_o, dw, T, C, C, part, &ns, s), "layer linear");
  if (rc) return rc;
  // 2. attention backward with the saved softmax: dO summed from the partials (and kept for
  //    dV), dP = dO V^T, dS = P o (dP - D), then dq = scale dS K (workspace),
  //    dK = scale dS^T Q, dV = P^T dO
  rc = hip_status(vtb::launch_attn_saved_p_bwd_parts(sv->q, sv->k, sv->v, ns > 1 ? part : d_o, ns, (int64_t)T * C, d_o,
                                                     sv->P, ds, dq, dk, dv, T, H, D, C, C, C, c->scale, c->causal, s),
                  "layer attention");
  if (rc) return rc;
  // 3. dh_in = dh_out + RMSNormBackward(x, gamma, RoPEBackward(dq))
  return hip_status(vtb::launch_rope_rmsnorm_res_bwd(dq, 1.0f, sv->x, sv->gamma, dh_out, dh_in, T, H, D, 0,
                                                     c->rope_base, c->rope_layout, c->eps, s),
                    "layer rope/rmsnorm/residual");
}


size_t ffn_bwd_workspace_size(const ffn_bwd_cfg* c) {
  if (!c || c->T < 1 || c->C < 1 || c->F < 1) return 0;
  const size_t T = c->T, C = c->C, F = c->F;
  // dhn [T, F], dgu [T, 2F], dxn [T, C], and the dX partials of either split contraction
  const size_t parts = std::max((size_t)vtb::linear_bwd_splits(c->T, c->F, c->C) * T * F,
                                (size_t)vtb::linear_bwd_splits(c->T, c->C, 2 * c->F) * T * C);
  return align256(T * F * 4) + align256(T * 2 * F * 4) + align256(T * C * 4) + align256(parts * 4);
}

int ffn_bwd(const ffn_bwd_cfg* c, const ffn_saved* sv, const float* dout, float* dx, float* dw_gu, float* dw_down,
            void* workspace, size_t workspace_bytes, vtb_stream_t stream) {
  g_last_error.clear();
  if (!c || !sv) return fail(VTB_ERR_ARG, "cfg and saved must be non-NULL");
  if (c->T < 1 || c->C < 1 || c->F < 1) return fail(VTB_ERR_ARG, "T=%d C=%d F=%d must be >= 1", c->T, c->C, c->F);
  if ((int64_t)c->C * 2 * c->F > (int64_t)1 << 31 || (int64_t)c->T * 2 * c->F > (int64_t)1 << 31)
    return fail(VTB_ERR_UNSUPPORTED, "a tensor exceeds 2^31 elements");
  if (!(c->eps >= 0.f) || !std::isfinite(c->eps)) return fail(VTB_ERR_ARG, "eps must be finite and >= 0");
  const float* in_ptrs[9] = {sv->x, sv->gamma1, sv->xn, sv->w_gu, sv->gu, sv->gamma2, sv->hn, sv->w_down, dout};
  for (const float* ptr : in_ptrs)
    if (!ptr) return fail(VTB_ERR_ARG, "a saved tensor or dout is NULL");
  if (!dx || !dw_gu || !dw_down) return fail(VTB_ERR_ARG, "outputs must be non-NULL");
  for (const float* ptr : in_ptrs)
    if (!aligned16(ptr)) return fail(VTB_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  if (!aligned16(dx) || !aligned16(dw_gu) || !aligned16(dw_down) || !aligned16(workspace))
    return fail(VTB_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  const int T = c->T, C = c->C, F = c->F;
  const size_t TC = (size_t)T * C * 4, TF = (size_t)T * F * 4;
  const size_t in_bytes[9] = {TC, (size_t)C * 4, TC, (size_t)C * 2 * F * 4, 2 * TF, (size_t)F * 4, TF, (size_t)F * C * 4, TC};
  Span ins[9];
  for (int i = 0; i < 9; ++i) ins[i] = span_of(in_ptrs[i], in_bytes[i]);
  const Span sdx = span_of(dx, TC), sgu = span_of(dw_gu, (size_t)C * 2 * F * 4), sdn = span_of(dw_down, (size_t)F * C * 4);
  for (int i = 0; i < 9; ++i) {
    if (i != 8 && overlap(sdx, ins[i])) return fail(VTB_ERR_ALIAS, "dx overlaps saved tensor %d", i);
    if (overlap(sgu, ins[i]) || overlap(sdn, ins[i])) return fail(VTB_ERR_ALIAS, "a weight gradient overlaps input %d", i);
  }
  if (dx != dout && overlap(sdx, ins[8])) return fail(VTB_ERR_ALIAS, "dx partially overlaps dout");
  if (overlap(sdx, sgu) || overlap(sdx, sdn) || overlap(sgu, sdn)) return fail(VTB_ERR_ALIAS, "outputs overlap");
  const size_t need = ffn_bwd_workspace_size(c);
  if (!workspace || workspace_bytes < need)
    return fail(VTB_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0, need);
  const Span sws = span_of(workspace, need);
  for (int i = 0; i < 9; ++i)
    if (overlap(sws, ins[i])) return fail(VTB_ERR_ALIAS, "workspace overlaps input %d", i);
  if (overlap(sws, sdx) || overlap(sws, sgu) || overlap(sws, sdn)) return fail(VTB_ERR_ALIAS, "workspace overlaps an output");

  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = reinterpret_cast<char*>(workspace);
  float* dhn = reinterpret_cast<float*>(base);
  float* dgu = reinterpret_cast<float*>(base + align256(TF));
  float* dxn = reinterpret_cast<float*>(base + align256(TF) + align256(2 * TF));
  float* part = reinterpret_cast<float*>(base + align256(TF) + align256(2 * TF) + align256(TC));

  // 1. ffnDown transpose: dhn = dout Wdown^T, dWdown = hn^T dout
  int rc = hip_status(vtb::launch_linear_bwd_split(sv->hn, sv->w_down, dout, dhn, dw_down, T, F, C, part, s), "ffn down");
  if (rc) return rc;
  // 2. ffnSubNorm backward fused with ReLU^2 x Mul backward: dgu = [dgate | dup]
  rc = hip_status(vtb::launch_subnorm_relu2_bwd(sv->gu, dhn, sv->gamma2, dgu, T, F, c->eps, s), "ffn sub-norm/relu2");
  if (rc) return rc;
  // 3. ffnGate/Up transposes as one product: dxn = dgu Wgu^T, dWgu = xn^T dgu
  rc = hip_status(vtb::launch_linear_bwd_split(sv->xn, sv->w_gu, dgu, dxn, dw_gu, T, C, 2 * F, part, s), "ffn gate/up");
  if (rc) return rc;
  // 4. ffnNorm backward plus the residual: dx = dout + RMSNormBackward(x, gamma1, dxn)
  return hip_status(vtb::launch_rmsnorm_res_bwd(sv->x, sv->gamma1, dxn, dout, dx, T, C, c->eps, s), "ffn norm/residual");
}


size_t attn_block_bwd_workspace_size(const attn_block_cfg* c) {
  if (!c || c->B < 1 || c->T < 1 || c->H < 1 || c->D < 1) return 0;
  const size_t BT = (size_t)c->B * c->T, C = (size_t)c->H * c->D, T = c->T;
  const int bt = c->B * c->T, ci = c->H * c->D;
  // dctx [BT, C], dS [H, T, T], dqkv [BT, 3C], dln [BT, C], dX partials of either split product
  const size_t parts = std::max((size_t)vtb::linear_bwd_splits(bt, ci, ci), (size_t)vtb::linear_bwd_splits(bt, ci, 3 * ci)) *
                       BT * C;
  return align256(BT * C * 4) * 2 + align256((size_t)c->H * T * T * 4) + align256(BT * 3 * C * 4) + align256(parts * 4);
}

int attn_block_bwd(const attn_block_cfg* c, const attn_block_saved* sv, const float* dx2, float* dx, float* dw_qkv,
                   float* dw_o, void* workspace, size_t workspace_bytes, vtb_stream_t stream) {
  g_last_error.clear();
  if (!c || !sv) return fail(VTB_ERR_ARG, "cfg and saved must be non-NULL");
  if (c->B < 1 || c->T < 1 || c->H < 1 || c->D < 1)
    return fail(VTB_ERR_ARG, "B=%d T=%d H=%d D=%d must be >= 1", c->B, c->T, c->H, c->D);
  if (!std::isfinite(c->scale)) return fail(VTB_ERR_ARG, "scale is not finite");
  if (c->causal != 0 && c->causal != 1) return fail(VTB_ERR_ARG, "causal must be 0 or 1");
  const int64_t BT = (int64_t)c->B * c->T, C = (int64_t)c->H * c->D, T = c->T;
  if (BT * 3 * C > ((int64_t)1 << 31) || C * 3 * C > ((int64_t)1 << 31) || (int64_t)c->B * c->H * T * T > ((int64_t)1 << 31))
    return fail(VTB_ERR_UNSUPPORTED, "a tensor exceeds 2^31 elements");
  const float* in_ptrs[8] = {sv->ln_y, sv->ln_sig, sv->w_qkv, sv->qkv, sv->P, sv->ctx, sv->w_o, dx2};
  for (const float* ptr : in_ptrs)
    if (!ptr) return fail(VTB_ERR_ARG, "a saved tensor or dx2 is NULL");
  if (!dx || !dw_qkv || !dw_o) return fail(VTB_ERR_ARG, "outputs must be non-NULL");
  for (const float* ptr : in_ptrs)
    if (!aligned16(ptr)) return fail(VTB_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  if (!aligned16(dx) || !aligned16(dw_qkv) || !aligned16(dw_o) || !aligned16(workspace))
    return fail(VTB_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  const size_t in_bytes[8] = {(size_t)(BT * C * 4), (size_t)(BT * 4), (size_t)(C * 3 * C * 4), (size_t)(BT * 3 * C * 4),
                              (size_t)((int64_t)c->B * c->H * T * T * 4), (size_t)(BT * C * 4), (size_t)(C * C * 4),
                              (size_t)(BT * C * 4)};
  Span ins[8];
  for (int i = 0; i < 8; ++i) ins[i] = span_of(in_ptrs[i], in_bytes[i]);
  const Span sdx = span_of(dx, BT * C * 4), sq = span_of(dw_qkv, C * 3 * C * 4), so = span_of(dw_o, C * C * 4);
  for (int i = 0; i < 8; ++i) {
    if (i != 7 && overlap(sdx, ins[i])) return fail(VTB_ERR_ALIAS, "dx overlaps saved tensor %d", i);
    if (overlap(sq, ins[i]) || overlap(so, ins[i])) return fail(VTB_ERR_ALIAS, "a weight gradient overlaps input %d", i);
  }
  if (dx != dx2 && overlap(sdx, ins[7])) return fail(VTB_ERR_ALIAS, "dx partially overlaps dx2");
  if (overlap(sdx, sq) || overlap(sdx, so) || overlap(sq, so)) return fail(VTB_ERR_ALIAS, "outputs overlap");
  const size_t need = attn_block_bwd_workspace_size(c);
  if (!workspace || workspace_bytes < need)
    return fail(VTB_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0, need);
  const Span sws = span_of(workspace, need);
  for (int i = 0; i < 8; ++i)
    if (overlap(sws, ins[i])) return fail(VTB_ERR_ALIAS, "workspace overlaps input %d", i);
  if (overlap(sws, sdx) || overlap(sws, sq) || overlap(sws, so)) return fail(VTB_ERR_ALIAS, "workspace overlaps an output");

  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int bt = (int)BT, ci = (int)C, H = c->H, D = c->D, Ti = c->T;
  char* base = reinterpret_cast<char*>(workspace);
  float* dctx = reinterpret_cast<float*>(base);
  float* dln = reinterpret_cast<float*>(base + align256(BT * C * 4));
  float* ds = reinterpret_cast<float*>(base + 2 * align256(BT * C * 4));
  float* dqkv = reinterpret_cast<float*>(base + 2 * align256(BT * C * 4) + align256((size_t)H * T * T * 4));
  float* part = reinterpret_cast<float*>(base + 2 * align256(BT * C * 4) + align256((size_t)H * T * T * 4) +
                                         align256(BT * 3 * C * 4));

  // 1. output projection: dctx = dx2 Wo^T, gWo = ctx^T dx2
  int ns = 1;
  int rc = hip_status(vtb::launch_linear_bwd_parts(sv->ctx, sv->w_o, dx2, dctx, dw_o, bt, ci, ci, part, &ns, s), "block Wo");
  if (rc) return rc;
  // 2. attention backward with the saved softmax, one sequence at a time (dS reused), dctx
  //    summed from the partials on the way, gradients written into the q | k | v thirds of dqkv
  for (int b = 0; b < c->B; ++b) {
    const int64_t r3 = (int64_t)b * Ti * 3 * C, r1 = (int64_t)b * Ti * C;
    const float* q = sv->qkv + r3;
    float* dq = dqkv + r3;
    rc = hip_status(vtb::launch_attn_saved_p_bwd_parts(q, q + C, q + 2 * C, (ns > 1 ? part : dctx) + r1, ns, BT * C,
                                                       dctx + r1, sv->P + (int64_t)b * H * T * T, ds, dq, dq + C,
                                                       dq + 2 * C, Ti, H, D, 3 * ci, ci, 3 * ci, c->scale, c->causal, s),
                    "block attention");
    if (rc) return rc;
  }
  // 3. QKV projection as one product: dln = dqkv Wqkv^T, gWqkv = ln.y^T dqkv
  rc = hip_status(vtb::launch_linear_bwd_split(sv->ln_y, sv->w_qkv, dqkv, dln, dw_qkv, bt, ci, 3 * ci, part, s),
                  "block Wqkv");
  if (rc) return rc;
  // 4. LayerNorm backward plus the residual: dx = dx2 + lnBwd(dln, ln.y, sigma)
  return hip_status(vtb::launch_layernorm_bwd(0, dln, sv->ln_y, sv->ln_sig, dx2, dx, bt, ci, s), "block layernorm");
}


size_t rms_attn_block_bwd_workspace_size(const rms_attn_block_cfg* c) {
  if (!c || c->B < 1 || c->T < 1 || c->H < 1 || c->D < 2) return 0;
  const size_t BT = (size_t)c->B * c->T, C = (size_t)c->H * c->D, T = c->T;
  const int bt = c->B * c->T, ci = c->H * c->D;
  // dctx [BT, C], dn [BT, C], dS [H, T, T], dqkv [BT, 3C], 1/r [BT], dX partials of either split product
  const size_t parts = std::max((size_t)vtb::linear_bwd_splits(bt, ci, ci), (size_t)vtb::linear_bwd_splits(bt, ci, 3 * ci)) *
                       BT * C;
  return align256(BT * C * 4) * 2 + align256((size_t)c->H * T * T * 4) + align256(BT * 3 * C * 4) + align256(BT * 4) +
         align256(parts * 4);
}

int rms_attn_block_bwd(const rms_attn_block_cfg* c, const rms_attn_block_saved* sv, const float* dx2, float* dx,
                       float* dgamma, float* dw_qkv, float* dw_o, void* workspace, size_t workspace_bytes,
                       vtb_stream_t stream) {
  g_last_error.clear();
  if (!c || !sv) return fail(VTB_ERR_ARG, "cfg and saved must be non-NULL");
  if (c->B < 1 || c->T < 1 || c->H < 1 || c->D < 2 || (c->D & 1))
    return fail(VTB_ERR_ARG, "B=%d T=%d H=%d D=%d must be >= 1 (D even, >= 2)", c->B, c->T, c->H, c->D);
  if (!std::isfinite(c->scale)) return fail(VTB_ERR_ARG, "scale is not finite");
  if (c->causal != 0 && c->causal != 1) return fail(VTB_ERR_ARG, "causal must be 0 or 1");
  if (!(c->eps > 0.f) || !std::isfinite(c->eps)) return fail(VTB_ERR_ARG, "eps must be positive and finite");
  if (!(c->rope_base > 0.0) || !std::isfinite(c->rope_base)) return fail(VTB_ERR_ARG, "rope_base must be positive");
  if (c->rope_layout != 0 && c->rope_layout != 1) return fail(VTB_ERR_ARG, "rope_layout must be 0 or 1");
  const int64_t BT = (int64_t)c->B * c->T, C = (int64_t)c->H * c->D, T = c->T;
  if (BT * 3 * C > ((int64_t)1 << 31) || C * 3 * C > ((int64_t)1 << 31) || (int64_t)c->B * c->H * T * T > ((int64_t)1 << 31))
    return fail(VTB_ERR_UNSUPPORTED, "a tensor exceeds 2^31 elements");
  const float* in_ptrs[9] = {sv->x, sv->gamma, sv->n, sv->w_qkv, sv->qkv, sv->P, sv->ctx, sv->w_o, dx2};
  for (const float* ptr : in_ptrs)
    if (!ptr) return fail(VTB_ERR_ARG, "a saved tensor or dx2 is NULL");
  if (!dx || !dgamma || !dw_qkv || !dw_o) return fail(VTB_ERR_ARG, "outputs must be non-NULL");
  for (const float* ptr : in_ptrs)
    if (!aligned16(ptr)) return fail(VTB_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  if (!aligned16(dx) || !aligned16(dgamma) || !aligned16(dw_qkv) || !aligned16(dw_o) || !aligned16(workspace))
    return fail(VTB_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  const size_t in_bytes[9] = {(size_t)(BT * C * 4), (size_t)(C * 4), (size_t)(BT * C * 4), (size_t)(C * 3 * C * 4),
                              (size_t)(BT * 3 * C * 4), (size_t)((int64_t)c->B * c->H * T * T * 4), (size_t)(BT * C * 4),
                              (size_t)(C * C * 4), (size_t)(BT * C * 4)};
  Span ins[9];
  for (int i = 0; i < 9; ++i) ins[i] = span_of(in_ptrs[i], in_bytes[i]);
  const Span sdx = span_of(dx, BT * C * 4), sg = span_of(dgamma, C * 4), sq = span_of(dw_qkv, C * 3 * C * 4),
             so = span_of(dw_o, C * C * 4);
  for (int i = 0; i < 9; ++i) {
    if (i != 8 && overlap(sdx, ins[i])) return fail(VTB_ERR_ALIAS, "dx overlaps saved tensor %d", i);
    if (overlap(sg, ins[i]) || overlap(sq, ins[i]) || overlap(so, ins[i]))
      return fail(VTB_ERR_ALIAS, "a parameter gradient overlaps input %d", i);
  }
  if (dx != dx2 && overlap(sdx, ins[8])) return fail(VTB_ERR_ALIAS, "dx partially overlaps dx2");
  const Span outs[4] = {sdx, sg, sq, so};
  for (int a = 0; a < 4; ++a)
    for (int b = a + 1; b < 4; ++b)
      if (overlap(outs[a], outs[b])) return fail(VTB_ERR_ALIAS, "outputs overlap");
  const size_t need = rms_attn_block_bwd_workspace_size(c);
  if (!workspace || workspace_bytes < need)
    return fail(VTB_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0, need);
  const Span sws = span_of(workspace, need);
  for (int i = 0; i < 9; ++i)
    if (overlap(sws, ins[i])) return fail(VTB_ERR_ALIAS, "workspace overlaps input %d", i);
  for (int a = 0; a < 4; ++a)
    if (overlap(sws, outs[a])) return fail(VTB_ERR_ALIAS, "workspace overlaps an output");

  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int bt = (int)BT, ci = (int)C, H = c->H, D = c->D, Ti = c->T;
  char* base = reinterpret_cast<char*>(workspace);
  size_t off = 0;
  auto carve = [&](size_t bytes) {
    float* ptr = reinterpret_cast<float*>(base + off);
    off += align256(bytes);
    return ptr;
  };
  float* dctx = carve(BT * C * 4);
  float* dn = carve(BT * C * 4);
  float* ds = carve((size_t)H * T * T * 4);
  float* dqkv = carve(BT * 3 * C * 4);
  float* rinv = carve(BT * 4);
  float* part = carve(0);

  // 1. output projection: dctx = dx2 Wo^T, gWo = ctx^T dx2
  int ns = 1;
  int rc = hip_status(vtb::launch_linear_bwd_parts(sv->ctx, sv->w_o, dx2, dctx, dw_o, bt, ci, ci, part, &ns, s), "layer Wo");
  if (rc) return rc;
  for (int b = 0; b < c->B; ++b) {
    const int64_t r3 = (int64_t)b * Ti * 3 * C, r1 = (int64_t)b * Ti * C;
    const float* q = sv->qkv + r3;
    float* dq = dqkv + r3;
    // 2. attention backward with the saved softmax into the q | k | v thirds of dqkv, dctx
    //    summed from the partials on the way
    rc = hip_status(vtb::launch_attn_saved_p_bwd_parts(q, q + C, q + 2 * C, (ns > 1 ? part : dctx) + r1, ns, BT * C,
                                                       dctx + r1, sv->P + (int64_t)b * H * T * T, ds, dq, dq + C,
                                                       dq + 2 * C, Ti, H, D, 3 * ci, ci, 3 * ci, c->scale, c->causal, s),
                    "layer attention");
    if (rc) return rc;
    // 3. RoPE backward on dq and dk in place: their 2H heads are the first 2C columns of
    //    each dqkv row, positions 0 .. T-1 of this sequence
    rc = hip_status(vtb::launch_rope_bwd(0, dq, dq, Ti, 2 * H, D, 3 * C, nullptr, 0, c->rope_base, c->rope_layout, s),
                    "layer RoPE backward");
    if (rc) return rc;
  }
  // 4. Q/K/V projection as one product: dn = dqkv Wqkv^T, gWqkv = n^T dqkv
  rc = hip_status(vtb::launch_linear_bwd_split(sv->n, sv->w_qkv, dqkv, dn, dw_qkv, bt, ci, 3 * ci, part, s), "layer Wqkv");
  if (rc) return rc;
  // 5. RMSNorm backward plus the residual (dx = dx2 + RMSNormBackward(x, gamma, dn), 1/r kept),
  //    then the gain gradient dgamma = sum_t dn_t o x_t / r_t
  rc = hip_status(vtb::launch_rmsnorm_res_bwd(sv->x, sv->gamma, dn, dx2, dx, bt, ci, c->eps, s, rinv), "layer RMSNorm");
  if (rc) return rc;
  return hip_status(vtb::launch_rmsnorm_gamma(sv->x, dn, rinv, dgamma, bt, ci, s), "layer RMSNorm gain");
}

}  // extern "C"
