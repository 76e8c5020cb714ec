// C ABI of libcsa.so: host-side validation of every argument, then the
// launch.  Nothing is enqueued unless all checks pass.  A call with no rows
// to process returns CSA_OK once its sizes are known to be >= 0, before any
// pointer is looked at (zero-element arrays often have NULL addresses).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <mutex>

#include "common.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

csa_status fail(csa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

csa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return CSA_OK;
  return fail(CSA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// CSA_DEBUG_SYNC=1: synchronise the stream after a launch and report any
// asynchronous failure of the enqueued kernels.
csa_status launched(hipError_t e, hipStream_t stream, const char* what) {
  if (e != hipSuccess) return hip_status(e, what);
  const char* dbg = getenv("CSA_DEBUG_SYNC");
  if (dbg && dbg[0] == '1') {
    e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return fail(CSA_EHIP, "%s (CSA_DEBUG_SYNC): %s", what, hipGetErrorString(e));
  }
  return CSA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool dim_ok(int d) { return d == 32 || d == 64 || d == 128 || d == 256 || d == 512; }

int expected_row_bytes(const csa_store& s) {
  switch (s.fmt) {
    case CSA_F32: return 4 * s.dim;
    case CSA_FP8_E4M3: return (s.dim - s.rope_dim) + 2 * s.rope_dim;
    case CSA_MXFP4: return s.dim / 2;
    default: return -1;
  }
}

// Common checks of an entry store.
csa_status check_store(const csa_store& s, const char* name) {
  if (!s.rows) return fail(CSA_EINVAL, "%s.rows is NULL", name);
  if (!aligned(s.rows, 16)) return fail(CSA_EINVAL, "%s.rows is not 16-byte aligned", name);
  if (s.cap < 0) return fail(CSA_EINVAL, "%s.cap < 0", name);
  if (!dim_ok(s.dim)) return fail(CSA_EUNSUPPORTED, "%s.dim = %d (supported: 32, 64, 128, 256, 512)", name, s.dim);
  if (s.fmt != CSA_F32 && s.fmt != CSA_FP8_E4M3 && s.fmt != CSA_MXFP4)
    return fail(CSA_EUNSUPPORTED, "%s.fmt = %d is not a store format", name, s.fmt);
  if (s.rope_dim < 0 || s.rope_dim >= s.dim) return fail(CSA_EINVAL, "%s.rope_dim out of range", name);
  if (s.fmt != CSA_FP8_E4M3 && s.rope_dim != 0)
    return fail(CSA_EUNSUPPORTED, "%s: rope_dim is only meaningful for FP8 stores", name);
  if (s.fmt == CSA_FP8_E4M3 && ((s.dim - s.rope_dim) % 16 != 0 || s.rope_dim % 8 != 0))
    return fail(CSA_EUNSUPPORTED, "%s: FP8 stores need (dim - rope_dim) %% 16 == 0 and rope_dim %% 8 == 0", name);
  if (s.fmt == CSA_MXFP4 && s.dim > 64) return fail(CSA_EUNSUPPORTED, "%s: MXFP4 stores need dim <= 64", name);
  if (s.row_bytes != expected_row_bytes(s))
    return fail(CSA_EINVAL, "%s.row_bytes = %d, expected %d", name, s.row_bytes, expected_row_bytes(s));
  if (s.fmt != CSA_MXFP4 && s.row_bytes % 16 != 0) return fail(CSA_EINVAL, "%s.row_bytes %% 16 != 0", name);
  if (s.fmt != CSA_F32 && !s.scales) return fail(CSA_EINVAL, "%s.scales is NULL", name);
  if (s.fmt == CSA_FP8_E4M3 && !aligned(s.scales, 4)) return fail(CSA_EINVAL, "%s.scales not 4-byte aligned", name);
  return CSA_OK;
}

csa_status check_kv_pair(const csa_store& a, const char* an, const csa_store& b, const char* bn) {
  if (a.fmt != b.fmt || a.dim != b.dim || a.rope_dim != b.rope_dim || a.row_bytes != b.row_bytes)
    return fail(CSA_EUNSUPPORTED, "%s and %s must share format, dim and rope_dim", an, bn);
  if (a.fmt == CSA_MXFP4) return fail(CSA_EUNSUPPORTED, "%s: attention entries must be F32 or FP8", an);
  return CSA_OK;
}

csa_status check_q(const void* q, int q_fmt, int H, int dim, const void* out) {
  if (!q) return fail(CSA_EINVAL, "q is NULL");
  if (!out) return fail(CSA_EINVAL, "out is NULL");
  if (q_fmt != CSA_F32 && q_fmt != CSA_BF16) return fail(CSA_EUNSUPPORTED, "q_fmt must be CSA_F32 or CSA_BF16");
  // the MFMA kernel moves q and out rows with 16-byte accesses
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(CSA_EINVAL, "q and out must be 16-byte aligned");
  if (H < 1) return fail(CSA_EINVAL, "H < 1");
  if (!csa::attn_supported(H, dim)) return fail(CSA_EUNSUPPORTED, "H = %d with dim = %d is not supported", H, dim);
  return CSA_OK;
}

#define CSA_TRY(x) do { csa_status _s = (x); if (_s != CSA_OK) return _s; } while (0)

// The optional RMSNorm / partial RoPE of rows of `dim` values.
csa_status check_post(const csa_norm_rope* p, int dim, const char* name) {
  if (!p) return CSA_OK;
  if (p->norm_gain && !aligned(p->norm_gain, 16)) return fail(CSA_EINVAL, "%s.norm_gain must be 16-byte aligned", name);
  if (p->norm_gain && (!std::isfinite(p->norm_eps) || p->norm_eps < 0.0f))
    return fail(CSA_EINVAL, "%s.norm_eps must be finite and >= 0", name);
  if (p->rope_dims < 0 || p->rope_dims > dim || p->rope_dims % 2 != 0)
    return fail(CSA_EINVAL, "%s.rope_dims = %d must be even and within [0, %d]", name, p->rope_dims, dim);
  if (p->rope_dims > 0 && (!p->rope_theta || !aligned(p->rope_theta, 4)))
    return fail(CSA_EINVAL, "%s.rope_theta must be a 4-byte aligned array when rope_dims > 0", name);
  return CSA_OK;
}

// Scratch of the allocation-free decode entry point: split partials of the
// decode attention (float32 o, m, l per head and split).  Each device holds
// its own copy for the life of the process.  In host code `scratch` names a
// host-side stand-in, never the device memory: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kScratchBytes = (size_t)48 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

csa_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(CSA_EUNSUPPORTED, "device %d beyond the scratch table", dev);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return CSA_OK;
}

}  // namespace

extern "C" {

const char* csa_version(void) { return "csa-mi355x 0.1.0 (gfx950)"; }

const char* csa_status_string(int s) {
  switch (s) {
    case CSA_OK: return "CSA_OK";
    case CSA_EINVAL: return "CSA_EINVAL: invalid argument";
    case CSA_EUNSUPPORTED: return "CSA_EUNSUPPORTED: unsupported format or shape";
    case CSA_EWORKSPACE: return "CSA_EWORKSPACE: workspace missing or too small";
    case CSA_EHIP: return "CSA_EHIP: HIP error";
    default: return "unknown csa_status";
  }
}

const char* csa_last_error(void) { return g_err; }

csa_status csa_compress_kv(const void* tok, int tok_fmt, int B, int64_t T, int64_t tok_bstride, int m,
                           const float* gate, const float* bias, csa_store out, int64_t out_row0,
                           const csa_norm_rope* post, hipStream_t stream) {
  g_err[0] = 0;
  if (B < 0 || T < 0) return fail(CSA_EINVAL, "B and T must be >= 0");
  if ((int64_t)B * T == 0) return CSA_OK;
  if (m < 1 || m > csa::compress_max_m()) return fail(CSA_EINVAL, "m = %d outside [1, %d]", m, csa::compress_max_m());
  if (!tok || !gate || !bias) return fail(CSA_EINVAL, "tok, gate and bias must be non-NULL");
  if (tok_fmt != CSA_F32 && tok_fmt != CSA_BF16) return fail(CSA_EUNSUPPORTED, "tok_fmt must be CSA_F32 or CSA_BF16");
  CSA_TRY(check_store(out, "out"));
  const int es = tok_fmt == CSA_F32 ? 4 : 2;
  if (!aligned(tok, 16) || (tok_bstride * es) % 16 != 0)
    return fail(CSA_EINVAL, "tok must be 16-byte aligned with a 16-byte multiple batch stride");
  if (B > 1 && tok_bstride < T * out.dim) return fail(CSA_EINVAL, "tok_bstride < T * dim");
  const int vpl = out.dim >= 64 ? out.dim / 64 : 1;
  if (out.fmt == CSA_FP8_E4M3 && out.rope_dim % vpl != 0)
    return fail(CSA_EUNSUPPORTED, "rope_dim must be a multiple of dim / 64");
  if (out.fmt == CSA_MXFP4 && out.dim > 64) return fail(CSA_EUNSUPPORTED, "MXFP4 output needs dim <= 64");
  if (out_row0 < 0 || out_row0 + T / m > out.cap) return fail(CSA_EINVAL, "out_row0 + floor(T/m) > out.cap");
  CSA_TRY(check_post(post, out.dim, "post"));
  return launched(csa::launch_compress(tok, tok_fmt, B, T, tok_bstride, m, gate, bias, out, out_row0,
                                       csa::norm_rope_of(post), stream),
                  stream, "csa_compress_kv launch");
}

csa_status csa_decode_append(const void* tok, int tok_fmt, int B, const int64_t* pos, void* tail, int tail_rows,
                             int m, const float* gate, const float* bias, csa_store out, csa_store win, int W,
                             const csa_norm_rope* post, hipStream_t stream) {
  g_err[0] = 0;
  if (B < 0) return fail(CSA_EINVAL, "B must be >= 0");
  if (B == 0) return CSA_OK;
  if (m < 1 || m > csa::compress_max_m()) return fail(CSA_EINVAL, "m = %d outside [1, %d]", m, csa::compress_max_m());
  if (!tok || !pos || !tail || !gate || !bias) return fail(CSA_EINVAL, "tok, pos, tail, gate and bias must be non-NULL");
  if (tok_fmt != CSA_F32 && tok_fmt != CSA_BF16) return fail(CSA_EUNSUPPORTED, "tok_fmt must be CSA_F32 or CSA_BF16");
  if (!aligned(tok, 16) || !aligned(tail, 16)) return fail(CSA_EINVAL, "tok and tail must be 16-byte aligned");
  if (!aligned(pos, 8)) return fail(CSA_EINVAL, "pos must be 8-byte aligned");
  if (tail_rows < m || tail_rows % m != 0) return fail(CSA_EINVAL, "tail_rows = %d is not a positive multiple of m", tail_rows);
  CSA_TRY(check_store(out, "out"));
  const int vpl = out.dim >= 64 ? out.dim / 64 : 1;
  if (out.fmt == CSA_FP8_E4M3 && out.rope_dim % vpl != 0)
    return fail(CSA_EUNSUPPORTED, "rope_dim must be a multiple of dim / 64");
  if (win.rows) {
    CSA_TRY(check_store(win, "win"));
    if (win.dim != out.dim) return fail(CSA_EINVAL, "win.dim != out.dim");
    if (W < 1 || W > win.cap) return fail(CSA_EINVAL, "W = %d outside [1, win.cap]", W);
    if (win.fmt == CSA_FP8_E4M3 && win.rope_dim % vpl != 0)
      return fail(CSA_EUNSUPPORTED, "win.rope_dim must be a multiple of dim / 64");
  }
  CSA_TRY(check_post(post, out.dim, "post"));
  return launched(csa::launch_decode_append(tok, tok_fmt, B, pos, tail, tail_rows, m, gate, bias, out, win, W,
                                            csa::norm_rope_of(post), stream),
                  stream, "csa_decode_append launch");
}

csa_status csa_decode_rebuild(const void* tok, int tok_fmt, int B, int n, int64_t bstride, const int64_t* p0,
                              const int32_t* n_valid, void* tail, int tail_rows, int m, const float* gate, const float* bias, csa_store out,
                              csa_store win, int W, const csa_norm_rope* post, hipStream_t stream) {
  g_err[0] = 0;
  if (B < 0 || n < 0) return fail(CSA_EINVAL, "B and n must be >= 0");
  if ((int64_t)B * n == 0) return CSA_OK;
  if (m < 1 || m > csa::compress_max_m()) return fail(CSA_EINVAL, "m = %d outside [1, %d]", m, csa::compress_max_m());
  if (!tok || !p0 || !tail || !gate || !bias) return fail(CSA_EINVAL, "tok, p0, tail, gate and bias must be non-NULL");
  if (tok_fmt != CSA_F32 && tok_fmt != CSA_BF16) return fail(CSA_EUNSUPPORTED, "tok_fmt must be CSA_F32 or CSA_BF16");
  if (!aligned(tok, 16) || !aligned(tail, 16)) return fail(CSA_EINVAL, "tok and tail must be 16-byte aligned");
  if (!aligned(p0, 8) || !aligned(n_valid, 4)) return fail(CSA_EINVAL, "p0 must be 8-byte and n_valid 4-byte aligned");
  if (tail_rows < m || tail_rows % m != 0) return fail(CSA_EINVAL, "tail_rows = %d is not a positive multiple of m", tail_rows);
  CSA_TRY(check_store(out, "out"));
  const int esz = tok_fmt == CSA_F32 ? 4 : 2;
  if (B > 1 && bstride < (int64_t)n * out.dim) return fail(CSA_EINVAL, "bstride below n * dim");
  if ((bstride * esz) % 16 != 0) return fail(CSA_EINVAL, "bstride must keep rows 16-byte aligned");
  const int vpl = out.dim >= 64 ? out.dim / 64 : 1;
  if (out.fmt == CSA_FP8_E4M3 && out.rope_dim % vpl != 0)
    return fail(CSA_EUNSUPPORTED, "rope_dim must be a multiple of dim / 64");
  if (win.rows) {
    CSA_TRY(check_store(win, "win"));
    if (win.dim != out.dim) return fail(CSA_EINVAL, "win.dim != out.dim");
    if (W < 1 || W > win.cap) return fail(CSA_EINVAL, "W = %d outside [1, win.cap]", W);
    if (win.fmt == CSA_FP8_E4M3 && win.rope_dim % vpl != 0)
      return fail(CSA_EUNSUPPORTED, "win.rope_dim must be a multiple of dim / 64");
  }
  CSA_TRY(check_post(post, out.dim, "post"));
  return launched(csa::launch_decode_rebuild(tok, tok_fmt, B, n, bstride, p0, n_valid, tail, tail_rows, m, gate, bias,
                                             out, win, W, csa::norm_rope_of(post), stream),
                  stream, "csa_decode_rebuild launch");
}

size_t csa_indexer_topk_workspace(int B, int Tq, int64_t n_entries, int k) {
  if (B < 0 || Tq < 0 || k < 1) return 0;
  csa::IdxPlan p = csa::indexer_plan(B, Tq, n_entries, k);
  return p.ok ? p.ws : 0;
}

csa_status csa_indexer_topk(csa_store q_idx, const float* head_w, csa_store keys, int64_t n_entries,
                            const int64_t* q_pos, int B, int Tq, int H_I, int m, int k, int32_t* sel,
                            float* sel_score, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (B < 0 || Tq < 0) return fail(CSA_EINVAL, "B and Tq must be >= 0");
  if ((int64_t)B * Tq == 0) return CSA_OK;
  if (H_I < 1 || H_I > 16) return fail(CSA_EUNSUPPORTED, "H_I = %d outside [1, 16]", H_I);
  if (k < 1 || k > 2048) return fail(CSA_EUNSUPPORTED, "k = %d outside [1, 2048]", k);
  if (m < 1) return fail(CSA_EINVAL, "m < 1");
  if (!head_w || !sel) return fail(CSA_EINVAL, "head_w and sel must be non-NULL");
  CSA_TRY(check_store(q_idx, "q_idx"));
  CSA_TRY(check_store(keys, "keys"));
  if (keys.dim != 32 && keys.dim != 64) return fail(CSA_EUNSUPPORTED, "indexer dim must be 32 or 64");
  if (q_idx.fmt != keys.fmt || q_idx.dim != keys.dim || q_idx.rope_dim != 0 || keys.rope_dim != 0)
    return fail(CSA_EUNSUPPORTED, "q_idx and keys must share format and dim, with rope_dim 0");
  if (n_entries < 0 || n_entries > keys.cap) return fail(CSA_EINVAL, "n_entries outside [0, keys.cap]");
  if (q_idx.cap < (int64_t)Tq * H_I) return fail(CSA_EINVAL, "q_idx.cap < Tq * H_I");
  csa::IdxPlan plan = csa::indexer_plan(B, Tq, n_entries, k);
  if (csa::indexer_stream_ok(keys, H_I, B, Tq, n_entries, k)) plan.ws = 0;
  else if (!plan.ok) return fail(CSA_EUNSUPPORTED, "n_entries * k too large for the candidate merge");
  if (plan.ws > 0 && (!ws || ws_bytes < plan.ws))
    return fail(CSA_EWORKSPACE, "workspace of %zu bytes needed, %zu given", plan.ws, ws ? ws_bytes : (size_t)0);
  if (plan.ws > 0 && !aligned(ws, 16)) return fail(CSA_EINVAL, "ws must be 16-byte aligned");
  return launched(csa::launch_indexer(q_idx, head_w, keys, n_entries, q_pos, B, Tq, H_I, m, k, sel, sel_score, ws,
                                      plan, stream),
                  stream, "csa_indexer_topk launch");
}

size_t csa_attn_workspace(int B, int Tq, int H, int dim, int64_t max_list) {
  if (B < 0 || Tq < 0 || H < 1 || max_list < 0) return 0;
  return csa::attn_workspace(B, Tq, H, dim, max_list);
}

static csa_status run_attn(csa::AttnCall& c, int flags, const csa_norm_rope* q_post, hipStream_t stream,
                           const char* what) {
  CSA_TRY(check_post(q_post, c.D, "q_post"));
  c.qn = csa::norm_rope_of(q_post);
  if (flags & ~(CSA_ATTN_PARTIAL | CSA_WIN_RING | CSA_BATCH_INVARIANT))
    return fail(CSA_EINVAL, "unknown flags 0x%x", flags);
  if (!std::isfinite(c.tau)) return fail(CSA_EINVAL, "sm_scale must be finite");
  if (c.W < 0 || c.W > 65536) return fail(CSA_EINVAL, "W outside [0, 65536]");
  c.partial = (flags & CSA_ATTN_PARTIAL) != 0;
  if (c.partial && c.prior_o) return fail(CSA_EINVAL, "swa_merge takes no CSA_ATTN_PARTIAL flag");
  if (c.partial) c.W = 0;   // compressed entries only
  const int64_t max_list = (c.mode == csa::kModeSel ? c.k : (c.mode == csa::kModeRange ? c.n_entries : 0)) + c.W;
  // The workspace is optional: without one every query runs in a single
  // workgroup; with one, few-query calls split long entry lists.
  const size_t need = c.prior_o ? 0 : csa::attn_workspace(c.B, c.Tq, c.H, c.D, max_list);
  if (need > 0 && c.ws && c.ws_bytes < need)
    return fail(CSA_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, c.ws_bytes);
  if (need > 0 && c.ws && !aligned(c.ws, 16)) return fail(CSA_EINVAL, "ws must be 16-byte aligned");
  c.invariant = (flags & CSA_BATCH_INVARIANT) != 0;
  c.allow_split = need > 0 && c.ws != nullptr && (!c.invariant || c.Tq == 1);
  return launched(csa::launch_attn(c, stream), stream, what);
}

static csa::AttnCall base_call(const void* q, int q_fmt, int B, int Tq, int H, int D, float sm_scale,
                               const float* sink, void* out, float* lse) {
  csa::AttnCall c;
  memset(&c, 0, sizeof(c));
  c.q = q; c.q_fmt = q_fmt; c.B = B; c.Tq = Tq; c.H = H; c.D = D;
  c.tau = sm_scale; c.sink = sink; c.out = out; c.lse = lse;
  return c;
}

csa_status csa_sparse_attn_prefill(const void* q, int q_fmt, int B, int T, int H, csa_store ckv,
                                   int64_t n_entries, const int32_t* sel, int k, csa_store win, int W,
                                   const float* sink, float sm_scale, void* out, float* lse, int flags,
                                   const csa_norm_rope* q_post, hipStream_t stream) {
  g_err[0] = 0;
  if (B < 0 || T < 0) return fail(CSA_EINVAL, "B and T must be >= 0");
  if ((int64_t)B * T == 0) return CSA_OK;
  CSA_TRY(check_store(ckv, "ckv"));
  CSA_TRY(check_store(win, "win"));
  CSA_TRY(check_kv_pair(ckv, "ckv", win, "win"));
  CSA_TRY(check_q(q, q_fmt, H, ckv.dim, out));
  if (!sel) return fail(CSA_EINVAL, "sel is NULL");
  if (k < 1) return fail(CSA_EINVAL, "k < 1");
  if (flags & CSA_WIN_RING) return fail(CSA_EINVAL, "prefill windows are position-indexed (no CSA_WIN_RING)");
  if (n_entries < 0 || n_entries > ckv.cap) return fail(CSA_EINVAL, "n_entries outside [0, ckv.cap]");
  if (!(flags & CSA_ATTN_PARTIAL) && W > 0 && win.cap < T) return fail(CSA_EINVAL, "win.cap < T");
  csa::AttnCall c = base_call(q, q_fmt, B, T, H, ckv.dim, sm_scale, sink, out, lse);
  c.ckv = ckv; c.n_entries = n_entries; c.mode = csa::kModeSel; c.sel = sel; c.k = k; c.m = 1;
  c.win = win; c.W = W; c.ring = 0;
  return run_attn(c, flags, q_post, stream, "csa_sparse_attn_prefill launch");
}

csa_status csa_sparse_attn_decode(const void* q, int q_fmt, int B, int H, csa_store ckv, int64_t n_entries,
                                  const int32_t* sel, int k, csa_store ring, const int64_t* pos, int W,
                                  const float* sink, float sm_scale, void* out, float* lse, int flags,
                                  void* ws, size_t ws_bytes, const csa_norm_rope* q_post, hipStream_t stream) {
  g_err[0] = 0;
  if (B < 0) return fail(CSA_EINVAL, "B must be >= 0");
  if (B == 0) return CSA_OK;
  CSA_TRY(check_store(ckv, "ckv"));
  CSA_TRY(check_store(ring, "ring"));
  CSA_TRY(check_kv_pair(ckv, "ckv", ring, "ring"));
  CSA_TRY(check_q(q, q_fmt, H, ckv.dim, out));
  if (!sel || !pos) return fail(CSA_EINVAL, "sel and pos must be non-NULL");
  if (k < 1) return fail(CSA_EINVAL, "k < 1");
  if (n_entries < 0 || n_entries > ckv.cap) return fail(CSA_EINVAL, "n_entries outside [0, ckv.cap]");
  if (!(flags & CSA_ATTN_PARTIAL) && W > 0 && ring.cap < W) return fail(CSA_EINVAL, "ring.cap < W");
  csa::AttnCall c = base_call(q, q_fmt, B, 1, H, ckv.dim, sm_scale, sink, out, lse);
  c.ckv = ckv; c.n_entries = n_entries; c.mode = csa::kModeSel; c.sel = sel; c.k = k; c.m = 1;
  c.win = ring; c.W = W; c.ring = 1; c.q_pos = pos; c.ws = ws; c.ws_bytes = ws_bytes;
  return run_attn(c, flags, q_post, stream, "csa_sparse_attn_decode launch");
}

csa_status csa_sparse_attn_decode_noalloc(const void* q, int q_fmt, int B, int H, csa_store ckv, int64_t n_entries,
                                          const int32_t* sel, int k, csa_store ring, const int64_t* pos, int W,
                                          const float* sink, float sm_scale, void* out, float* lse, int flags,
                                          const csa_norm_rope* q_post, hipStream_t stream) {
  g_err[0] = 0;
  if (B < 0) return fail(CSA_EINVAL, "B must be >= 0");
  if (B == 0) return CSA_OK;
  if (H < 1 || k < 1) return fail(CSA_EINVAL, "H >= 1 and k >= 1 needed");
  const int64_t max_list = (int64_t)k + ((flags & CSA_ATTN_PARTIAL) ? 0 : (W > 0 ? W : 0));
  const size_t need = csa::attn_workspace(B, 1, H, ckv.dim, max_list);
  if (need > kScratchBytes)
    return fail(CSA_EINVAL, "these sizes need %zu bytes of scratch, more than the %zu bytes of the no-allocation path",
                need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) CSA_TRY(scratch_of_current_device(&ws));
  return csa_sparse_attn_decode(q, q_fmt, B, H, ckv, n_entries, sel, k, ring, pos, W, sink, sm_scale, out, lse, flags,
                                ws, need > 0 ? kScratchBytes : 0, q_post, stream);
}

csa_status hca_attn(const void* q, int q_fmt, int B, int Tq, int H, csa_store hkv, int m_prime,
                    int64_t n_entries, const int64_t* q_pos, csa_store win, int W, const float* sink,
                    float sm_scale, void* out, float* lse, int flags, void* ws, size_t ws_bytes,
                    const csa_norm_rope* q_post, hipStream_t stream) {
  g_err[0] = 0;
  if (B < 0 || Tq < 0) return fail(CSA_EINVAL, "B and Tq must be >= 0");
  if ((int64_t)B * Tq == 0) return CSA_OK;
  if (m_prime < 1) return fail(CSA_EINVAL, "m_prime < 1");
  CSA_TRY(check_store(hkv, "hkv"));
  CSA_TRY(check_store(win, "win"));
  CSA_TRY(check_kv_pair(hkv, "hkv", win, "win"));
  CSA_TRY(check_q(q, q_fmt, H, hkv.dim, out));
  if (n_entries < 0 || n_entries > hkv.cap) return fail(CSA_EINVAL, "n_entries outside [0, hkv.cap]");
  const bool ring = (flags & CSA_WIN_RING) != 0;
  if (ring && !q_pos) return fail(CSA_EINVAL, "CSA_WIN_RING needs q_pos");
  if (!(flags & CSA_ATTN_PARTIAL) && W > 0) {
    if (ring && win.cap < W) return fail(CSA_EINVAL, "win.cap < W");
    if (!ring && !q_pos && win.cap < Tq) return fail(CSA_EINVAL, "win.cap < Tq");
  }
  csa::AttnCall c = base_call(q, q_fmt, B, Tq, H, hkv.dim, sm_scale, sink, out, lse);
  c.ckv = hkv; c.n_entries = n_entries; c.mode = csa::kModeRange; c.m = m_prime;
  c.win = win; c.W = W; c.ring = ring; c.q_pos = q_pos; c.ws = ws; c.ws_bytes = ws_bytes;
  return run_attn(c, flags, q_post, stream, "hca_attn launch");
}

csa_status swa_merge(const void* q, int q_fmt, int B, int Tq, int H, csa_store win, const int64_t* q_pos, int W,
                     int flags, const float* part_out, const float* part_lse, const float* sink, float sm_scale,
                     void* out, const csa_norm_rope* q_post, hipStream_t stream) {
  g_err[0] = 0;
  if (B < 0 || Tq < 0) return fail(CSA_EINVAL, "B and Tq must be >= 0");
  if ((int64_t)B * Tq == 0) return CSA_OK;
  if (flags & CSA_ATTN_PARTIAL) return fail(CSA_EINVAL, "swa_merge takes no CSA_ATTN_PARTIAL flag");
  CSA_TRY(check_store(win, "win"));
  if (win.fmt == CSA_MXFP4) return fail(CSA_EUNSUPPORTED, "window rows must be F32 or FP8");
  CSA_TRY(check_q(q, q_fmt, H, win.dim, out));
  if (!part_out || !part_lse) return fail(CSA_EINVAL, "part_out and part_lse must be non-NULL");
  if (!aligned(part_out, 16) || !aligned(part_lse, 4)) return fail(CSA_EINVAL, "part_out must be 16-byte aligned");
  const bool ring = (flags & CSA_WIN_RING) != 0;
  if (ring && !q_pos) return fail(CSA_EINVAL, "CSA_WIN_RING needs q_pos");
  if (W > 0 && ring && win.cap < W) return fail(CSA_EINVAL, "win.cap < W");
  if (W > 0 && !ring && !q_pos && win.cap < Tq) return fail(CSA_EINVAL, "win.cap < Tq");
  csa::AttnCall c = base_call(q, q_fmt, B, Tq, H, win.dim, sm_scale, sink, out, nullptr);
  c.mode = csa::kModeNone; c.win = win; c.W = W; c.ring = ring; c.q_pos = q_pos;
  c.prior_o = part_out; c.prior_lse = part_lse;
  return run_attn(c, flags, q_post, stream, "swa_merge launch");
}

csa_status csa_diag_counters(uint64_t* out, int n, int reset) {
  g_err[0] = 0;
  if (!out || n < 0) return fail(CSA_EINVAL, "out is NULL or n < 0");
  return hip_status(csa::diag_counters(out, n, reset != 0), "csa_diag_counters");
}

}  // extern "C"
