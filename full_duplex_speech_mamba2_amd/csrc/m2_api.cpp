// C-ABI layer of libm2.so: argument validation, handles and dispatch.
// Every check runs on the host before anything is enqueued; the operation and
// its sources are described in include/m2.h.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "m2_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return M2_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int gcd(int a, int b) {
  while (b) {
    int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

int check_config(const m2_config *c) {
  if (!c) return fail(M2_ERR_NULL, "config is NULL");
  if (c->d_model <= 0 || c->n_heads <= 0 || c->head_dim <= 0 || c->d_state <= 0 || c->n_groups <= 0)
    return fail(M2_ERR_SHAPE, "dimensions must be positive");
  if (c->d_conv < 2 || c->d_conv > 8) return fail(M2_ERR_SHAPE, "d_conv %d outside [2, 8]", c->d_conv);
  if (c->n_heads % c->n_groups)
    return fail(M2_ERR_SHAPE, "n_heads %d is not a multiple of n_groups %d", c->n_heads, c->n_groups);
  if (c->d_model % 16) return fail(M2_ERR_SHAPE, "d_model %d is not a multiple of 16", c->d_model);
  const long d_inner = (long)c->n_heads * c->head_dim;
  if (d_inner % 16) return fail(M2_ERR_SHAPE, "d_inner %ld is not a multiple of 16", d_inner);
  if (c->head_dim % 4) return fail(M2_ERR_SHAPE, "head_dim %d is not a multiple of 4", c->head_dim);
  const int N = c->d_state;
  if (N < 4 || N > 256 || (N & (N - 1)))
    return fail(M2_ERR_SHAPE, "d_state %d must be a power of two in [4, 256]", N);
  const long ng = c->norm_group > 0 ? c->norm_group : d_inner / c->n_groups;
  if (c->norm_group < 0 || ng <= 0 || d_inner % ng)
    return fail(M2_ERR_SHAPE, "norm_group %d does not divide d_inner %ld", c->norm_group, d_inner);
  if (ng % 4) return fail(M2_ERR_SHAPE, "channels per RMS group (%ld) must be a multiple of 4", ng);
  if (!(c->norm_eps >= 0.0f)) return fail(M2_ERR_SHAPE, "norm_eps must be >= 0");
  if (d_inner / ng > 4096) return fail(M2_ERR_UNSUPPORTED, "more than 4096 RMS groups");
  if (c->wtype != M2_W_F32 && c->wtype != M2_W_BF16 && c->wtype != M2_W_INT8G && c->wtype != M2_W_INT4G &&
      c->wtype != M2_W_INT3G)
    return fail(M2_ERR_DTYPE, "unknown wtype %d", c->wtype);
  if (c->wtype == M2_W_INT4G || c->wtype == M2_W_INT3G) {
    if (c->q_group < 32 || (c->q_group & (c->q_group - 1)))
      return fail(M2_ERR_SHAPE, "q_group %d must be a power of two >= 32", c->q_group);
    if (c->d_model % c->q_group || d_inner % c->q_group)
      return fail(M2_ERR_SHAPE, "q_group %d does not divide d_model %d and d_inner %ld", c->q_group,
                  c->d_model, d_inner);
  }
  if (c->wtype == M2_W_INT8G) {
    if (c->q_group < 16 || (c->q_group & (c->q_group - 1)))
      return fail(M2_ERR_SHAPE, "q_group %d must be a power of two >= 16", c->q_group);
    if (c->d_model % c->q_group || d_inner % c->q_group)
      return fail(M2_ERR_SHAPE, "q_group %d does not divide d_model %d and d_inner %ld", c->q_group,
                  c->d_model, d_inner);
  }
  const long conv_dim = d_inner + 2L * c->n_groups * N;
  const long d_in_proj = 2 * d_inner + 2L * c->n_groups * N + c->n_heads;
  if (d_in_proj > (1L << 30) / 1 || conv_dim > (1L << 28))
    return fail(M2_ERR_SHAPE, "layer too large");
  return M2_OK;
}

}  // namespace

extern "C" {

int m2_abi_version(void) { return M2_ABI_VERSION; }

const char *m2_last_error(void) { return g_err; }

size_t m2_panels_bytes(int32_t wtype, int32_t rows, int32_t K) {
  if (rows > (1 << 24) || K > (1 << 24)) return 0;
  return m2d::panels_bytes(wtype, rows, K);
}

int m2_pack_panels(int32_t wtype, const void *w, int32_t rows, int32_t K, void *out, void *stream) {
  if (wtype != M2_W_BF16 && wtype != M2_W_INT8G) return fail(M2_ERR_DTYPE, "panels: wtype must be bf16 or int8");
  if (rows <= 0 || K <= 0 || rows > (1 << 24) || K > (1 << 24))
    return fail(M2_ERR_SHAPE, "panels: rows and K must be in [1, 2^24]");
  if (!w || !out) return fail(M2_ERR_NULL, "panels: w and out must not be NULL");
  if (!aligned16(out)) return fail(M2_ERR_ALIGN, "panels: out must be 16-byte aligned");
  const hipError_t e = m2d::launch_pack_panels(wtype, w, rows, K, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(M2_ERR_HIP, "panel pack launch: %s", hipGetErrorString(e));
  return ok();
}

int m2_layer_create(const m2_config *cfg, const m2_weights *w, m2_layer *out) {
  if (!out) return fail(M2_ERR_NULL, "out is NULL");
  *out = nullptr;
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!w) return fail(M2_ERR_NULL, "weights struct is NULL");
  const void *req[] = {w->w_in, w->w_out, w->conv_w, w->conv_b, w->dt_bias, w->A_log, w->D, w->norm_w};
  const char *names[] = {"w_in", "w_out", "conv_w", "conv_b", "dt_bias", "A_log", "D", "norm_w"};
  for (int i = 0; i < 8; ++i)
    if (!req[i]) return fail(M2_ERR_NULL, "weight pointer %s is NULL", names[i]);
  const bool quantized = cfg->wtype == M2_W_INT8G || cfg->wtype == M2_W_INT4G || cfg->wtype == M2_W_INT3G;
  if (quantized && (!w->s_in || !w->s_out))
    return fail(M2_ERR_NULL, "quantized weights need s_in and s_out");
  if (!aligned16(w->w_in) || !aligned16(w->w_out))
    return fail(M2_ERR_ALIGN, "w_in and w_out must be 16-byte aligned");
  if (quantized && (!aligned16(w->s_in) || !aligned16(w->s_out)))
    return fail(M2_ERR_ALIGN, "s_in and s_out must be 16-byte aligned");
  for (int i = 2; i < 8; ++i)
    if (!aligned16(req[i])) return fail(M2_ERR_ALIGN, "%s must be 16-byte aligned", names[i]);
  if ((w->w_in_panels || w->w_out_panels) && cfg->wtype != M2_W_BF16 && cfg->wtype != M2_W_INT8G)
    return fail(M2_ERR_DTYPE, "panel copies exist for bf16 and int8 weights only");
  if (!aligned16(w->w_in_panels) || !aligned16(w->w_out_panels))
    return fail(M2_ERR_ALIGN, "w_in_panels and w_out_panels must be 16-byte aligned");

  m2_layer_s *L = new (std::nothrow) m2_layer_s();
  if (!L) return fail(M2_ERR_SHAPE, "out of host memory");
  L->cfg = *cfg;
  L->w = *w;
  L->d_inner = cfg->n_heads * cfg->head_dim;
  L->conv_dim = L->d_inner + 2 * cfg->n_groups * cfg->d_state;
  L->d_in_proj = 2 * L->d_inner + 2 * cfg->n_groups * cfg->d_state + cfg->n_heads;
  L->zx_stride = (L->d_in_proj + 3) & ~3;
  L->hpg = cfg->n_heads / cfg->n_groups;
  L->ng = cfg->norm_group > 0 ? cfg->norm_group : L->d_inner / cfg->n_groups;
  L->cfg.norm_group = L->ng;
  L->n_norm = L->d_inner / L->ng;
  // SSD workgroup row range: the largest multiple of 4 not above 32 that divides
  // gcd(head_dim, ng), so a workgroup's channels never straddle an RMS group and its
  // conv works on whole float4s (head_dim and ng are multiples of 4).
  const int gg = gcd(cfg->head_dim, L->ng);
  int pr = 4;
  for (int d = 4; d <= 32 && d <= gg; d += 4)
    if (gg % d == 0) pr = d;
  L->prange = pr;
  L->psplit = cfg->head_dim / pr;
  L->n_partials = L->d_inner / pr;
  *out = L;
  return ok();
}

void m2_layer_destroy(m2_layer layer) { delete layer; }

int m2_state_sizes(const m2_config *cfg, int32_t n_slots, size_t *ssm_bytes, size_t *conv_bytes) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (n_slots <= 0) return fail(M2_ERR_SHAPE, "n_slots must be positive");
  if (!ssm_bytes || !conv_bytes) return fail(M2_ERR_NULL, "size outputs are NULL");
  const size_t d_inner = (size_t)cfg->n_heads * cfg->head_dim;
  const size_t conv_dim = d_inner + 2 * (size_t)cfg->n_groups * cfg->d_state;
  *ssm_bytes = (size_t)n_slots * d_inner * cfg->d_state * sizeof(float);
  *conv_bytes = (size_t)n_slots * (cfg->d_conv - 1) * conv_dim * sizeof(float);
  return ok();
}

int m2_state_create(m2_layer layer, int32_t n_slots, float *ssm, float *conv, m2_state *out) {
  if (!out) return fail(M2_ERR_NULL, "out is NULL");
  *out = nullptr;
  if (!layer) return fail(M2_ERR_NULL, "layer is NULL");
  if (n_slots <= 0) return fail(M2_ERR_SHAPE, "n_slots must be positive");
  if (!ssm || !conv) return fail(M2_ERR_NULL, "ssm and conv buffers are required");
  if (!aligned16(ssm) || !aligned16(conv)) return fail(M2_ERR_ALIGN, "state buffers must be 16-byte aligned");
  m2_state_s *S = new (std::nothrow) m2_state_s();
  if (!S) return fail(M2_ERR_SHAPE, "out of host memory");
  S->layer = layer;
  S->n_slots = n_slots;
  S->ssm = ssm;
  S->conv = conv;
  *out = S;
  return ok();
}

void m2_state_destroy(m2_state st) { delete st; }

int m2_state_zero(m2_state st, const int32_t *slot_ids, int32_t n, void *stream) {
  if (!st) return fail(M2_ERR_NULL, "state is NULL");
  if (slot_ids && n <= 0) return fail(M2_ERR_SHAPE, "n must be positive");
  if (slot_ids && n > st->n_slots) return fail(M2_ERR_SLOT, "n %d exceeds n_slots %d", n, st->n_slots);
  hipError_t e = m2d::launch_state_zero(*st, slot_ids, slot_ids ? n : st->n_slots,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(M2_ERR_HIP, "state zero launch: %s", hipGetErrorString(e));
  return ok();
}

size_t m2_step_workspace(m2_layer layer, int32_t batch) {
  if (!layer || batch <= 0) return 0;
  return m2d::step_ws_layout(*layer, batch, nullptr).bytes;
}

// A state made for one layer serves another of the same state shape.
static bool same_state_shape(const m2_config &a, const m2_config &b) {
  return a.n_heads == b.n_heads && a.head_dim == b.head_dim && a.d_state == b.d_state && a.n_groups == b.n_groups &&
         a.d_conv == b.d_conv;
}

// check_only: every argument check except the workspace's, then return without launching.
static int step_impl(m2_layer layer, m2_state st, const float *x, float *y, int32_t batch,
                     const int32_t *slot_ids, int32_t flags, void *ws, size_t ws_bytes, void *stream,
                     void *const *events, bool check_only = false) {
  if (!layer || !st) return fail(M2_ERR_NULL, "layer or state is NULL");
  if (st->layer != layer && !same_state_shape(st->layer->cfg, layer->cfg))
    return fail(M2_ERR_SHAPE, "state was created for a layer of another shape");
  if (!x || !y) return fail(M2_ERR_NULL, "x and y are required");
  if (!aligned16(x) || !aligned16(y)) return fail(M2_ERR_ALIGN, "x and y must be 16-byte aligned");
  if (batch <= 0) return fail(M2_ERR_SHAPE, "batch must be positive");
  if (batch > st->n_slots) return fail(M2_ERR_SLOT, "batch %d exceeds n_slots %d", batch, st->n_slots);
  if (flags & ~(M2_RESIDUAL | M2_PERSISTENT)) return fail(M2_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
  if (!(flags & M2_RESIDUAL) && x == y)
    return fail(M2_ERR_SHAPE, "y may alias x only with M2_RESIDUAL");
  if (check_only) return M2_OK;
  const size_t need = m2_step_workspace(layer, batch);
  if (!ws || ws_bytes < need)
    return fail(M2_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
  if (!aligned16(ws)) return fail(M2_ERR_ALIGN, "workspace must be 16-byte aligned");
  m2d::StepWs W = m2d::step_ws_layout(*layer, batch, ws);
  hipError_t e = m2d::launch_step(*layer, *st, x, y, batch, slot_ids, flags, W,
                                  static_cast<hipStream_t>(stream),
                                  reinterpret_cast<hipEvent_t const *>(events));
  if (e != hipSuccess) return fail(M2_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

int m2_step(m2_layer layer, m2_state st, const float *x, float *y, int32_t batch,
            const int32_t *slot_ids, int32_t flags, void *ws, size_t ws_bytes, void *stream) {
  return step_impl(layer, st, x, y, batch, slot_ids, flags, ws, ws_bytes, stream, nullptr);
}

int m2_step_timed(m2_layer layer, m2_state st, const float *x, float *y, int32_t batch,
                  const int32_t *slot_ids, int32_t flags, void *ws, size_t ws_bytes, void *stream,
                  void *const *events) {
  return step_impl(layer, st, x, y, batch, slot_ids, flags, ws, ws_bytes, stream, events);
}

// m2_step_noalloc's workspace: one array per GPU, in the code object's zero-filled device
// memory, alive until the process ends. Host code never names it in a launch or a copy:
// the array's name is a host-side stand-in, so every use goes through the device address
// hipGetSymbolAddress returns, looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[M2_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

int scratch_for_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(M2_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(M2_ERR_UNSUPPORTED, "device %d above %d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(M2_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return M2_OK;
}
}  // namespace

size_t m2_noalloc_scratch_bytes(void) { return M2_NOALLOC_SCRATCH_BYTES; }

int m2_step_noalloc(m2_layer layer, m2_state st, const float *x, float *y, int32_t batch,
                    const int32_t *slot_ids, int32_t flags, void *stream) {
  if (!layer || !st) return fail(M2_ERR_NULL, "layer or state is NULL");
  if (batch <= 0) return fail(M2_ERR_SHAPE, "batch must be positive");
  const size_t need = m2_step_workspace(layer, batch);
  if (need > M2_NOALLOC_SCRATCH_BYTES)
    return fail(M2_ERR_WORKSPACE, "a step of %d sessions needs %zu bytes of scratch; the static scratch holds %zu",
                batch, need, (size_t)M2_NOALLOC_SCRATCH_BYTES);
  // the host checks that need no device run first, so that a rejected call makes no HIP call
  int rc = step_impl(layer, st, x, y, batch, slot_ids, flags, nullptr, 0, stream, nullptr, /*check_only=*/true);
  if (rc != M2_OK) return rc;
  void *ws = nullptr;
  rc = scratch_for_current_device(&ws);
  if (rc != M2_OK) return rc;
  return step_impl(layer, st, x, y, batch, slot_ids, flags, ws, M2_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int m2_step_plan(m2_layer layer, int32_t batch) {
  if (!layer || batch <= 0) return -1;
  return m2d::step_plan(*layer, batch);
}

int m2_step_plan_flags(m2_layer layer, int32_t batch, int32_t flags) {
  if (!layer || batch <= 0 || (flags & ~(M2_RESIDUAL | M2_PERSISTENT))) return -1;
  return m2d::step_plan(*layer, batch, flags);
}

static int check_head(const m2_head_config *c) {
  if (!c) return fail(M2_ERR_NULL, "head config is NULL");
  if (c->wtype != M2_W_F32 && c->wtype != M2_W_BF16 && c->wtype != M2_W_INT8G && c->wtype != M2_W_INT4G &&
      c->wtype != M2_W_INT3G)
    return fail(M2_ERR_DTYPE, "unknown wtype %d", c->wtype);
  if (c->vocab < 1 || c->vocab > (1 << 24)) return fail(M2_ERR_SHAPE, "vocab %d outside [1, 2^24]", c->vocab);
  const int epc = c->wtype == M2_W_F32 ? 4 : c->wtype == M2_W_BF16 ? 8 : c->wtype == M2_W_INT8G ? 16 : 32;
  if (c->d_model <= 0 || c->d_model % epc)
    return fail(M2_ERR_SHAPE, "d_model %d is not a positive multiple of %d", c->d_model, epc);
  if (c->d_model > 8192) return fail(M2_ERR_UNSUPPORTED, "d_model %d above 8192", c->d_model);
  if (c->wtype == M2_W_INT8G || c->wtype == M2_W_INT4G || c->wtype == M2_W_INT3G) {
    const int qmin = c->wtype == M2_W_INT8G ? 16 : 32;
    if (c->q_group < qmin || (c->q_group & (c->q_group - 1)) || c->d_model % c->q_group)
      return fail(M2_ERR_SHAPE, "q_group %d must be a power of two >= %d dividing d_model %d", c->q_group, qmin,
                  c->d_model);
  }
  return M2_OK;
}

size_t m2_head_workspace(const m2_head_config *cfg, int32_t batch) {
  if (check_head(cfg) || batch <= 0) return 0;
  return m2d::head_ws_bytes(cfg->vocab);
}

static int head_impl(const m2_head_config *cfg, const void *w, const void *scales, const float *h, int32_t batch,
                     int32_t *token, float *logits, void *ws, size_t ws_bytes, void *stream, void *const *events) {
  int rc = check_head(cfg);
  if (rc) return rc;
  if (!w || !h || !token) return fail(M2_ERR_NULL, "w, h and token are required");
  const bool quantized = cfg->wtype == M2_W_INT8G || cfg->wtype == M2_W_INT4G || cfg->wtype == M2_W_INT3G;
  if (quantized && !scales) return fail(M2_ERR_NULL, "quantized heads need scales");
  if (!aligned16(w) || !aligned16(h) || (quantized && !aligned16(scales)))
    return fail(M2_ERR_ALIGN, "w, h and scales must be 16-byte aligned");
  if (batch <= 0) return fail(M2_ERR_SHAPE, "batch must be positive");
  const size_t need = m2d::head_ws_bytes(cfg->vocab);
  if (!ws || ws_bytes < need)
    return fail(M2_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
  if (!aligned16(ws)) return fail(M2_ERR_ALIGN, "workspace must be 16-byte aligned");
  hipError_t e = m2d::launch_head(*cfg, w, scales, h, batch, token, logits, ws, static_cast<hipStream_t>(stream),
                                  reinterpret_cast<hipEvent_t const *>(events));
  if (e != hipSuccess) return fail(M2_ERR_HIP, "head launch: %s", hipGetErrorString(e));
  return ok();
}

int m2_head_argmax(const m2_head_config *cfg, const void *w, const void *scales, const float *h, int32_t batch,
                   int32_t *token, float *logits, void *ws, size_t ws_bytes, void *stream) {
  return head_impl(cfg, w, scales, h, batch, token, logits, ws, ws_bytes, stream, nullptr);
}

int m2_head_argmax_timed(const m2_head_config *cfg, const void *w, const void *scales, const float *h,
                         int32_t batch, int32_t *token, float *logits, void *ws, size_t ws_bytes, void *stream,
                         void *const *events) {
  if (batch > 4) return fail(M2_ERR_UNSUPPORTED, "timed head calls take at most 4 sessions (one launch pair)");
  return head_impl(cfg, w, scales, h, batch, token, logits, ws, ws_bytes, stream, events);
}

static int check_attn(const m2_attn_config *c) {
  if (!c) return fail(M2_ERR_NULL, "attention config is NULL");
  if (c->wtype != M2_W_F32 && c->wtype != M2_W_BF16 && c->wtype != M2_W_INT8G && c->wtype != M2_W_INT4G &&
      c->wtype != M2_W_INT3G)
    return fail(M2_ERR_DTYPE, "unknown wtype %d", c->wtype);
  if (c->n_q < 1 || c->n_kv < 1 || c->n_q % c->n_kv)
    return fail(M2_ERR_SHAPE, "n_q %d must be a positive multiple of n_kv %d", c->n_q, c->n_kv);
  if (c->n_q / c->n_kv > 8) return fail(M2_ERR_UNSUPPORTED, "more than 8 query heads per key/value head");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(M2_ERR_UNSUPPORTED, "head_dim %d: 64 and 128 are supported", c->head_dim);
  if (c->max_len < 1 || c->max_len > 65536) return fail(M2_ERR_SHAPE, "max_len %d outside [1, 65536]", c->max_len);
  const int epc = c->wtype == M2_W_F32 ? 4 : c->wtype == M2_W_BF16 ? 8 : c->wtype == M2_W_INT8G ? 16 : 32;
  const int o_dim = c->n_q * c->head_dim;
  if (c->d_model <= 0 || c->d_model % epc || o_dim % epc)
    return fail(M2_ERR_SHAPE, "d_model %d and n_q*head_dim %d must be positive multiples of %d", c->d_model, o_dim,
                epc);
  if (c->wtype == M2_W_INT8G || c->wtype == M2_W_INT4G || c->wtype == M2_W_INT3G) {
    const int qmin = c->wtype == M2_W_INT8G ? 16 : 32;
    if (c->q_group < qmin || (c->q_group & (c->q_group - 1)) || c->d_model % c->q_group || o_dim % c->q_group)
      return fail(M2_ERR_SHAPE, "q_group %d must be a power of two >= %d dividing d_model and n_q*head_dim",
                  c->q_group, qmin);
  }
  return M2_OK;
}

int m2_attn_create(const m2_attn_config *cfg, const m2_attn_weights *w, m2_attn *out) {
  if (!out) return fail(M2_ERR_NULL, "out is NULL");
  *out = nullptr;
  int rc = check_attn(cfg);
  if (rc) return rc;
  if (!w || !w->w_qkv || !w->w_o) return fail(M2_ERR_NULL, "w_qkv and w_o are required");
  const bool quantized = cfg->wtype == M2_W_INT8G || cfg->wtype == M2_W_INT4G || cfg->wtype == M2_W_INT3G;
  if (quantized && (!w->s_qkv || !w->s_o)) return fail(M2_ERR_NULL, "quantized weights need s_qkv and s_o");
  if (!aligned16(w->w_qkv) || !aligned16(w->w_o) || (quantized && (!aligned16(w->s_qkv) || !aligned16(w->s_o))))
    return fail(M2_ERR_ALIGN, "attention weights and scales must be 16-byte aligned");
  m2_attn_s *A = new (std::nothrow) m2_attn_s();
  if (!A) return fail(M2_ERR_SHAPE, "out of host memory");
  A->cfg = *cfg;
  A->w = *w;
  A->qkv_rows = (cfg->n_q + 2 * cfg->n_kv) * cfg->head_dim;
  A->o_dim = cfg->n_q * cfg->head_dim;
  A->nsplit = m2d::attn_nsplit(cfg->max_len);
  *out = A;
  return ok();
}

void m2_attn_destroy(m2_attn a) { delete a; }

size_t m2_attn_workspace(m2_attn a, int32_t batch) {
  if (!a || batch <= 0) return 0;
  return m2d::attn_ws_bytes(*a, batch);
}

static int attn_impl(m2_attn a, void *k_cache, void *v_cache, int32_t *pos, int32_t n_slots, const float *x,
                     float *y, int32_t batch, const int32_t *slot_ids, int32_t flags, void *ws, size_t ws_bytes,
                     void *stream, void *const *events) {
  if (!a || !k_cache || !v_cache || !pos || !x || !y) return fail(M2_ERR_NULL, "a required pointer is NULL");
  if (batch <= 0) return fail(M2_ERR_SHAPE, "batch must be positive");
  if (n_slots < 1) return fail(M2_ERR_SLOT, "n_slots must be positive");
  if (!slot_ids && batch > n_slots) return fail(M2_ERR_SLOT, "batch %d exceeds n_slots %d", batch, n_slots);
  if (flags & ~M2_RESIDUAL) return fail(M2_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(x) || !aligned16(y) ||
      (reinterpret_cast<uintptr_t>(pos) & 3u))
    return fail(M2_ERR_ALIGN, "caches, x and y must be 16-byte aligned, pos 4-byte aligned");
  const size_t need = m2d::attn_ws_bytes(*a, batch);
  if (!ws || ws_bytes < need)
    return fail(M2_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
  if (!aligned16(ws)) return fail(M2_ERR_ALIGN, "workspace must be 16-byte aligned");
  hipError_t e = m2d::launch_attn_step(*a, static_cast<uint16_t *>(k_cache), static_cast<uint16_t *>(v_cache), pos,
                                       n_slots, x, y, batch, slot_ids, flags, ws, static_cast<hipStream_t>(stream),
                                       reinterpret_cast<hipEvent_t const *>(events));
  if (e != hipSuccess) return fail(M2_ERR_HIP, "attention step launch: %s", hipGetErrorString(e));
  return ok();
}

int m2_attn_step(m2_attn a, void *k_cache, void *v_cache, int32_t *pos, int32_t n_slots, const float *x, float *y,
                 int32_t batch, const int32_t *slot_ids, int32_t flags, void *ws, size_t ws_bytes, void *stream) {
  return attn_impl(a, k_cache, v_cache, pos, n_slots, x, y, batch, slot_ids, flags, ws, ws_bytes, stream, nullptr);
}

int m2_attn_step_timed(m2_attn a, void *k_cache, void *v_cache, int32_t *pos, int32_t n_slots, const float *x,
                       float *y, int32_t batch, const int32_t *slot_ids, int32_t flags, void *ws, size_t ws_bytes,
                       void *stream, void *const *events) {
  return attn_impl(a, k_cache, v_cache, pos, n_slots, x, y, batch, slot_ids, flags, ws, ws_bytes, stream, events);
}

struct m2_stack_s {
  std::vector<m2_stack_layer> layers;
  int n_slots;
  int d_model;
  void *dtab = nullptr;     // the persistent kernel's layer table, on the device current at create
  int dev = -1;             // that device
  size_t area = 0;          // bytes of the persistent path's workspace area (a multiple of 256)
  ~m2_stack_s() {
    if (dtab) (void)hipFree(dtab);
  }
};

int m2_stack_create(const m2_stack_layer *layers, int32_t n_layers, int32_t n_slots, m2_stack *out) {
  if (!out) return fail(M2_ERR_NULL, "out is NULL");
  *out = nullptr;
  if (!layers || n_layers < 1) return fail(M2_ERR_SHAPE, "a stack needs at least one layer");
  if (n_slots < 1) return fail(M2_ERR_SLOT, "n_slots must be positive");
  int d_model = -1;
  for (int i = 0; i < n_layers; ++i) {
    const m2_stack_layer &l = layers[i];
    if (!l.layer) return fail(M2_ERR_NULL, "layer %d is NULL", i);
    int dm;
    // every check a layer's step would make on its own arguments is made here, so that
    // m2_stack_step cannot fail part-way through the chain (after earlier layers ran)
    if (l.kind == M2_LAYER_MIXER) {
      const m2_state st = static_cast<m2_state>(l.state);
      if (!st) return fail(M2_ERR_NULL, "mixer layer %d has no state", i);
      if (st->n_slots < n_slots) return fail(M2_ERR_SLOT, "mixer layer %d: state of %d slots", i, st->n_slots);
      const m2_layer ml = static_cast<m2_layer>(l.layer);
      if (!same_state_shape(st->layer->cfg, ml->cfg))
        return fail(M2_ERR_SHAPE, "mixer layer %d: state was created for a layer of another shape", i);
      dm = ml->cfg.d_model;
    } else if (l.kind == M2_LAYER_ATTN) {
      if (!l.k_cache || !l.v_cache || !l.pos) return fail(M2_ERR_NULL, "attention layer %d needs caches and pos", i);
      if (!aligned16(l.k_cache) || !aligned16(l.v_cache) || (reinterpret_cast<uintptr_t>(l.pos) & 3u))
        return fail(M2_ERR_ALIGN, "attention layer %d: caches must be 16-byte aligned, pos 4-byte aligned", i);
      dm = static_cast<m2_attn>(l.layer)->cfg.d_model;
    } else {
      return fail(M2_ERR_SHAPE, "layer %d: unknown kind %d", i, l.kind);
    }
    if (d_model >= 0 && dm != d_model) return fail(M2_ERR_SHAPE, "layer %d: d_model %d, not %d", i, dm, d_model);
    d_model = dm;
  }
  m2_stack_s *S = new (std::nothrow) m2_stack_s();
  if (!S) return fail(M2_ERR_SHAPE, "out of host memory");
  S->layers.assign(layers, layers + n_layers);
  S->n_slots = n_slots;
  S->d_model = d_model;
  // the persistent path's area (barrier words, then each mixer's buffers) and its layer
  // table, which goes to the current device when there is one (without one, the persistent
  // path never applies and the table is not made)
  const size_t rb = m2d::stack_rec_bytes();
  std::vector<unsigned char> tab(rb * (size_t)n_layers, 0);
  size_t off = m2d::stack_area_head();
  for (int i = 0; i < n_layers; ++i) {
    if (layers[i].kind != M2_LAYER_MIXER) continue;
    const m2_layer ml = static_cast<m2_layer>(layers[i].layer);
    m2d::stack_rec_fill(*ml, *static_cast<m2_state>(layers[i].state), off, tab.data() + rb * (size_t)i);
    off += m2d::stack_area_layer_bytes(*ml);
  }
  S->area = (off + 255) & ~(size_t)255;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    hipError_t e = hipGetDevice(&S->dev);
    if (e == hipSuccess) e = hipMalloc(&S->dtab, tab.size());
    if (e == hipSuccess) e = hipMemcpy(S->dtab, tab.data(), tab.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      delete S;
      return fail(M2_ERR_HIP, "stack layer table: %s", hipGetErrorString(e));
    }
  } else {
    (void)hipGetLastError();
  }
  *out = S;
  return ok();
}

void m2_stack_destroy(m2_stack s) { delete s; }

size_t m2_stack_workspace(m2_stack s, int32_t batch) {
  if (!s || batch <= 0) return 0;
  size_t need = 0;
  for (const m2_stack_layer &l : s->layers) {
    const size_t n = l.kind == M2_LAYER_MIXER ? m2_step_workspace(static_cast<m2_layer>(l.layer), batch)
                                              : m2_attn_workspace(static_cast<m2_attn>(l.layer), batch);
    if (n == 0) return 0;
    need = std::max(need, n);
  }
  return need;
}

size_t m2_stack_workspace_flags(m2_stack s, int32_t batch, int32_t flags) {
  if (!s || batch <= 0 || (flags & ~M2_PERSISTENT)) return 0;
  const size_t base = m2_stack_workspace(s, batch);
  if (base == 0) return 0;
  return (flags & M2_PERSISTENT) ? s->area + base : base;
}

}  // extern "C"

namespace {

// The runs of consecutive mixer layers a step with these flags takes in one persistent
// launch each: [first, end) pairs, with the run's dynamic LDS bytes and grid.
struct StackRun {
  int l0, l1;
  size_t lds;
  int grid;
};

std::vector<StackRun> stack_runs(const m2_stack_s &s, int batch, int flags) {
  std::vector<StackRun> runs;
  if (!(flags & M2_PERSISTENT) || batch != 1 || !s.dtab) return runs;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != s.dev) return runs;   // the table is on s.dev
  const int n = (int)s.layers.size();
  for (int i = 0; i < n;) {
    if (s.layers[i].kind != M2_LAYER_MIXER) {
      ++i;
      continue;
    }
    int j = i;
    size_t lds = 0;
    while (j < n && s.layers[j].kind == M2_LAYER_MIXER) {
      const m2_layer_s &L = *static_cast<m2_layer>(s.layers[j].layer);
      lds = std::max(lds, m2d::stack_lds_bytes(L));
      ++j;
    }
    const int grid = m2d::stack_grid(lds);
    bool fits = grid > 0;
    for (int k = i; k < j && fits; ++k) {
      const m2_layer_s &L = *static_cast<m2_layer>(s.layers[k].layer);
      fits = L.cfg.wtype == M2_W_BF16 && m2d::stack_fits(L, grid);
    }
    if (fits) runs.push_back(StackRun{i, j, lds, grid});
    i = j;
  }
  return runs;
}

int stack_step_impl(m2_stack s, const float *x, float *y, int32_t batch, const int32_t *slot_ids, int32_t flags,
                    void *ws, size_t ws_bytes, void *stream) {
  if (!s || !x || !y) return fail(M2_ERR_NULL, "stack, x and y are required");
  if (batch <= 0) return fail(M2_ERR_SHAPE, "batch must be positive");
  if (batch > s->n_slots) return fail(M2_ERR_SLOT, "batch %d exceeds n_slots %d", batch, s->n_slots);
  if (flags & ~M2_PERSISTENT) return fail(M2_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
  if (!aligned16(x) || !aligned16(y)) return fail(M2_ERR_ALIGN, "x and y must be 16-byte aligned");
  const size_t need = m2_stack_workspace_flags(s, batch, flags);
  if (!ws || ws_bytes < need)
    return fail(M2_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
  if (!aligned16(ws)) return fail(M2_ERR_ALIGN, "workspace must be 16-byte aligned");
  // with M2_PERSISTENT the persistent area comes first; the layers' own workspace after it
  const size_t skip = (flags & M2_PERSISTENT) ? s->area : 0;
  void *lws = static_cast<char *>(ws) + skip;
  const size_t lws_bytes = ws_bytes - skip;
  const std::vector<StackRun> runs = stack_runs(*s, batch, flags);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (x != y) {
    hipError_t e = hipMemcpyAsync(y, x, sizeof(float) * (size_t)batch * s->d_model, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return fail(M2_ERR_HIP, "stack input copy: %s", hipGetErrorString(e));
  }
  size_t r = 0;
  for (int i = 0; i < (int)s->layers.size();) {
    if (r < runs.size() && runs[r].l0 == i) {
      const StackRun &R = runs[r++];
      hipError_t e = m2d::launch_stack_run(s->dtab, R.l0, R.l1, R.lds, ws, y, slot_ids, s->n_slots, R.grid, st);
      if (e != hipSuccess) return fail(M2_ERR_HIP, "persistent stack launch: %s", hipGetErrorString(e));
      i = R.l1;
      continue;
    }
    const m2_stack_layer &l = s->layers[i++];
    const int rc = l.kind == M2_LAYER_MIXER
                       ? step_impl(static_cast<m2_layer>(l.layer), static_cast<m2_state>(l.state), y, y, batch,
                                   slot_ids, M2_RESIDUAL, lws, lws_bytes, stream, nullptr)
                       : attn_impl(static_cast<m2_attn>(l.layer), l.k_cache, l.v_cache, l.pos, s->n_slots, y, y,
                                   batch, slot_ids, M2_RESIDUAL, lws, lws_bytes, stream, nullptr);
    if (rc != M2_OK) return rc;
  }
  return ok();
}

}  // namespace

extern "C" {

int m2_stack_step(m2_stack s, const float *x, float *y, int32_t batch, const int32_t *slot_ids, void *ws,
                  size_t ws_bytes, void *stream) {
  return stack_step_impl(s, x, y, batch, slot_ids, 0, ws, ws_bytes, stream);
}

int m2_stack_step_flags(m2_stack s, const float *x, float *y, int32_t batch, const int32_t *slot_ids, int32_t flags,
                        void *ws, size_t ws_bytes, void *stream) {
  return stack_step_impl(s, x, y, batch, slot_ids, flags, ws, ws_bytes, stream);
}

int m2_stack_persistent_runs(m2_stack s, int32_t batch, int32_t flags) {
  if (!s || batch <= 0 || (flags & ~M2_PERSISTENT)) return -1;
  return (int)stack_runs(*s, batch, flags).size();
}

size_t m2_prefill_workspace(m2_layer layer, int32_t batch, int32_t seqlen, int32_t chunk) {
  if (!layer || batch <= 0 || seqlen <= 0 || chunk < 16 || chunk > 256 || chunk % 16) return 0;
  return m2d::prefill_ws_bytes(*layer, batch, seqlen, chunk);
}

int m2_prefill(m2_layer layer, m2_state st, const float *x, float *y, int32_t batch, int32_t seqlen,
               int32_t chunk, const int32_t *slot_ids, int32_t flags, void *ws, size_t ws_bytes,
               void *stream) {
  if (!layer || !st) return fail(M2_ERR_NULL, "layer or state is NULL");
  if (!x || !y) return fail(M2_ERR_NULL, "x and y are required");
  if (!aligned16(x) || !aligned16(y)) return fail(M2_ERR_ALIGN, "x and y must be 16-byte aligned");
  if (batch <= 0 || seqlen <= 0) return fail(M2_ERR_SHAPE, "batch and seqlen must be positive");
  if (chunk < 16 || chunk > 256 || chunk % 16)
    return fail(M2_ERR_SHAPE, "chunk %d must be a multiple of 16 in [16, 256]", chunk);
  if (batch > st->n_slots) return fail(M2_ERR_SLOT, "batch %d exceeds n_slots %d", batch, st->n_slots);
  if (flags & ~M2_RESIDUAL) return fail(M2_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
  if (!(flags & M2_RESIDUAL) && x == y)
    return fail(M2_ERR_SHAPE, "y may alias x only with M2_RESIDUAL");
  if ((long)batch * seqlen > (1L << 24)) return fail(M2_ERR_SHAPE, "batch * seqlen too large");
  const size_t need = m2_prefill_workspace(layer, batch, seqlen, chunk);
  if (need == 0) return fail(M2_ERR_UNSUPPORTED, "prefill is not available for this layer");
  if (!ws || ws_bytes < need)
    return fail(M2_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
  if (!aligned16(ws)) return fail(M2_ERR_ALIGN, "workspace must be 16-byte aligned");
  hipError_t e = m2d::launch_prefill(*layer, *st, x, y, batch, seqlen, chunk, slot_ids, flags, ws,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(M2_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
