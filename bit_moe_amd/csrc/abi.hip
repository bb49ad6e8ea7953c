// C ABI of libbitmoe: argument validation, workspace carving and kernel
// dispatch.  Every declaration and its contract is in include/bitmoe.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "bitmoe.h"
#include "internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(const char *where, hipError_t e) {
  return fail(BITMOE_EHIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

constexpr int MAX_DECODE_T = 8;

// ---- per-device scratch of moe_route_noalloc ---------------------------------
// The status record and the router logits of up to BITMOE_NOALLOC_MAX_T tokens
// of up to 1024 experts, laid out as the common region of a workspace.
constexpr size_t NOALLOC_SCRATCH_BYTES = 256 + size_t(BITMOE_NOALLOC_MAX_T) * 1024 * sizeof(float);
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};

}  // namespace

// One copy per device, held until the process ends.  In host code the name is
// only a stand-in for the symbol: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of the current device's scratch, looked up once per device
// (with that device current) and kept.
int scratch_address(const char *fn, void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(fn, e);
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
    return fail(BITMOE_EUNSUPPORTED, "%s: device %d outside the %d devices with scratch slots", fn, dev,
                NOALLOC_MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(fn, e);
    if (!ptr || !aligned(ptr, 256)) return fail(BITMOE_EHIP, "%s: scratch address %p unusable", fn, ptr);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return BITMOE_OK;
}

int check_layer(const char *fn, const bitmoe_layer *L) {
  if (!L) return fail(BITMOE_EINVAL, "%s: layer is NULL", fn);
  if (L->wfmt != BITMOE_WFMT_Q2SB)
    return fail(BITMOE_EUNSUPPORTED, "%s: routed weight format %d is not Q2SB (%d)", fn, L->wfmt, BITMOE_WFMT_Q2SB);
  if (L->layout_flags != BITMOE_LAYOUT_CANONICAL)
    return fail(BITMOE_EUNSUPPORTED, "%s: layout_flags %d: only the canonical block layout (0) is implemented", fn,
                L->layout_flags);
  if (L->shared_wfmt != BITMOE_WFMT_NONE && L->shared_wfmt != BITMOE_WFMT_Q8_0)
    return fail(BITMOE_EUNSUPPORTED, "%s: shared weight format %d is neither NONE nor Q8_0", fn, L->shared_wfmt);
  if (!pow2(L->d_model) || L->d_model < 256 || L->d_model > 4096)
    return fail(BITMOE_EUNSUPPORTED, "%s: d_model %d must be a power of two in [256, 4096]", fn, L->d_model);
  if (!pow2(L->d_ff) || L->d_ff < 128 || L->d_ff > 4096)
    return fail(BITMOE_EUNSUPPORTED, "%s: d_ff %d must be a power of two in [128, 4096]", fn, L->d_ff);
  if (L->n_experts < 1 || L->n_experts > 1024)
    return fail(BITMOE_EUNSUPPORTED, "%s: n_experts %d outside [1, 1024]", fn, L->n_experts);
  if (L->top_k < 1 || L->top_k > 8 || L->top_k > L->n_experts)
    return fail(BITMOE_EINVAL, "%s: top_k %d outside [1, min(8, n_experts=%d)]", fn, L->top_k, L->n_experts);
  const void *w[3] = {L->w_gate, L->w_up, L->w_down};
  const char *wn[3] = {"w_gate", "w_up", "w_down"};
  for (int i = 0; i < 3; ++i)
    if (!w[i] || !aligned(w[i], 16)) return fail(BITMOE_EINVAL, "%s: %s is NULL or not 16-byte aligned", fn, wn[i]);
  if (!L->w_router || !aligned(L->w_router, 16))
    return fail(BITMOE_EINVAL, "%s: w_router is NULL or not 16-byte aligned", fn);
  if (L->shared_wfmt == BITMOE_WFMT_Q8_0) {
    const void *s[3] = {L->ws_gate, L->ws_up, L->ws_down};
    const char *sn[3] = {"ws_gate", "ws_up", "ws_down"};
    for (int i = 0; i < 3; ++i)
      if (!s[i] || !aligned(s[i], 16)) return fail(BITMOE_EINVAL, "%s: %s is NULL or not 16-byte aligned", fn, sn[i]);
  }
  return BITMOE_OK;
}

int resolve_mode(int mode, int T) {
  if (mode == BITMOE_MODE_AUTO) return T <= MAX_DECODE_T ? BITMOE_MODE_DECODE : BITMOE_MODE_PREFILL;
  return mode;
}

// Workspace layout (each region 256-byte aligned):
//   [status record + counters: 256 B][router logits T*E f32][mode-specific]
struct Carve {
  size_t off = 0;
  char *base;
  explicit Carve(void *b) : base(static_cast<char *>(b)) {}
  void *take(size_t bytes) {
    void *p = base ? base + off : nullptr;
    off += up256(bytes);
    return p;
  }
};

struct DecodeWs {
  uint16_t *h, *hs, *h_lo, *hs_lo;
  float *y, *ys;
};

struct PrefillWs {
  bm::PlanBufs plan;
  int32_t *tile_off, *tile_off2;
  uint16_t *xs, *h, *hs, *h_lo, *hs_lo, *sw, *xsum;
  float *xtot;
  float *y, *ys;
};

// Common region: status record, router logits and, for T > MAX_DECODE_T, the
// router matrix's three bf16 parts (rewritten by every router call).
size_t carve_common(Carve &c, const bitmoe_layer *L, int T, int64_t **status, float **logits,
                    uint16_t **wsplit = nullptr) {
  void *st = c.take(256);
  void *lg = c.take(size_t(T) * L->n_experts * sizeof(float));
  void *sp = c.take(T > MAX_DECODE_T ? bm::router_split_bytes(L->n_experts, L->d_model) : 0);
  if (status) *status = static_cast<int64_t *>(st);
  if (logits) *logits = static_cast<float *>(lg);
  if (wsplit) *wsplit = T > MAX_DECODE_T ? static_cast<uint16_t *>(sp) : nullptr;
  return c.off;
}

void carve_decode(Carve &c, const bitmoe_layer *L, int T, DecodeWs *w) {
  const size_t P = size_t(T) * L->top_k;
  w->h = static_cast<uint16_t *>(c.take(P * L->d_ff * 2));
  w->hs = static_cast<uint16_t *>(c.take(size_t(T) * L->d_ff * 2));
  w->h_lo = static_cast<uint16_t *>(c.take(P * L->d_ff * 2));
  w->hs_lo = static_cast<uint16_t *>(c.take(size_t(T) * L->d_ff * 2));
  w->y = static_cast<float *>(c.take(P * L->d_model * 4));
  w->ys = static_cast<float *>(c.take(size_t(T) * L->d_model * 4));
}

// int8 numerics: h in float32 (the quantiser's input) instead of bf16 parts
void carve_decode_i8(Carve &c, const bitmoe_layer *L, int T, DecodeWs *w, float **hf, float **hsf) {
  const size_t P = size_t(T) * L->top_k;
  *hf = static_cast<float *>(c.take(P * L->d_ff * 4));
  *hsf = static_cast<float *>(c.take(size_t(T) * L->d_ff * 4));
  w->h = w->hs = w->h_lo = w->hs_lo = nullptr;
  w->y = static_cast<float *>(c.take(P * L->d_model * 4));
  w->ys = static_cast<float *>(c.take(size_t(T) * L->d_model * 4));
}

// Decode-path kernel arguments over the workspace carve (after the common region).
bm::FfnArgs decode_args(Carve &c, const bitmoe_layer *L, const void *x, int T, const int32_t *ids, const float *wts,
                        void *y, int y_dtype, int64_t *status, bool int8 = false) {
  DecodeWs w;
  float *hf = nullptr, *hsf = nullptr;
  if (int8) carve_decode_i8(c, L, T, &w, &hf, &hsf);
  else carve_decode(c, L, T, &w);
  const bool shared = L->shared_wfmt == BITMOE_WFMT_Q8_0;
  bm::FfnArgs a{};
  a.D = L->d_model;
  a.F = L->d_ff;
  a.E = L->n_experts;
  a.k = L->top_k;
  a.T = T;
  a.wg = static_cast<const uint8_t *>(L->w_gate);
  a.wu = static_cast<const uint8_t *>(L->w_up);
  a.wd = static_cast<const uint8_t *>(L->w_down);
  a.sg = shared ? static_cast<const uint8_t *>(L->ws_gate) : nullptr;
  a.su = shared ? static_cast<const uint8_t *>(L->ws_up) : nullptr;
  a.sd = shared ? static_cast<const uint8_t *>(L->ws_down) : nullptr;
  a.x = x;
  a.ids = ids;
  a.wts = wts;
  a.h = w.h;
  a.hs = w.hs;
  a.h_lo = w.h_lo;
  a.hs_lo = w.hs_lo;
  a.hf = hf;
  a.hsf = hsf;
  a.y = w.y;
  a.ys = w.ys;
  a.out = y;
  a.out_bf16 = y_dtype == BITMOE_BF16;
  a.status = status;
  return a;
}

void carve_prefill(Carve &c, const bitmoe_layer *L, int T, PrefillWs *w) {
  const int E = L->n_experts;
  const size_t P = size_t(T) * L->top_k;
  w->plan.counts = static_cast<int32_t *>(c.take(size_t(E) * 4));
  w->plan.offsets = static_cast<int32_t *>(c.take(size_t(E + 1) * 4));
  w->plan.perm = static_cast<int32_t *>(c.take(P * 4));
  w->plan.union_ids = static_cast<int32_t *>(c.take(size_t(E) * 4));
  w->plan.n_union = static_cast<int32_t *>(c.take(4));
  w->plan.chunk_counts = static_cast<int32_t *>(c.take(bm::plan_scratch_bytes(T, E)));
  w->tile_off = static_cast<int32_t *>(c.take(size_t(E + 1) * 4));
  w->tile_off2 = static_cast<int32_t *>(c.take(size_t(E + 1) * 4));
  w->plan.tile_off = w->tile_off;
  w->plan.tile_off2 = w->tile_off2;
  w->xs = static_cast<uint16_t *>(c.take(size_t(T) * L->d_model * 2));
  w->h = static_cast<uint16_t *>(c.take(P * L->d_ff * 2));
  w->hs = static_cast<uint16_t *>(c.take(size_t(T) * L->d_ff * 2));
  w->h_lo = static_cast<uint16_t *>(c.take(P * L->d_ff * 2));
  w->hs_lo = static_cast<uint16_t *>(c.take(size_t(T) * L->d_ff * 2));
  const bool shared = L->shared_wfmt == BITMOE_WFMT_Q8_0;
  // expanded shared expert: bf16 codes (3 matrices) + float scales (one per 32 weights)
  w->sw = static_cast<uint16_t *>(c.take(shared ? size_t(3) * L->d_ff * L->d_model * (2 + 4 / 32.0) : 0));
  w->y = static_cast<float *>(c.take(P * L->d_model * 4));
  w->ys = static_cast<float *>(c.take(size_t(T) * L->d_model * 4));
  // sub-block sums of the grouped GEMMs' activation rows: 32 bf16 per row and 256 columns
  w->xsum = static_cast<uint16_t *>(c.take(std::max(size_t(T) * L->d_model, P * L->d_ff) / 256 * 32 * 2));
  // their float32 super-block sums: one per row and 256 columns
  w->xtot = static_cast<float *>(c.take(std::max(size_t(T) * L->d_model, P * L->d_ff) / 256 * 4));
}

// int8 numerics on the prefill path: plan, quantised x and h with their
// scales and stored sums, h in float32, the shared expert's int8 codes
void carve_prefill_i8(Carve &c, const bitmoe_layer *L, int T, bm::PrefillI8Args *a) {
  const int E = L->n_experts, D = L->d_model, F = L->d_ff;
  const size_t P = size_t(T) * L->top_k;
  a->plan.counts = static_cast<int32_t *>(c.take(size_t(E) * 4));
  a->plan.offsets = static_cast<int32_t *>(c.take(size_t(E + 1) * 4));
  a->plan.perm = static_cast<int32_t *>(c.take(P * 4));
  a->plan.union_ids = static_cast<int32_t *>(c.take(size_t(E) * 4));
  a->plan.n_union = static_cast<int32_t *>(c.take(4));
  a->plan.chunk_counts = static_cast<int32_t *>(c.take(bm::plan_scratch_bytes(T, E)));
  a->tile_off = static_cast<int32_t *>(c.take(size_t(E + 1) * 4));
  a->tile_off2 = static_cast<int32_t *>(c.take(size_t(E + 1) * 4));
  a->plan.tile_off = a->tile_off;
  a->plan.tile_off2 = a->tile_off2;
  a->xq = static_cast<int8_t *>(c.take(size_t(T) * D));
  a->xd = static_cast<float *>(c.take(size_t(T) * D / 32 * 4));
  a->xs = static_cast<float *>(c.take(size_t(T) * D / 16 * 4));
  a->sums = static_cast<uint16_t *>(c.take(std::max(size_t(T) * D, P * F) / 256 * 32 * 2));
  a->hf = static_cast<float *>(c.take(P * F * 4));
  a->hq = static_cast<int8_t *>(c.take(P * F));
  a->hd = static_cast<float *>(c.take(P * F / 32 * 4));
  a->hs = static_cast<float *>(c.take(P * F / 16 * 4));
  const bool shared = L->shared_wfmt == BITMOE_WFMT_Q8_0;
  a->sw_i8 = static_cast<int8_t *>(c.take(shared ? size_t(3) * F * D : 0));
  a->sw_d = static_cast<float *>(c.take(shared ? size_t(3) * F * D / 32 * 4 : 0));
  a->hsf = static_cast<float *>(c.take(size_t(T) * F * 4));
  a->hsq = static_cast<int8_t *>(c.take(size_t(T) * F));
  a->hsd = static_cast<float *>(c.take(size_t(T) * F / 32 * 4));
  a->hss = static_cast<float *>(c.take(size_t(T) * F / 16 * 4));
  a->y = static_cast<float *>(c.take(P * D * 4));
  a->ys = static_cast<float *>(c.take(size_t(T) * D * 4));
}

size_t ws_bytes_for(const bitmoe_layer *L, int T, int mode) {
  Carve c(nullptr);
  carve_common(c, L, T, nullptr, nullptr);
  const int m = resolve_mode(mode, T);
  if (m == BITMOE_MODE_DECODE) {
    DecodeWs w;
    carve_decode(c, L, T, &w);
  } else if (m == BITMOE_MODE_DECODE_INT8) {
    DecodeWs w;
    float *hf, *hsf;
    carve_decode_i8(c, L, T, &w, &hf, &hsf);
  } else if (m == BITMOE_MODE_PREFILL_INT8) {
    bm::PrefillI8Args a{};
    carve_prefill_i8(c, L, T, &a);
  } else {
    PrefillWs w;
    carve_prefill(c, L, T, &w);
  }
  return c.off;
}

int check_ws(const char *fn, const bitmoe_layer *L, int T, int mode, const void *ws, size_t ws_bytes) {
  if (!ws || !aligned(ws, 256)) return fail(BITMOE_EINVAL, "%s: workspace is NULL or not 256-byte aligned", fn);
  const size_t need = ws_bytes_for(L, T, mode);
  if (ws_bytes < need)
    return fail(BITMOE_EWORKSPACE, "%s: workspace has %zu bytes, needs %zu for T=%d", fn, ws_bytes, need, T);
  return BITMOE_OK;
}

}  // namespace

extern "C" {

const char *bitmoe_strerror(int code) {
  switch (code) {
    case BITMOE_OK: return "BITMOE_OK: success";
    case BITMOE_EINVAL: return "BITMOE_EINVAL: invalid argument";
    case BITMOE_EUNSUPPORTED: return "BITMOE_EUNSUPPORTED: unsupported shape or format";
    case BITMOE_EWORKSPACE: return "BITMOE_EWORKSPACE: workspace too small";
    case BITMOE_EHIP: return "BITMOE_EHIP: HIP runtime error";
    case BITMOE_EDEVICE: return "BITMOE_EDEVICE: a device-side fault was recorded";
    default: return "unknown bitmoe status";
  }
}

const char *bitmoe_last_error(void) { return g_last_error; }

int bitmoe_workspace_size(const bitmoe_layer *L, int32_t T, int32_t mode, size_t *bytes) {
  int rc = check_layer("bitmoe_workspace_size", L);
  if (rc) return rc;
  if (!bytes) return fail(BITMOE_EINVAL, "bitmoe_workspace_size: bytes is NULL");
  if (T < 0) return fail(BITMOE_EINVAL, "bitmoe_workspace_size: T=%d is negative", T);
  if (mode < BITMOE_MODE_AUTO || mode > BITMOE_MODE_PREFILL_INT8)
    return fail(BITMOE_EINVAL, "bitmoe_workspace_size: unknown mode %d", mode);
  *bytes = ws_bytes_for(L, T, mode);
  return BITMOE_OK;
}

const int64_t *bitmoe_ws_status(const void *ws) { return static_cast<const int64_t *>(ws); }

int moe_route(const bitmoe_layer *L, const void *x, int32_t x_dtype, int32_t T, const float *logit_bias,
              int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, hipStream_t stream) {
  const char *fn = "moe_route";
  int rc = check_layer(fn, L);
  if (rc) return rc;
  if (T < 0) return fail(BITMOE_EINVAL, "%s: T=%d is negative", fn, T);
  if (x_dtype != BITMOE_F32 && x_dtype != BITMOE_BF16) return fail(BITMOE_EUNSUPPORTED, "%s: x_dtype %d", fn, x_dtype);
  if (T == 0) return BITMOE_OK;
  if (!x || !aligned(x, 16)) return fail(BITMOE_EINVAL, "%s: x is NULL or not 16-byte aligned", fn);
  if (!topk_ids || !topk_w || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return fail(BITMOE_EINVAL, "%s: topk_ids/topk_w NULL or misaligned", fn);
  if (logit_bias && !aligned(logit_bias, 4)) return fail(BITMOE_EINVAL, "%s: logit_bias misaligned", fn);
  // the router needs only the common region of the workspace
  if (!ws || !aligned(ws, 256)) return fail(BITMOE_EINVAL, "%s: workspace is NULL or not 256-byte aligned", fn);
  Carve c(ws);
  int64_t *status;
  float *logits;
  uint16_t *wsplit;
  carve_common(c, L, T, &status, &logits, &wsplit);
  if (ws_bytes < c.off)
    return fail(BITMOE_EWORKSPACE, "%s: workspace has %zu bytes, needs %zu for T=%d", fn, ws_bytes, c.off, T);
  hipError_t e = bm::launch_route(x, x_dtype == BITMOE_BF16, T, L->d_model, L->n_experts, L->top_k, L->w_router,
                                  logit_bias, logits, topk_ids, topk_w, wsplit, stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return BITMOE_OK;
}

int moe_route_noalloc(const bitmoe_layer *L, const void *x, int32_t x_dtype, int32_t T, const float *logit_bias,
                      int32_t *topk_ids, float *topk_w, hipStream_t stream) {
  const char *fn = "moe_route_noalloc";
  int rc = check_layer(fn, L);
  if (rc) return rc;
  if (T < 0) return fail(BITMOE_EINVAL, "%s: T=%d is negative", fn, T);
  if (T > BITMOE_NOALLOC_MAX_T)
    return fail(BITMOE_EUNSUPPORTED, "%s: T=%d exceeds the scratch limit of %d tokens", fn, T, BITMOE_NOALLOC_MAX_T);
  if (x_dtype != BITMOE_F32 && x_dtype != BITMOE_BF16) return fail(BITMOE_EUNSUPPORTED, "%s: x_dtype %d", fn, x_dtype);
  if (T == 0) return BITMOE_OK;
  if (!x || !aligned(x, 16)) return fail(BITMOE_EINVAL, "%s: x is NULL or not 16-byte aligned", fn);
  if (!topk_ids || !topk_w || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return fail(BITMOE_EINVAL, "%s: topk_ids/topk_w NULL or misaligned", fn);
  if (logit_bias && !aligned(logit_bias, 4)) return fail(BITMOE_EINVAL, "%s: logit_bias misaligned", fn);
  void *sc = nullptr;
  if ((rc = scratch_address(fn, &sc))) return rc;
  Carve c(sc);
  int64_t *status;
  float *logits;
  uint16_t *wsplit;
  carve_common(c, L, T, &status, &logits, &wsplit);  // no router split below MAX_DECODE_T tokens
  if (c.off > NOALLOC_SCRATCH_BYTES || wsplit)
    return fail(BITMOE_EUNSUPPORTED, "%s: needs %zu bytes of scratch, has %zu", fn, c.off, NOALLOC_SCRATCH_BYTES);
  // the logits are written in full before they are read: nothing in the
  // scratch has to start at zero
  hipError_t e = bm::launch_route(x, x_dtype == BITMOE_BF16, T, L->d_model, L->n_experts, L->top_k, L->w_router,
                                  logit_bias, logits, topk_ids, topk_w, nullptr, stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return BITMOE_OK;
}

int moe_route_ex(const bitmoe_layer *L, const void *x, int32_t x_dtype, int32_t T, const bitmoe_route_opts *opts,
                 int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, hipStream_t stream) {
  const char *fn = "moe_route_ex";
  int rc = check_layer(fn, L);
  if (rc) return rc;
  if (!opts) return fail(BITMOE_EINVAL, "%s: opts is NULL", fn);
  if (T < 0) return fail(BITMOE_EINVAL, "%s: T=%d is negative", fn, T);
  if (x_dtype != BITMOE_F32 && x_dtype != BITMOE_BF16) return fail(BITMOE_EUNSUPPORTED, "%s: x_dtype %d", fn, x_dtype);
  if (opts->score != BITMOE_SCORE_SOFTMAX && opts->score != BITMOE_SCORE_SQRT_SOFTPLUS)
    return fail(BITMOE_EUNSUPPORTED, "%s: score %d", fn, opts->score);
  if ((opts->hash_table == nullptr) != (opts->token_ids == nullptr))
    return fail(BITMOE_EINVAL, "%s: hash_table and token_ids go together", fn);
  if (opts->hash_table && opts->vocab < 1) return fail(BITMOE_EINVAL, "%s: vocab=%lld", fn, (long long)opts->vocab);
  if (T == 0) return BITMOE_OK;
  if (!x || !aligned(x, 16)) return fail(BITMOE_EINVAL, "%s: x is NULL or not 16-byte aligned", fn);
  if (!topk_ids || !topk_w || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return fail(BITMOE_EINVAL, "%s: topk_ids/topk_w NULL or misaligned", fn);
  const void *opt_ptrs[4] = {opts->logit_bias, opts->select_bias, opts->hash_table, opts->token_ids};
  for (const void *q : opt_ptrs)
    if (q && !aligned(q, 4)) return fail(BITMOE_EINVAL, "%s: an option array is misaligned", fn);
  if (!ws || !aligned(ws, 256)) return fail(BITMOE_EINVAL, "%s: workspace is NULL or not 256-byte aligned", fn);
  Carve c(ws);
  int64_t *status;
  float *logits;
  uint16_t *wsplit;
  carve_common(c, L, T, &status, &logits, &wsplit);
  if (ws_bytes < c.off)
    return fail(BITMOE_EWORKSPACE, "%s: workspace has %zu bytes, needs %zu for T=%d", fn, ws_bytes, c.off, T);
  hipError_t e = bm::launch_route_variant(x, x_dtype == BITMOE_BF16, T, L->d_model, L->n_experts, L->top_k,
                                          L->w_router, opts->logit_bias, opts->score, opts->select_bias,
                                          opts->hash_table, opts->token_ids, opts->vocab, logits, topk_ids, topk_w,
                                          status, wsplit, stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return BITMOE_OK;
}

// moe_expert_ffn; with x_next set (x bf16, checked by the caller) the combine
// launch also runs the stack's residual step into x_next.
static int expert_ffn_impl(const char *fn, const bitmoe_layer *L, const void *x, int32_t x_dtype, int32_t T,
                           const int32_t *topk_ids, const float *topk_w, void *y, int32_t y_dtype, int32_t mode,
                           void *ws, size_t ws_bytes, uint16_t *x_next, hipStream_t stream) {
  const uint16_t *x_res = x_next ? static_cast<const uint16_t *>(x) : nullptr;
  int rc = check_layer(fn, L);
  if (rc) return rc;
  if (T < 0) return fail(BITMOE_EINVAL, "%s: T=%d is negative", fn, T);
  if (x_dtype != BITMOE_F32 && x_dtype != BITMOE_BF16) return fail(BITMOE_EUNSUPPORTED, "%s: x_dtype %d", fn, x_dtype);
  if (y_dtype != BITMOE_F32 && y_dtype != BITMOE_BF16) return fail(BITMOE_EUNSUPPORTED, "%s: y_dtype %d", fn, y_dtype);
  if (mode < BITMOE_MODE_AUTO || mode > BITMOE_MODE_PREFILL_INT8)
    return fail(BITMOE_EINVAL, "%s: unknown mode %d", fn, mode);
  if ((mode == BITMOE_MODE_DECODE_INT8 || mode == BITMOE_MODE_PREFILL_INT8) && L->d_ff < 256)
    return fail(BITMOE_EUNSUPPORTED, "%s: int8 numerics need d_ff >= 256 (got %d)", fn, L->d_ff);
  if (T == 0) return BITMOE_OK;
  const int m = resolve_mode(mode, T);
  if ((m == BITMOE_MODE_DECODE || m == BITMOE_MODE_DECODE_INT8) && T > MAX_DECODE_T)
    return fail(BITMOE_EUNSUPPORTED, "%s: decode mode takes at most %d tokens, got T=%d", fn, MAX_DECODE_T, T);
  if (!x || !aligned(x, 16)) return fail(BITMOE_EINVAL, "%s: x is NULL or not 16-byte aligned", fn);
  if (!y || !aligned(y, 16)) return fail(BITMOE_EINVAL, "%s: y is NULL or not 16-byte aligned", fn);
  if (!topk_ids || !topk_w || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return fail(BITMOE_EINVAL, "%s: topk_ids/topk_w NULL or misaligned", fn);
  rc = check_ws(fn, L, T, m, ws, ws_bytes);
  if (rc) return rc;
  Carve c(ws);
  int64_t *status;
  carve_common(c, L, T, &status, nullptr);
  const bool shared = L->shared_wfmt == BITMOE_WFMT_Q8_0;
  if (m == BITMOE_MODE_DECODE) {
    bm::FfnArgs a = decode_args(c, L, x, T, topk_ids, topk_w, y, y_dtype, status);
    a.x_res = x_res;
    a.x_next = x_next;
    hipError_t e = bm::launch_decode_ffn(a, x_dtype == BITMOE_F32, stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return BITMOE_OK;
  }
  if (m == BITMOE_MODE_DECODE_INT8) {
    bm::FfnArgs a = decode_args(c, L, x, T, topk_ids, topk_w, y, y_dtype, status, true);
    a.x_res = x_res;
    a.x_next = x_next;
    hipError_t e = bm::launch_decode_ffn_i8(a, x_dtype == BITMOE_F32, stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return BITMOE_OK;
  }
  if (m == BITMOE_MODE_PREFILL_INT8) {
    bm::PrefillI8Args a{};
    carve_prefill_i8(c, L, T, &a);
    a.D = L->d_model;
    a.F = L->d_ff;
    a.E = L->n_experts;
    a.k = L->top_k;
    a.T = T;
    a.wg = static_cast<const uint8_t *>(L->w_gate);
    a.wu = static_cast<const uint8_t *>(L->w_up);
    a.wd = static_cast<const uint8_t *>(L->w_down);
    a.sg = shared ? static_cast<const uint8_t *>(L->ws_gate) : nullptr;
    a.su = shared ? static_cast<const uint8_t *>(L->ws_up) : nullptr;
    a.sd = shared ? static_cast<const uint8_t *>(L->ws_down) : nullptr;
    a.x = x;
    a.x_f32 = x_dtype == BITMOE_F32;
    a.ids = topk_ids;
    a.wts = topk_w;
    a.plan.status = status;
    a.out = y;
    a.out_bf16 = y_dtype == BITMOE_BF16;
    a.status = status;
    a.x_res = x_res;
    a.x_next = x_next;
    hipError_t e = bm::launch_prefill_ffn_i8(a, stream);
    if (e == hipErrorNotSupported)
      return fail(BITMOE_EUNSUPPORTED, "%s: int8 prefill path not available for this shape", fn);
    if (e != hipSuccess) return hip_fail(fn, e);
    return BITMOE_OK;
  }
  PrefillWs w;
  carve_prefill(c, L, T, &w);
  bm::PrefillArgs a{};
  a.D = L->d_model;
  a.F = L->d_ff;
  a.E = L->n_experts;
  a.k = L->top_k;
  a.T = T;
  a.wg = static_cast<const uint8_t *>(L->w_gate);
  a.wu = static_cast<const uint8_t *>(L->w_up);
  a.wd = static_cast<const uint8_t *>(L->w_down);
  a.sg = shared ? static_cast<const uint8_t *>(L->ws_gate) : nullptr;
  a.su = shared ? static_cast<const uint8_t *>(L->ws_up) : nullptr;
  a.sd = shared ? static_cast<const uint8_t *>(L->ws_down) : nullptr;
  a.x = x;
  a.x_f32 = x_dtype == BITMOE_F32;
  a.ids = topk_ids;
  a.wts = topk_w;
  a.plan = w.plan;
  a.plan.status = status;
  a.tile_off = w.tile_off;
  a.tile_off2 = w.tile_off2;
  a.xs = w.xs;
  a.h = w.h;
  a.hs = w.hs;
  a.h_lo = w.h_lo;
  a.hs_lo = w.hs_lo;
  a.sw_bf16 = w.sw;
  a.xsum = w.xsum;
  a.xtot = w.xtot;
  a.y = w.y;
  a.ys = w.ys;
  a.out = y;
  a.out_bf16 = y_dtype == BITMOE_BF16;
  a.status = status;
  a.x_res = x_res;
  a.x_next = x_next;
  hipError_t e = bm::launch_prefill_ffn(a, stream);
  if (e == hipErrorNotSupported) return fail(BITMOE_EUNSUPPORTED, "%s: prefill path not available for this shape", fn);
  if (e != hipSuccess) return hip_fail(fn, e);
  return BITMOE_OK;
}

int moe_expert_ffn(const bitmoe_layer *L, const void *x, int32_t x_dtype, int32_t T, const int32_t *topk_ids,
                   const float *topk_w, void *y, int32_t y_dtype, int32_t mode, void *ws, size_t ws_bytes,
                   hipStream_t stream) {
  return expert_ffn_impl("moe_expert_ffn", L, x, x_dtype, T, topk_ids, topk_w, y, y_dtype, mode, ws, ws_bytes,
                         nullptr, stream);
}

static int layer_impl(const char *fn, const bitmoe_layer *L, const void *x, int32_t x_dtype, int32_t T,
                      const float *logit_bias, int32_t *topk_ids, float *topk_w, void *y, int32_t y_dtype, int32_t mode,
                      void *ws, size_t ws_bytes, uint16_t *x_next, hipStream_t stream) {
  int rc = check_layer(fn, L);
  if (rc) return rc;
  if (T < 0) return fail(BITMOE_EINVAL, "%s: T=%d is negative", fn, T);
  if (mode < BITMOE_MODE_AUTO || mode > BITMOE_MODE_PREFILL_INT8)
    return fail(BITMOE_EINVAL, "%s: unknown mode %d", fn, mode);
  if (T != 1 || resolve_mode(mode, T) != BITMOE_MODE_DECODE || L->top_k > 8) {
    // the two calls' launches in order
    rc = moe_route(L, x, x_dtype, T, logit_bias, topk_ids, topk_w, ws, ws_bytes, stream);
    if (rc) return rc;
    return expert_ffn_impl(fn, L, x, x_dtype, T, topk_ids, topk_w, y, y_dtype, mode, ws, ws_bytes, x_next, stream);
  }
  if (x_dtype != BITMOE_F32 && x_dtype != BITMOE_BF16) return fail(BITMOE_EUNSUPPORTED, "%s: x_dtype %d", fn, x_dtype);
  if (y_dtype != BITMOE_F32 && y_dtype != BITMOE_BF16) return fail(BITMOE_EUNSUPPORTED, "%s: y_dtype %d", fn, y_dtype);
  if (!x || !aligned(x, 16)) return fail(BITMOE_EINVAL, "%s: x is NULL or not 16-byte aligned", fn);
  if (!y || !aligned(y, 16)) return fail(BITMOE_EINVAL, "%s: y is NULL or not 16-byte aligned", fn);
  if (!topk_ids || !topk_w || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return fail(BITMOE_EINVAL, "%s: topk_ids/topk_w NULL or misaligned", fn);
  if (logit_bias && !aligned(logit_bias, 4)) return fail(BITMOE_EINVAL, "%s: logit_bias misaligned", fn);
  rc = check_ws(fn, L, T, BITMOE_MODE_DECODE, ws, ws_bytes);
  if (rc) return rc;
  Carve c(ws);
  int64_t *status;
  float *logits;
  carve_common(c, L, T, &status, &logits);
  bm::FfnArgs a = decode_args(c, L, x, T, topk_ids, topk_w, y, y_dtype, status);
  a.x_res = x_next ? static_cast<const uint16_t *>(x) : nullptr;
  a.x_next = x_next;
  hipError_t e = bm::launch_decode_layer(a, x_dtype == BITMOE_F32, L->w_router, logit_bias, logits, stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return BITMOE_OK;
}

int moe_layer(const bitmoe_layer *L, const void *x, int32_t x_dtype, int32_t T, const float *logit_bias,
              int32_t *topk_ids, float *topk_w, void *y, int32_t y_dtype, int32_t mode, void *ws, size_t ws_bytes,
              hipStream_t stream) {
  return layer_impl("moe_layer", L, x, x_dtype, T, logit_bias, topk_ids, topk_w, y, y_dtype, mode, ws, ws_bytes,
                    nullptr, stream);
}

int moe_layer_residual(const bitmoe_layer *L, const void *x, int32_t T, const float *logit_bias, int32_t *topk_ids,
                       float *topk_w, void *y, int32_t y_dtype, void *x_next, int32_t mode, void *ws, size_t ws_bytes,
                       hipStream_t stream) {
  const char *fn = "moe_layer_residual";
  int rc = check_layer(fn, L);
  if (rc) return rc;
  if (L->d_model % 16 || L->d_model > 4096)
    return fail(BITMOE_EUNSUPPORTED, "%s: the residual step takes d_model a multiple of 16 up to 4096, got %d", fn,
                L->d_model);
  if (T < 0) return fail(BITMOE_EINVAL, "%s: T=%d is negative", fn, T);
  if (T == 0) return BITMOE_OK;
  if (!x_next || !aligned(x_next, 16)) return fail(BITMOE_EINVAL, "%s: x_next is NULL or not 16-byte aligned", fn);
  if (x_next == y) return fail(BITMOE_EINVAL, "%s: x_next must not alias y", fn);
  return layer_impl(fn, L, x, BITMOE_BF16, T, logit_bias, topk_ids, topk_w, y, y_dtype, mode, ws, ws_bytes,
                    static_cast<uint16_t *>(x_next), stream);
}

int engram_gather(const uint8_t *table, int64_t n_rows, const int64_t *row_ids, int64_t n, uint16_t *out,
                  int64_t *status, hipStream_t stream) {
  const char *fn = "engram_gather";
  if (n < 0) return fail(BITMOE_EINVAL, "%s: n=%lld is negative", fn, (long long)n);
  if (n_rows < 0) return fail(BITMOE_EINVAL, "%s: n_rows=%lld is negative", fn, (long long)n_rows);
  if (n == 0) return BITMOE_OK;
  if (!table || !aligned(table, 8)) return fail(BITMOE_EINVAL, "%s: table is NULL or not 8-byte aligned", fn);
  if (!row_ids || !aligned(row_ids, 8)) return fail(BITMOE_EINVAL, "%s: row_ids is NULL or not 8-byte aligned", fn);
  if (!out || !aligned(out, 16)) return fail(BITMOE_EINVAL, "%s: out is NULL or not 16-byte aligned", fn);
  if (status && !aligned(status, 8)) return fail(BITMOE_EINVAL, "%s: status not 8-byte aligned", fn);
  if (n > (int64_t(1) << 33)) return fail(BITMOE_EUNSUPPORTED, "%s: n=%lld rows in one call", fn, (long long)n);
  bm::EngramTables tabs{};
  tabs.table[0] = table;
  tabs.rows[0] = n_rows;
  tabs.n = 1;
  hipError_t e = bm::launch_engram_gather(tabs, int32_t(1), row_ids, n, out, status, stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return BITMOE_OK;
}

int engram_gather_tables(const uint8_t *const *tables, const int64_t *n_rows, int32_t n_tables,
                         const int64_t *row_ids, int64_t n_groups, int32_t per, uint16_t *out, int64_t *status,
                         hipStream_t stream) {
  const char *fn = "engram_gather_tables";
  if (n_tables < 1 || n_tables > bm::ENGRAM_MAX_TABLES)
    return fail(BITMOE_EINVAL, "%s: n_tables=%d outside 1..%d", fn, n_tables, bm::ENGRAM_MAX_TABLES);
  if (!tables || !n_rows) return fail(BITMOE_EINVAL, "%s: tables or n_rows is NULL", fn);
  if (n_groups < 0 || per < 1) return fail(BITMOE_EINVAL, "%s: n_groups=%lld per=%d", fn, (long long)n_groups, per);
  bm::EngramTables tabs{};
  tabs.n = n_tables;
  for (int j = 0; j < n_tables; ++j) {
    if (n_rows[j] < 0) return fail(BITMOE_EINVAL, "%s: n_rows[%d]=%lld is negative", fn, j, (long long)n_rows[j]);
    if (!tables[j] || !aligned(tables[j], 8))
      return fail(BITMOE_EINVAL, "%s: tables[%d] is NULL or not 8-byte aligned", fn, j);
    tabs.table[j] = tables[j];
    tabs.rows[j] = n_rows[j];
  }
  if (n_groups > ((int64_t(1) << 33) / n_tables / per))
    return fail(BITMOE_EUNSUPPORTED, "%s: %lld groups of %d x %d rows in one call", fn, (long long)n_groups, n_tables,
                per);
  const int64_t n = n_groups * n_tables * per;
  if (n == 0) return BITMOE_OK;
  if (!row_ids || !aligned(row_ids, 8)) return fail(BITMOE_EINVAL, "%s: row_ids is NULL or not 8-byte aligned", fn);
  if (!out || !aligned(out, 16)) return fail(BITMOE_EINVAL, "%s: out is NULL or not 16-byte aligned", fn);
  if (status && !aligned(status, 8)) return fail(BITMOE_EINVAL, "%s: status not 8-byte aligned", fn);
  hipError_t e = bm::launch_engram_gather(tabs, per, row_ids, n, out, status, stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return BITMOE_OK;
}

int engram_inject_workspace_size(int32_t T, int32_t width, size_t *bytes) {
  if (!bytes || T < 0 || width < 256 || width > 8192 || width % 256)
    return fail(BITMOE_EINVAL, "engram_inject_workspace_size: bad arguments (T=%d width=%d)", T, width);
  *bytes = up256(size_t(T) * 5 * width * sizeof(float));
  return BITMOE_OK;
}

int engram_inject(const uint16_t *rows, int32_t T, int32_t n_rows, const uint16_t *w_kv, int32_t width,
                  const float *q_norm, const float *k_norm, float eps, const uint8_t *mask, uint16_t *residual,
                  float *gate_out, void *ws, size_t ws_bytes, hipStream_t stream) {
  const char *fn = "engram_inject";
  if (T < 0) return fail(BITMOE_EINVAL, "%s: T=%d is negative", fn, T);
  if (T > 262144) return fail(BITMOE_EUNSUPPORTED, "%s: T=%d above 262144 positions per call", fn, T);
  if (n_rows < 2 || n_rows > 32 || n_rows % 2)
    return fail(BITMOE_EUNSUPPORTED, "%s: n_rows=%d must be even in [2, 32]", fn, n_rows);
  if (width < 256 || width > 8192 || width % 256)
    return fail(BITMOE_EUNSUPPORTED, "%s: width=%d must be a multiple of 256 in [256, 8192]", fn, width);
  if (!(eps >= 0.f) || eps > 1.f) return fail(BITMOE_EINVAL, "%s: eps=%g", fn, double(eps));
  if (T == 0) return BITMOE_OK;
  if (!rows || !w_kv || !residual || !aligned(rows, 16) || !aligned(w_kv, 16) || !aligned(residual, 16))
    return fail(BITMOE_EINVAL, "%s: rows, w_kv or residual NULL or not 16-byte aligned", fn);
  if (!q_norm || !k_norm || !aligned(q_norm, 16) || !aligned(k_norm, 16) || (gate_out && !aligned(gate_out, 4)))
    return fail(BITMOE_EINVAL, "%s: q_norm/k_norm NULL or not 16-byte aligned, or gate_out misaligned", fn);
  size_t need = 0;
  engram_inject_workspace_size(T, width, &need);
  if (!ws || !aligned(ws, 256)) return fail(BITMOE_EINVAL, "%s: workspace is NULL or not 256-byte aligned", fn);
  if (ws_bytes < need) return fail(BITMOE_EWORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn, ws_bytes, need);
  hipError_t e = bm::launch_engram_inject(rows, T, n_rows, w_kv, width, q_norm, k_norm, eps, mask, residual, gate_out,
                                          static_cast<float *>(ws), stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return BITMOE_OK;
}

int bitmoe_plan_workspace_size(int32_t T, int32_t k, int32_t n_experts, size_t *bytes) {
  if (!bytes || T < 0 || k < 1 || n_experts < 1 || n_experts > 1024)
    return fail(BITMOE_EINVAL, "bitmoe_plan_workspace_size: bad arguments (T=%d k=%d E=%d)", T, k, n_experts);
  (void)k;
  *bytes = up256(bm::plan_scratch_bytes(T, n_experts));
  return BITMOE_OK;
}

int moe_plan(const int32_t *topk_ids, int32_t T, int32_t k, int32_t n_experts, int32_t *counts, int32_t *offsets,
             int32_t *perm, int32_t *union_ids, int32_t *n_union, int64_t *status, void *ws, size_t ws_bytes,
             hipStream_t stream) {
  const char *fn = "moe_plan";
  if (T < 0 || k < 1 || k > 64 || n_experts < 1 || n_experts > 1024)
    return fail(BITMOE_EINVAL, "%s: bad sizes T=%d k=%d n_experts=%d", fn, T, k, n_experts);
  if (!counts || !offsets || !n_union || !union_ids) return fail(BITMOE_EINVAL, "%s: NULL output", fn);
  if (T > 0 && (!topk_ids || !perm)) return fail(BITMOE_EINVAL, "%s: NULL ids or perm", fn);
  size_t need = up256(bm::plan_scratch_bytes(T, n_experts));
  if (!ws || ws_bytes < need) return fail(BITMOE_EWORKSPACE, "%s: workspace %zu bytes, needs %zu", fn, ws_bytes, need);
  bm::PlanBufs p{counts, offsets, perm, union_ids, n_union, static_cast<int32_t *>(ws), nullptr, nullptr, status};
  hipError_t e = bm::launch_plan(topk_ids, T, k, n_experts, 0, 0, p, stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return BITMOE_OK;
}

int moe_dequant(const void *blocks, int32_t wfmt, int64_t n_weights, void *out, int32_t out_dtype,
                hipStream_t stream) {
  const char *fn = "moe_dequant";
  if (wfmt != BITMOE_WFMT_Q2SB && wfmt != BITMOE_WFMT_Q8_0) return fail(BITMOE_EUNSUPPORTED, "%s: format %d", fn, wfmt);
  if (out_dtype != BITMOE_F32 && out_dtype != BITMOE_BF16) return fail(BITMOE_EUNSUPPORTED, "%s: out_dtype %d", fn, out_dtype);
  const int64_t blk = wfmt == BITMOE_WFMT_Q2SB ? 256 : 32;
  if (n_weights < 0 || n_weights % blk) return fail(BITMOE_EINVAL, "%s: n_weights %lld not a multiple of %lld", fn,
                                                    (long long)n_weights, (long long)blk);
  if (n_weights == 0) return BITMOE_OK;
  if (!blocks || !aligned(blocks, 4) || !out || !aligned(out, 16))
    return fail(BITMOE_EINVAL, "%s: NULL or misaligned pointer", fn);
  hipError_t e = bm::launch_dequant(blocks, wfmt, n_weights, out, out_dtype == BITMOE_BF16, stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return BITMOE_OK;
}

int moe_quantize_q8_1(const void *x, int32_t x_dtype, int64_t rows, int32_t cols, int8_t *q, float *d, float *s,
                      hipStream_t stream) {
  const char *fn = "moe_quantize_q8_1";
  if (x_dtype != BITMOE_F32 && x_dtype != BITMOE_BF16) return fail(BITMOE_EUNSUPPORTED, "%s: x_dtype %d", fn, x_dtype);
  if (rows < 0 || cols <= 0 || cols % 32)
    return fail(BITMOE_EINVAL, "%s: rows %lld / cols %d (cols must be a positive multiple of 32)", fn,
                (long long)rows, cols);
  if (rows == 0) return BITMOE_OK;
  if (!x || !aligned(x, 16) || !q || !aligned(q, 16) || !d || !aligned(d, 4) || !s || !aligned(s, 4))
    return fail(BITMOE_EINVAL, "%s: NULL or misaligned pointer", fn);
  hipError_t e = bm::launch_quantize_q8(x, x_dtype == BITMOE_F32, rows, cols, reinterpret_cast<uint8_t *>(q), d, s,
                                        stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return BITMOE_OK;
}

int bitmoe_fill(void *dst, int64_t n_bytes, uint64_t key, int32_t kind, const uint16_t *lut, hipStream_t stream) {
  const char *fn = "bitmoe_fill";
  static const int64_t unit[4] = {1, 84, 34, 264};
  if (kind < 0 || kind > 3) return fail(BITMOE_EINVAL, "%s: kind %d", fn, kind);
  if (n_bytes < 0 || n_bytes % unit[kind])
    return fail(BITMOE_EINVAL, "%s: n_bytes %lld not a multiple of %lld", fn, (long long)n_bytes, (long long)unit[kind]);
  if (n_bytes == 0) return BITMOE_OK;
  if (!dst) return fail(BITMOE_EINVAL, "%s: dst is NULL", fn);
  if ((kind == 1 || kind == 2) && !lut) return fail(BITMOE_EINVAL, "%s: lut is NULL", fn);
  hipError_t e = bm::launch_fill(dst, n_bytes, key, kind, lut, stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return BITMOE_OK;
}

int bitmoe_probe_read(const void *src, int64_t n_bytes, uint32_t *sink, int32_t blocks, hipStream_t stream) {
  if (!src || !sink || !aligned(src, 16) || n_bytes < 0 || blocks < 1 || blocks > (1 << 20))
    return fail(BITMOE_EINVAL, "bitmoe_probe_read: bad arguments (n_bytes=%lld blocks=%d)", (long long)n_bytes, blocks);
  hipError_t e = bm::launch_probe_read(src, n_bytes, sink, blocks, stream);
  if (e != hipSuccess) return hip_fail("bitmoe_probe_read", e);
  return BITMOE_OK;
}

int bitmoe_probe_mfma(int32_t blocks, int32_t iters, uint32_t *sink, hipStream_t stream) {
  if (!sink || !aligned(sink, 4) || blocks < 1 || blocks > (1 << 20) || iters < 0)
    return fail(BITMOE_EINVAL, "bitmoe_probe_mfma: bad arguments (blocks=%d iters=%d)", blocks, iters);
  hipError_t e = bm::launch_probe_mfma(blocks, iters, sink, stream);
  if (e != hipSuccess) return hip_fail("bitmoe_probe_mfma", e);
  return BITMOE_OK;
}

int bitmoe_residual_rescale(const void *x, const void *y, int32_t y_dtype, int32_t T, int32_t D, void *x_out,
                            hipStream_t stream) {
  const char *fn = "bitmoe_residual_rescale";
  if (T < 0 || D < 16 || D > 4096 || D % 16) return fail(BITMOE_EINVAL, "%s: T=%d D=%d unsupported", fn, T, D);
  if (y_dtype != BITMOE_F32 && y_dtype != BITMOE_BF16) return fail(BITMOE_EUNSUPPORTED, "%s: y_dtype %d", fn, y_dtype);
  if (T == 0) return BITMOE_OK;
  if (!x || !y || !x_out || !aligned(x, 16) || !aligned(y, 16) || !aligned(x_out, 16))
    return fail(BITMOE_EINVAL, "%s: NULL or misaligned pointer", fn);
  hipError_t e = bm::launch_residual_rescale(static_cast<const uint16_t *>(x), y, y_dtype == BITMOE_F32, T, D,
                                             static_cast<uint16_t *>(x_out), stream);
  if (e != hipSuccess) return hip_fail(fn, e);
  return BITMOE_OK;
}

int bitmoe_read_status(const int64_t *status, hipStream_t stream, int64_t *code, int64_t *detail) {
  if (!status || !code || !detail) return fail(BITMOE_EINVAL, "bitmoe_read_status: NULL argument");
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail("bitmoe_read_status", e);
  int64_t h[2];
  e = hipMemcpy(h, status, sizeof(h), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail("bitmoe_read_status", e);
  *code = h[0];
  *detail = h[0] ? INT64_MAX - h[1] : -1;
  return h[0] ? BITMOE_EDEVICE : BITMOE_OK;
}

}  // extern "C"
