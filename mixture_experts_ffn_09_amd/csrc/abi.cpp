// C ABI of the MoE FFN library: argument checks (all on the host, before any
// HIP call), workspace carving, and kernel orchestration.  See moe_ffn.h.

#include <initializer_list>

#include "moe_ffn.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kernels.h"

namespace {

constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 64;

thread_local char g_err[512] = "";

moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

moe_status_t hip_fail(const char* where, hipError_t e) {
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define HIP_TRY(where, expr)                     \
  do {                                           \
    hipError_t e_ = (expr);                      \
    if (e_ != hipSuccess) return hip_fail(where, e_); \
  } while (0)

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int act_size(const moe_shape_t* s) { return s->act_dtype == MOE_F32 ? 4 : 2; }

// bytes per weight element; 0 marks MXFP4 (two elements per byte)
int w_size(const moe_shape_t* s) {
  return s->w_dtype == MOE_F32 ? 4 : (s->w_dtype == MOE_BF16 ? 2 : (s->w_dtype == MOE_MXFP4 ? 0 : 1));
}

bool scaled(const moe_shape_t* s) { return s->w_dtype == MOE_FP8_E4M3 || s->w_dtype == MOE_MXFP4; }

moe_status_t check_shape(const moe_shape_t* s) {
  if (!s) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
  if (s->n_tokens < 0) return fail(MOE_ERR_INVALID_ARG, "n_tokens < 0");
  if (s->d_model < 1 || s->d_ff < 1) return fail(MOE_ERR_INVALID_ARG, "d_model, d_ff must be >= 1");
  if (s->n_experts < 1) return fail(MOE_ERR_INVALID_ARG, "n_experts must be >= 1");
  if (s->top_k < 1 || s->top_k > s->n_experts)
    return fail(MOE_ERR_INVALID_ARG, "need 1 <= top_k <= n_experts");
  if (s->n_shared != 0 && s->n_shared != 1) return fail(MOE_ERR_INVALID_ARG, "n_shared must be 0 or 1");
  if (s->route != MOE_ROUTE_SOFTMAX_TOPK && s->route != MOE_ROUTE_SIGMOID_BIAS)
    return fail(MOE_ERR_INVALID_ARG, "unknown route %d", s->route);
  if (s->act_dtype != MOE_F32 && s->act_dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "act_dtype must be MOE_F32 or MOE_BF16");
  if (s->w_dtype != MOE_F32 && s->w_dtype != MOE_BF16 && s->w_dtype != MOE_FP8_E4M3 &&
      s->w_dtype != MOE_MXFP4)
    return fail(MOE_ERR_INVALID_ARG, "unknown w_dtype %d", s->w_dtype);
  if (s->n_experts > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "n_experts > %d", kMaxExperts);
  if (s->top_k > kMaxTopK) return fail(MOE_ERR_UNSUPPORTED, "top_k > %d", kMaxTopK);
  if ((s->act_dtype == MOE_F32) != (s->w_dtype == MOE_F32))
    return fail(MOE_ERR_UNSUPPORTED, "float32 activations pair with float32 weights only");
  if (s->w_dtype == MOE_BF16 && (s->d_model % 32 || s->d_ff % 32))
    return fail(MOE_ERR_UNSUPPORTED, "bfloat16 weights need d_model %% 32 == 0 and d_ff %% 32 == 0");
  if (s->w_dtype == MOE_FP8_E4M3 && (s->d_model % 128 || s->d_ff % 128))
    return fail(MOE_ERR_UNSUPPORTED, "FP8 weights need d_model %% 128 == 0 and d_ff %% 128 == 0");
  if (s->w_dtype == MOE_MXFP4 && (s->d_model % 128 || s->d_ff % 128))
    return fail(MOE_ERR_UNSUPPORTED, "MXFP4 weights need d_model %% 128 == 0 and d_ff %% 128 == 0");
  const long long tk = (long long)s->n_tokens * s->top_k;
  if (tk > INT_MAX / 2) return fail(MOE_ERR_UNSUPPORTED, "n_tokens * top_k too large");
  if (s->act_dtype == MOE_F32 && (tk + 15) / 16 > 65535)
    return fail(MOE_ERR_UNSUPPORTED, "float32 path: n_tokens * top_k > %d", 16 * 65535);
  return MOE_OK;
}

struct WsLayout {
  size_t logits, idx, w, counts, offsets, perm, inv, hist, stats, ccounts, coffsets, cperm, cinv,
      sched, H, H_sh, Y, Y_sh, total;
};

WsLayout ws_layout(const moe_shape_t* s) {
  WsLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t T = s->n_tokens, k = s->top_k, N = s->n_experts, d = s->d_model, f = s->d_ff;
  const size_t es = act_size(s), sh = s->n_shared;
  L.logits = take(router_scratch_bytes(s->n_tokens, s->n_experts, s->d_model,
                                       s->act_dtype == MOE_BF16));
  L.idx = take(T * k * 4);
  L.w = take(T * k * 4);
  L.counts = take(N * 4);
  L.offsets = take((N + 1) * 4);
  L.perm = take(T * k * 4);
  L.inv = take(T * k * 4);
  L.hist = take((size_t)permute_blocks(s->n_tokens) * N * 4);
  L.stats = take((size_t)stats_blocks(s->n_tokens) * N * 4);
  L.ccounts = take(N * 4);
  L.coffsets = take((N + 1) * 4);
  L.cperm = take(T * k * 4);
  L.cinv = take(T * k * 4);
  L.sched = take(2048 * 4);
  L.H = take(T * k * f * es);
  L.H_sh = take(sh * T * f * es);
  L.Y = take(T * k * d * es);
  L.Y_sh = take(sh * T * d * es);
  L.total = off;
  return L;
}

// The kernels move activations, weights and workspace pieces with 16-byte
// vector loads and stores, so those buffers must be 16-byte aligned (every
// hipMalloc and torch allocation is).
bool misaligned(std::initializer_list<const void*> ps) {
  for (const void* q : ps)
    if (q && (reinterpret_cast<uintptr_t>(q) & 15)) return true;
  return false;
}

moe_status_t check_aligned(std::initializer_list<const void*> ps) {
  if (misaligned(ps)) return fail(MOE_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
  return MOE_OK;
}

moe_status_t check_ws(const moe_shape_t* s, void* ws, size_t ws_bytes) {
  const size_t need = ws_layout(s).total;
  if (!ws) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL");
  if (misaligned({ws})) return fail(MOE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, need);
  return MOE_OK;
}

moe_status_t check_weights(const moe_shape_t* s, const moe_weights_t* w, bool router, bool ffn) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  if (router) {
    if (!w->w_router) return fail(MOE_ERR_INVALID_ARG, "w_router is NULL");
    if (w->select_bias && s->route != MOE_ROUTE_SIGMOID_BIAS)
      return fail(MOE_ERR_INVALID_ARG, "select_bias belongs to the sigmoid router");
  }
  if (ffn) {
    if (!w->w13 || !w->w2) return fail(MOE_ERR_INVALID_ARG, "w13 / w2 is NULL");
    if (scaled(s) && (!w->w13_scale || !w->w2_scale))
      return fail(MOE_ERR_INVALID_ARG, "FP8 / MXFP4 weights need w13_scale and w2_scale");
    if (s->n_shared) {
      if (!w->w13_shared || !w->w2_shared)
        return fail(MOE_ERR_INVALID_ARG, "n_shared == 1 needs w13_shared / w2_shared");
      if (scaled(s) && (!w->w13_shared_scale || !w->w2_shared_scale))
        return fail(MOE_ERR_INVALID_ARG, "FP8 / MXFP4 shared expert needs its scales");
    }
    if (misaligned({w->w13, w->w2, w->w13_shared, w->w2_shared, w->w13_scale, w->w2_scale,
                    w->w13_shared_scale, w->w2_shared_scale}))
      return fail(MOE_ERR_INVALID_ARG, "weights and scales must be 16-byte aligned");
  }
  if (router && misaligned({w->w_router}))
    return fail(MOE_ERR_INVALID_ARG, "w_router must be 16-byte aligned");
  return MOE_OK;
}

// Group limit of the selection: 0 groups = none.  Checked on the host.
struct GroupLimit {
  int n_groups = 0, max_groups = 0;
};

moe_status_t check_groups(const moe_shape_t* s, const GroupLimit& g) {
  if (g.n_groups == 0) return MOE_OK;
  if (g.n_groups < 1 || s->n_experts % g.n_groups)
    return fail(MOE_ERR_INVALID_ARG, "n_groups must divide n_experts");
  if (g.n_groups > 64) return fail(MOE_ERR_UNSUPPORTED, "n_groups > 64");
  if (g.max_groups < 1 || g.max_groups > g.n_groups)
    return fail(MOE_ERR_INVALID_ARG, "need 1 <= max_groups <= n_groups");
  if ((long long)s->top_k > (long long)g.max_groups * (s->n_experts / g.n_groups))
    return fail(MOE_ERR_INVALID_ARG, "top_k exceeds the experts of max_groups groups");
  return MOE_OK;
}

moe_status_t run_router(const moe_shape_t* s, const void* x, const moe_weights_t* w,
                        int32_t* idx, float* gw, float* logits, hipStream_t st,
                        const GroupLimit& g = GroupLimit()) {
  if (router_fused_small(s->n_tokens, s->n_experts)) {
    HIP_TRY("router_fused",
            launch_router_fused_small(x, s->act_dtype == MOE_BF16, w->w_router, w->logit_offset,
                                      s->route == MOE_ROUTE_SIGMOID_BIAS ? w->select_bias : nullptr,
                                      s->route == MOE_ROUTE_SIGMOID_BIAS, s->n_tokens, s->d_model,
                                      s->n_experts, s->top_k,
                                      g.n_groups ? s->n_experts / g.n_groups : 0, g.max_groups,
                                      idx, gw, st));
    return MOE_OK;
  }
  HIP_TRY("router_logits", launch_router_logits(x, s->act_dtype == MOE_BF16, w->w_router, logits,
                                                s->n_tokens, s->d_model, s->n_experts, st));
  HIP_TRY("router_topk",
          launch_router_topk(logits,
                             router_splits(s->n_tokens, s->n_experts, s->d_model,
                                           s->act_dtype == MOE_BF16),
                             w->logit_offset,
                             s->route == MOE_ROUTE_SIGMOID_BIAS ? w->select_bias : nullptr,
                             s->route == MOE_ROUTE_SIGMOID_BIAS, s->n_tokens, s->n_experts,
                             s->top_k, g.n_groups ? s->n_experts / g.n_groups : 0,
                             g.max_groups, idx, gw, st));
  return MOE_OK;
}

moe_status_t run_ffn(const moe_shape_t* s, const void* x, const void* x_rows,
                     const int32_t* perm, const int32_t* offsets, const moe_weights_t* w,
                     void* H, void* H_sh, void* y, void* y_sh, void* sched, int pass,
                     hipStream_t st) {
  if (s->w_dtype == MOE_F32) {
    FfnF32Args a{};
    a.x_rows = static_cast<const float*>(x_rows);
    a.perm_token = perm;
    a.x_sh = static_cast<const float*>(x);
    a.offsets = offsets;
    a.T = s->n_tokens;
    a.N = s->n_experts;
    a.n_shared = s->n_shared;
    a.d = s->d_model;
    a.d_ff = s->d_ff;
    a.max_rows = s->n_tokens * s->top_k;
    a.w13 = static_cast<const float*>(w->w13);
    a.w2 = static_cast<const float*>(w->w2);
    a.w13_sh = static_cast<const float*>(w->w13_shared);
    a.w2_sh = static_cast<const float*>(w->w2_shared);
    a.H = static_cast<float*>(H);
    a.H_sh = static_cast<float*>(H_sh);
    a.Y = static_cast<float*>(y);
    a.Y_sh = static_cast<float*>(y_sh);
    HIP_TRY("ffn_f32", launch_ffn_f32(a, pass, st));
    return MOE_OK;
  }
  FfnArgs a{};
  a.x_rows = static_cast<const uint16_t*>(x_rows);
  a.perm_token = perm;
  a.x_sh = static_cast<const uint16_t*>(x);
  a.offsets = offsets;
  a.T = s->n_tokens;
  a.k = s->top_k;
  a.N = s->n_experts;
  a.n_shared = s->n_shared;
  a.d = s->d_model;
  a.d_ff = s->d_ff;
  a.fp8 = s->w_dtype == MOE_FP8_E4M3;
  a.mxfp4 = s->w_dtype == MOE_MXFP4;
  a.sched = static_cast<int32_t*>(sched);
  a.w13 = w->w13;
  a.w2 = w->w2;
  a.s13 = w->w13_scale;
  a.s2 = w->w2_scale;
  a.w13_sh = w->w13_shared;
  a.w2_sh = w->w2_shared;
  a.s13_sh = w->w13_shared_scale;
  a.s2_sh = w->w2_shared_scale;
  a.H = static_cast<uint16_t*>(H);
  a.H_sh = static_cast<uint16_t*>(H_sh);
  a.Y = static_cast<uint16_t*>(y);
  a.Y_sh = static_cast<uint16_t*>(y_sh);
  HIP_TRY("ffn", launch_ffn_lowp(a, pass, st));
  return MOE_OK;
}

}  // namespace

// Scratch of moe_layer_forward_noalloc: a file-scope device array (each GPU
// the library runs on holds its own copy until the process ends), in place
// of a caller workspace.  Host code never passes the array's name to a
// kernel or a copy (on the host it is only a stand-in for the symbol): it
// uses the device address that hipGetSymbolAddress returns, looked up once
// per device with that device current.  Every call on a GPU shares that
// GPU's array; no kernel needs it cleared (each piece is written before it
// is read within a call), and calls that overlap on one GPU race.
__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device.
moe_status_t static_scratch(void** out) {
  int dev = -1;
  HIP_TRY("hipGetDevice", hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d: the static scratch covers devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    HIP_TRY("hipGetSymbolAddress(scratch)", hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or type";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_err; }

size_t moe_packed_weight_bytes(const moe_shape_t* s, int which, int n_mats) {
  if (check_shape(s) != MOE_OK || which < 0 || which > 3 || n_mats < 1) return 0;
  if (which >= 2) {
    if (s->w_dtype != MOE_MXFP4) return 0;
    return which == 2 ? packed_scale_bytes(n_mats, s->d_ff, s->d_model, 2)
                      : packed_scale_bytes(n_mats, s->d_model, s->d_ff, 1);
  }
  const size_t elems = (size_t)s->d_model * s->d_ff * (which == 0 ? 2 : 1);
  const size_t per = w_size(s) ? elems * w_size(s) : elems / 2;
  return per * (size_t)n_mats;
}

moe_status_t moe_pack_weights(const moe_shape_t* s, int which, int n_mats, const void* src_a,
                              const void* src_b, void* dst, hipStream_t stream) {
  moe_status_t st = check_shape(s);
  if (st != MOE_OK) return st;
  if (which < 0 || which > 3) return fail(MOE_ERR_INVALID_ARG, "which must be 0, 1, 2 or 3");
  if (n_mats < 1) return fail(MOE_ERR_INVALID_ARG, "n_mats must be >= 1");
  if (!src_a || !dst) return fail(MOE_ERR_INVALID_ARG, "src_a / dst is NULL");
  if ((st = check_aligned({src_a, src_b, dst})) != MOE_OK) return st;
  if (which >= 2) {
    if (s->w_dtype != MOE_MXFP4)
      return fail(MOE_ERR_UNSUPPORTED, "scale packing (which 2, 3) is for MXFP4 weights only");
    if (src_b) return fail(MOE_ERR_INVALID_ARG, "src_b must be NULL for which 2 and 3");
    const int rows = which == 2 ? s->d_ff : s->d_model;
    const int cols = which == 2 ? s->d_model : s->d_ff;
    HIP_TRY("pack scales", launch_pack_scales(src_a, dst, n_mats, rows, cols, which == 2 ? 2 : 1,
                                              stream));
    return MOE_OK;
  }
  if ((which == 0) != (src_b != nullptr))
    return fail(MOE_ERR_INVALID_ARG, "src_b is W_up for which == 0 and NULL for which == 1");
  const int rows = which == 0 ? s->d_ff : s->d_model;
  const int cols = which == 0 ? s->d_model : s->d_ff;
  HIP_TRY("pack", launch_pack(src_a, src_b, dst, n_mats, rows, cols, w_size(s), stream));
  return MOE_OK;
}

size_t moe_workspace_bytes(const moe_shape_t* s) {
  if (check_shape(s) != MOE_OK) return (size_t)-1;
  if (s->n_tokens == 0) return 0;
  return ws_layout(s).total;
}

static moe_status_t router_topk(const moe_shape_t* s, const void* x, const moe_weights_t* w,
                                const GroupLimit& g, int32_t* topk_idx, float* topk_w, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = check_shape(s);
  if (st != MOE_OK) return st;
  if ((st = check_groups(s, g)) != MOE_OK) return st;
  if (s->n_tokens == 0) return MOE_OK;
  if ((st = check_weights(s, w, true, false)) != MOE_OK) return st;
  if (!x || !topk_idx || !topk_w) return fail(MOE_ERR_INVALID_ARG, "x / topk_idx / topk_w is NULL");
  if ((st = check_aligned({x})) != MOE_OK) return st;
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  const WsLayout L = ws_layout(s);
  return run_router(s, x, w, topk_idx, topk_w,
                    reinterpret_cast<float*>(static_cast<char*>(ws) + L.logits), stream, g);
}

moe_status_t moe_router_topk(const moe_shape_t* s, const void* x, const moe_weights_t* w,
                             int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  return router_topk(s, x, w, GroupLimit(), topk_idx, topk_w, ws, ws_bytes, stream);
}

moe_status_t moe_router_topk_grouped(const moe_shape_t* s, const void* x, const moe_weights_t* w,
                                     int32_t n_groups, int32_t max_groups, int32_t* topk_idx,
                                     float* topk_w, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  if (n_groups < 1) return fail(MOE_ERR_INVALID_ARG, "n_groups must be >= 1");
  GroupLimit g;
  g.n_groups = n_groups;
  g.max_groups = max_groups;
  return router_topk(s, x, w, g, topk_idx, topk_w, ws, ws_bytes, stream);
}

moe_status_t moe_permute(const moe_shape_t* s, const int32_t* topk_idx, const void* x,
                         moe_routing_t* out, void* x_perm, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  moe_status_t st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!out || !out->counts || !out->offsets || !out->perm_token || !out->inv_perm)
    return fail(MOE_ERR_INVALID_ARG, "routing counts / offsets / perm_token / inv_perm is NULL");
  if (!topk_idx) return fail(MOE_ERR_INVALID_ARG, "topk_idx is NULL");
  if (x_perm && !x) return fail(MOE_ERR_INVALID_ARG, "x_perm needs x");
  if ((st = check_aligned({x, x_perm})) != MOE_OK) return st;
  if (s->n_tokens > 0 && (st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  // T == 0 still yields well-defined (zero) counts and offsets
  int32_t* hist = s->n_tokens > 0
                      ? reinterpret_cast<int32_t*>(static_cast<char*>(ws) + ws_layout(s).hist)
                      : nullptr;
  HIP_TRY("permute", launch_permute(topk_idx, s->n_tokens, s->top_k, s->n_experts, hist,
                                    out->counts, out->offsets, out->perm_token, out->inv_perm,
                                    stream));
  if (x_perm && s->n_tokens > 0)
    HIP_TRY("gather", launch_gather_rows(x, out->perm_token, x_perm, s->n_tokens * s->top_k,
                                         s->d_model * act_size(s), stream));
  return MOE_OK;
}

moe_status_t moe_permute_capacity(const moe_shape_t* s, const int32_t* topk_idx, int32_t capacity,
                                  moe_routing_t* out, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  moe_status_t st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!out || !out->counts || !out->offsets || !out->perm_token || !out->inv_perm)
    return fail(MOE_ERR_INVALID_ARG, "routing counts / offsets / perm_token / inv_perm is NULL");
  if (!topk_idx) return fail(MOE_ERR_INVALID_ARG, "topk_idx is NULL");
  if (capacity < 0) return fail(MOE_ERR_INVALID_ARG, "capacity is negative");
  if (s->n_tokens == 0) {
    HIP_TRY("permute", launch_permute(topk_idx, 0, s->top_k, s->n_experts, nullptr, out->counts,
                                      out->offsets, out->perm_token, out->inv_perm, stream));
    return MOE_OK;
  }
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  const WsLayout L = ws_layout(s);
  char* b = static_cast<char*>(ws);
  int32_t* cf = reinterpret_cast<int32_t*>(b + L.counts);
  int32_t* of = reinterpret_cast<int32_t*>(b + L.offsets);
  int32_t* pf = reinterpret_cast<int32_t*>(b + L.perm);
  int32_t* vf = reinterpret_cast<int32_t*>(b + L.inv);
  HIP_TRY("permute", launch_permute(topk_idx, s->n_tokens, s->top_k, s->n_experts,
                                    reinterpret_cast<int32_t*>(b + L.hist), cf, of, pf, vf,
                                    stream));
  HIP_TRY("capacity", launch_capacity(topk_idx, s->n_tokens, s->top_k, s->n_experts, capacity, cf,
                                      of, vf, out->counts, out->offsets, out->perm_token,
                                      out->inv_perm, stream));
  return MOE_OK;
}

moe_status_t moe_grouped_ffn(const moe_shape_t* s, const void* x, const void* x_perm,
                             const int32_t* perm_token, const int32_t* offsets,
                             const moe_weights_t* w, void* y_perm, void* y_shared, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->n_tokens == 0) return MOE_OK;
  if ((st = check_weights(s, w, false, true)) != MOE_OK) return st;
  if (!offsets || !y_perm) return fail(MOE_ERR_INVALID_ARG, "offsets / y_perm is NULL");
  if (!x_perm && (!x || !perm_token))
    return fail(MOE_ERR_INVALID_ARG, "without x_perm, x and perm_token are required");
  if (s->n_shared && (!x || !y_shared))
    return fail(MOE_ERR_INVALID_ARG, "the shared expert needs x and y_shared");
  if ((st = check_aligned({x, x_perm, y_perm, y_shared})) != MOE_OK) return st;
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  const WsLayout L = ws_layout(s);
  char* b = static_cast<char*>(ws);
  return run_ffn(s, x, x_perm ? x_perm : x, x_perm ? nullptr : perm_token, offsets, w, b + L.H,
                 b + L.H_sh, y_perm, y_shared, b + L.sched, 3, stream);
}

moe_status_t moe_expert_gate_up(const moe_shape_t* s, const void* x, const void* x_perm,
                                const int32_t* perm_token, const int32_t* offsets,
                                const moe_weights_t* w, void* h, void* h_shared, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->n_tokens == 0) return MOE_OK;
  if ((st = check_weights(s, w, false, true)) != MOE_OK) return st;
  if (!offsets || !h) return fail(MOE_ERR_INVALID_ARG, "offsets / h is NULL");
  if (!x_perm && (!x || !perm_token))
    return fail(MOE_ERR_INVALID_ARG, "without x_perm, x and perm_token are required");
  if (s->n_shared && (!x || !h_shared))
    return fail(MOE_ERR_INVALID_ARG, "the shared expert needs x and h_shared");
  if ((st = check_aligned({x, x_perm, h, h_shared})) != MOE_OK) return st;
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  return run_ffn(s, x, x_perm ? x_perm : x, x_perm ? nullptr : perm_token, offsets, w, h,
                 h_shared, nullptr, nullptr, static_cast<char*>(ws) + ws_layout(s).sched, 1,
                 stream);
}

moe_status_t moe_expert_down(const moe_shape_t* s, const void* h, const void* h_shared,
                             const int32_t* offsets, const moe_weights_t* w, void* y_perm,
                             void* y_shared, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->n_tokens == 0) return MOE_OK;
  if ((st = check_weights(s, w, false, true)) != MOE_OK) return st;
  if (!offsets || !h || !y_perm) return fail(MOE_ERR_INVALID_ARG, "offsets / h / y_perm is NULL");
  if (s->n_shared && (!h_shared || !y_shared))
    return fail(MOE_ERR_INVALID_ARG, "the shared expert needs h_shared and y_shared");
  if ((st = check_aligned({h, h_shared, y_perm, y_shared})) != MOE_OK) return st;
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  return run_ffn(s, nullptr, nullptr, nullptr, offsets, w, const_cast<void*>(h),
                 const_cast<void*>(h_shared), y_perm, y_shared,
                 static_cast<char*>(ws) + ws_layout(s).sched, 2, stream);
}

moe_status_t moe_combine(const moe_shape_t* s, const void* y_perm, const void* y_shared,
                         const int32_t* inv_perm, const float* topk_w, void* out,
                         hipStream_t stream) {
  moe_status_t st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->n_tokens == 0) return MOE_OK;
  if (!y_perm || !inv_perm || !topk_w || !out)
    return fail(MOE_ERR_INVALID_ARG, "y_perm / inv_perm / topk_w / out is NULL");
  if (s->n_shared && !y_shared) return fail(MOE_ERR_INVALID_ARG, "n_shared == 1 needs y_shared");
  if ((st = check_aligned({y_perm, y_shared, out})) != MOE_OK) return st;
  HIP_TRY("combine", launch_combine(y_perm, s->n_shared ? y_shared : nullptr, inv_perm, topk_w,
                                    out, s->n_tokens, s->top_k, s->d_model,
                                    s->act_dtype == MOE_BF16, stream));
  return MOE_OK;
}

static moe_status_t check_stats_args(const moe_shape_t* s, float alpha, float step,
                                     const float* bias) {
  if (!(alpha == alpha) || !(step == step)) return fail(MOE_ERR_INVALID_ARG, "alpha / step is NaN");
  if (bias && s->route != MOE_ROUTE_SIGMOID_BIAS)
    return fail(MOE_ERR_INVALID_ARG, "the selection bias belongs to the sigmoid router");
  return MOE_OK;
}

// The statistics kernels on router logit partials already in the workspace.
static moe_status_t run_stats(const moe_shape_t* s, const moe_weights_t* w, const float* logits,
                              const int32_t* counts, float alpha, float step, float* frac,
                              float* prob, float* aux, float* bias, float* bp,
                              hipStream_t stream) {
  HIP_TRY("load_stats",
          launch_load_stats(logits,
                            router_splits(s->n_tokens, s->n_experts, s->d_model,
                                          s->act_dtype == MOE_BF16),
                            w->logit_offset, s->route == MOE_ROUTE_SIGMOID_BIAS, s->n_tokens,
                            s->n_experts, s->top_k, counts, alpha, step, bp, frac, prob, aux, bias,
                            stream));
  return MOE_OK;
}

moe_status_t moe_load_stats(const moe_shape_t* s, const void* x, const moe_weights_t* w,
                            const int32_t* counts, float alpha, float step, float* frac,
                            float* prob, float* aux, float* bias, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  moe_status_t st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->n_tokens == 0) return MOE_OK;
  if ((st = check_weights(s, w, true, false)) != MOE_OK) return st;
  if (!x || !counts) return fail(MOE_ERR_INVALID_ARG, "x / counts is NULL");
  if ((st = check_aligned({x})) != MOE_OK) return st;
  if ((st = check_stats_args(s, alpha, step, bias)) != MOE_OK) return st;
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  const WsLayout L = ws_layout(s);
  char* b = static_cast<char*>(ws);
  float* logits = reinterpret_cast<float*>(b + L.logits);
  HIP_TRY("router_logits", launch_router_logits(x, s->act_dtype == MOE_BF16, w->w_router, logits,
                                                s->n_tokens, s->d_model, s->n_experts, stream));
  return run_stats(s, w, logits, counts, alpha, step, frac, prob, aux, bias,
                   reinterpret_cast<float*>(b + L.stats), stream);
}

// Arguments of the whole-layer calls other than the workspace (checked on
// the host before any HIP call).
static moe_status_t check_layer_args(const moe_shape_t* s, const moe_weights_t* w, const void* x,
                                     void* out, const GroupLimit& g) {
  moe_status_t st = check_shape(s);
  if (st != MOE_OK) return st;
  if ((st = check_groups(s, g)) != MOE_OK) return st;
  if (s->n_tokens == 0) return MOE_OK;
  if ((st = check_weights(s, w, true, true)) != MOE_OK) return st;
  if (!x || !out) return fail(MOE_ERR_INVALID_ARG, "x / out is NULL");
  if (x == out) return fail(MOE_ERR_INVALID_ARG, "x and out must not overlap");
  return check_aligned({x, out});
}

static moe_status_t layer_forward(const moe_shape_t* s, const moe_weights_t* w, const void* x,
                                  void* out, moe_routing_t* r, int32_t capacity,
                                  const GroupLimit& g, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  moe_status_t st = check_layer_args(s, w, x, out, g);
  if (st != MOE_OK || s->n_tokens == 0) return st;
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  const WsLayout L = ws_layout(s);
  char* b = static_cast<char*>(ws);
  auto wsi = [&](size_t off) { return reinterpret_cast<int32_t*>(b + off); };
  int32_t* idx = (r && r->topk_idx) ? r->topk_idx : wsi(L.idx);
  float* gw = (r && r->topk_w) ? r->topk_w : reinterpret_cast<float*>(b + L.w);
  // the routing the experts and the combine use: the caller's buffers when
  // given, else the workspace; with a capacity, the dropless routing goes to
  // the workspace first and the capped one to these
  const bool capped = capacity >= 0;
  int32_t* counts = (r && r->counts) ? r->counts : wsi(capped ? L.ccounts : L.counts);
  int32_t* offs = (r && r->offsets) ? r->offsets : wsi(capped ? L.coffsets : L.offsets);
  int32_t* perm = (r && r->perm_token) ? r->perm_token : wsi(capped ? L.cperm : L.perm);
  int32_t* inv = (r && r->inv_perm) ? r->inv_perm : wsi(capped ? L.cinv : L.inv);

  if ((st = run_router(s, x, w, idx, gw, reinterpret_cast<float*>(b + L.logits), stream, g)) !=
      MOE_OK)
    return st;
  if (!capped) {
    HIP_TRY("permute", launch_permute(idx, s->n_tokens, s->top_k, s->n_experts, wsi(L.hist),
                                      counts, offs, perm, inv, stream));
  } else {
    HIP_TRY("permute", launch_permute(idx, s->n_tokens, s->top_k, s->n_experts, wsi(L.hist),
                                      wsi(L.counts), wsi(L.offsets), wsi(L.perm), wsi(L.inv),
                                      stream));
    HIP_TRY("capacity", launch_capacity(idx, s->n_tokens, s->top_k, s->n_experts, capacity,
                                        wsi(L.counts), wsi(L.offsets), wsi(L.inv), counts, offs,
                                        perm, inv, stream));
  }
  if ((st = run_ffn(s, x, x, perm, offs, w, b + L.H, b + L.H_sh, b + L.Y, b + L.Y_sh,
                    b + L.sched, 3, stream)) != MOE_OK)
    return st;
  HIP_TRY("combine", launch_combine(b + L.Y, s->n_shared ? b + L.Y_sh : nullptr, inv, gw, out,
                                    s->n_tokens, s->top_k, s->d_model, s->act_dtype == MOE_BF16,
                                    stream));
  return MOE_OK;
}

moe_status_t moe_layer_forward(const moe_shape_t* s, const moe_weights_t* w, const void* x,
                               void* out, moe_routing_t* r, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  return layer_forward(s, w, x, out, r, -1, GroupLimit(), ws, ws_bytes, stream);
}

moe_status_t moe_layer_forward_grouped(const moe_shape_t* s, const moe_weights_t* w,
                                       const void* x, void* out, int32_t n_groups,
                                       int32_t max_groups, moe_routing_t* r, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
  if (n_groups < 1) return fail(MOE_ERR_INVALID_ARG, "n_groups must be >= 1");
  GroupLimit g;
  g.n_groups = n_groups;
  g.max_groups = max_groups;
  return layer_forward(s, w, x, out, r, -1, g, ws, ws_bytes, stream);
}

moe_status_t moe_layer_forward_capacity(const moe_shape_t* s, const moe_weights_t* w,
                                        const void* x, void* out, int32_t capacity,
                                        moe_routing_t* r, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  if (capacity < 0) return fail(MOE_ERR_INVALID_ARG, "capacity is negative");
  return layer_forward(s, w, x, out, r, capacity, GroupLimit(), ws, ws_bytes, stream);
}

moe_status_t moe_layer_forward_stats(const moe_shape_t* s, const moe_weights_t* w, const void* x,
                                     void* out, moe_routing_t* r, float alpha, float step,
                                     float* frac, float* prob, float* aux, float* bias, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = check_layer_args(s, w, x, out, GroupLimit());
  if (st != MOE_OK || s->n_tokens == 0) return st;
  if ((st = check_stats_args(s, alpha, step, bias)) != MOE_OK) return st;
  if ((st = check_ws(s, ws, ws_bytes)) != MOE_OK) return st;
  if ((st = layer_forward(s, w, x, out, r, -1, GroupLimit(), ws, ws_bytes, stream)) != MOE_OK)
    return st;
  const WsLayout L = ws_layout(s);
  char* b = static_cast<char*>(ws);
  float* logits = reinterpret_cast<float*>(b + L.logits);
  // the router left its logit partials in the workspace, except where logits
  // and selection ran in one kernel (a few tokens, N <= 8)
  if (router_fused_small(s->n_tokens, s->n_experts))
    HIP_TRY("router_logits", launch_router_logits(x, s->act_dtype == MOE_BF16, w->w_router,
                                                  logits, s->n_tokens, s->d_model, s->n_experts,
                                                  stream));
  const int32_t* counts = (r && r->counts) ? r->counts : reinterpret_cast<int32_t*>(b + L.counts);
  return run_stats(s, w, logits, counts, alpha, step, frac, prob, aux, bias,
                   reinterpret_cast<float*>(b + L.stats), stream);
}

moe_status_t moe_layer_forward_noalloc(const moe_shape_t* s, const moe_weights_t* w,
                                       const void* x, void* out, moe_routing_t* r,
                                       hipStream_t stream) {
  moe_status_t st = check_layer_args(s, w, x, out, GroupLimit());
  if (st != MOE_OK || s->n_tokens == 0) return st;
  const size_t need = ws_layout(s).total;
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_UNSUPPORTED,
                "this shape needs %zu bytes of scratch; moe_layer_forward_noalloc holds %zu "
                "(use moe_layer_forward with a workspace)",
                need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* p = nullptr;
  if ((st = static_scratch(&p)) != MOE_OK) return st;
  return layer_forward(s, w, x, out, r, -1, GroupLimit(), p, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
