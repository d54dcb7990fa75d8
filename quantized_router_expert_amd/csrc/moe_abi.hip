// moe_abi.hip -- extern "C" entry points: host-side validation, workspace
// carving and kernel enqueue.  Nothing is enqueued unless every argument
// passes validation.
#include <string.h>

#include <mutex>

#include "../../include/moe_decode.h"
#include "moe_device.h"
#include "moe_internal.h"
#include "moe_stack.h"

using namespace moe;

// The scratch array of moe_decode_layer_noalloc: one copy per GPU the library
// runs on, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not the device array: kernels get the device address
// that hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = 256 * 1024;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
template <class T>
inline T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off); }

// router_topk's own workspace use: counters, then logits [n_tok][E+1]
constexpr size_t kRouterLogitsOff = ((sizeof(unsigned) * kCounterSlots) + 255) & ~(size_t)255;
inline size_t router_ws_bytes(int n_tok, int E) {
  return kRouterLogitsOff + ((sizeof(float) * (size_t)n_tok * (E + 1) + 255) & ~(size_t)255);
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGN;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// Host-side record of the workspaces that hold a bound stack: which layer
// table (its length and hash) moe_stack_bind copied into which workspace.
// moe_decode_stack consults it to refuse (PERSISTENT) or avoid (AUTO) the
// persistent kernel on a workspace that does not hold the caller's layers.
struct BindRecord {
  uintptr_t ws;
  size_t bytes;
  int n_layers;
  uint64_t hash;
};
constexpr int kBindRecords = 64;
std::mutex g_bind_mu;
BindRecord g_bind[kBindRecords];
int g_bind_next = 0;

void bind_forget(uintptr_t lo, size_t bytes) {
  const uintptr_t hi = lo + bytes;
  for (auto& r : g_bind)
    if (r.ws && r.ws < hi && lo < r.ws + r.bytes) r = BindRecord{};
}

void bind_record(void* ws, size_t bytes, int n_layers, uint64_t hash) {
  std::lock_guard<std::mutex> lock(g_bind_mu);
  bind_forget((uintptr_t)ws, bytes);
  g_bind[g_bind_next] = BindRecord{(uintptr_t)ws, bytes, n_layers, hash};
  g_bind_next = (g_bind_next + 1) % kBindRecords;
}

bool bind_holds(void* ws, int n_layers, uint64_t hash) {
  std::lock_guard<std::mutex> lock(g_bind_mu);
  for (const auto& r : g_bind)
    if (r.ws == (uintptr_t)ws && r.n_layers == n_layers && r.hash == hash) return true;
  return false;
}

// Argument checks of a single-layer call (everything but the workspace).
int check_layer_call(const moe_layer_desc* desc, const moe_layer_weights* w, const moe_layer_io* io) {
  int rc = check_desc(desc);
  if (rc) return rc;
  rc = check_weights(desc, w);
  if (rc) return rc;
  if (!io || !io->routed_out) return MOE_ERR_NULL;
  if (desc->norm ? (!io->residual || !io->out_sum) : !io->x) return MOE_ERR_NULL;
  if (desc->shared_ffn > 0 && !io->shared_out) return MOE_ERR_NULL;
  if (io->shared_in && !io->routed_in) return MOE_ERR_NULL;
  if ((io->x && !aligned(io->x, 16)) || (io->xn && !aligned(io->xn, 16)) || (io->xq && !aligned(io->xq, 4)) ||
      (io->residual && !aligned(io->residual, 2)) || (io->out_sum && !aligned(io->out_sum, 2)) ||
      !aligned(io->routed_out, 2) || (io->shared_out && !aligned(io->shared_out, 2)) ||
      (io->logits && !aligned(io->logits, 4)) || (io->ids && !aligned(io->ids, 4)) ||
      (io->weights && !aligned(io->weights, 4)) || (io->h && !aligned(io->h, 4)) || (io->hs && !aligned(io->hs, 4)))
    return MOE_ERR_ALIGN;
  return MOE_OK;
}

// a1..a6 for one token in one launch; ws holds at least the layer's
// intermediates (ws_layout(desc, 0) up to its pointer table) and its counters
// are zero.
int decode_layer(const moe_layer_desc* desc, const moe_layer_weights* w, const moe_layer_io* io, void* ws,
                 hipStream_t st) {
  int rc;
  const WsLayout L = ws_layout(desc, 0);
  const int H = desc->hidden, E = desc->n_experts, k = desc->top_k;
  void* xq = io->xq ? io->xq : at<void>(ws, L.xq);
  int32_t* ids = io->ids ? io->ids : at<int32_t>(ws, L.ids);
  float* wts = io->weights ? io->weights : at<float>(ws, L.wts);
  float* sg = io->shared_gate ? io->shared_gate : at<float>(ws, L.sg);
  float* h = io->h ? io->h : at<float>(ws, L.h);
  float* hs = io->hs ? io->hs : at<float>(ws, L.hs);
  const float* wsg = desc->shared_ffn > 0 ? w->shared_gate_w : nullptr;
  if (desc->norm) {
    // the fold + norm + router rows, then gate/up selecting from their logits
    // (and writing the folded residual sum), then down + combine
    rc = launch_norm_router(io->residual, io->routed_in, io->shared_in, w->norm_w, w->router_w, wsg, H, E, desc->eps,
                            io->xn, xq, at<float>(ws, L.logits), io->logits, st);
    if (rc) return rc;
    const GateUpSelect sel{at<float>(ws, L.logits), ids, wts, sg, io->residual, io->routed_in, io->shared_in,
                           io->out_sum};
    rc = launch_gate_up(desc, w, xq, nullptr, h, hs, st, &sel);
    if (rc) return rc;
    return launch_down(desc, w, h, hs, ids, wts, sg, io->routed_out, io->shared_out, st);
  } else {
    if (io->xn) {
      if (hipMemcpyAsync(io->xn, io->x, sizeof(float) * H, hipMemcpyDeviceToDevice, st) != hipSuccess)
        return MOE_ERR_HIP;
    }
    rc = launch_quantize(io->x, H, xq, st);
    if (rc) return rc;
    rc = launch_router(io->x, w->router_w, wsg, 1, H, E, k, at<float>(ws, L.logits), io->logits, ids, wts, sg,
                       at<unsigned>(ws, L.counters), st);
    if (rc) return rc;
  }
  rc = launch_gate_up(desc, w, xq, ids, h, hs, st);
  if (rc) return rc;
  return launch_down(desc, w, h, hs, ids, wts, sg, io->routed_out, io->shared_out, st);
}

// ---- the scratch array of moe_decode_layer_noalloc (declared at file scope below)
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's scratch address, looked up once per device; the first
// call on a device also queues the clearing of the router counters (the only
// part that must start at zero: every completed call returns them to zero).
int scratch_for_current_device(void** out, hipStream_t st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    const int rc = launch_fill(p, sizeof(unsigned) * kCounterSlots / 4, 0u, st);
    if (rc) return rc;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or not a whole number of blocks";
    case MOE_ERR_TYPE: return "unsupported block type";
    case MOE_ERR_ALIGN: return "pointer not aligned as required";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
    case MOE_ERR_UNSUPPORTED: return "combination not implemented";
    case MOE_ERR_NOT_BOUND: return "layer stack not bound to this workspace";
    default: return "unknown status";
  }
}

size_t moe_workspace_size(const moe_layer_desc* desc, int n_layers) {
  if (check_desc(desc) != MOE_OK || n_layers < 0 || n_layers > MOE_MAX_LAYERS) return 0;
  return ws_layout(desc, n_layers).total;
}

int moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGN;
  if (ws_bytes < 256) return MOE_ERR_WORKSPACE;
  {
    std::lock_guard<std::mutex> lock(g_bind_mu);
    bind_forget((uintptr_t)ws, ws_bytes);
  }
  return launch_fill(ws, ws_bytes / 4, 0u, as_stream(stream));
}

int add_rmsnorm3(const uint16_t* residual, const uint16_t* routed, const uint16_t* shared, const float* norm_w,
                 int hidden, int n_tok, float eps, uint16_t* out_sum, float* xn, void* xq, void* stream) {
  if (!residual || !norm_w || !out_sum) return MOE_ERR_NULL;
  if (shared && !routed) return MOE_ERR_NULL;
  if (hidden <= 0 || hidden % 256 || hidden > MOE_MAX_HIDDEN || n_tok <= 0 || n_tok > 65535) return MOE_ERR_SHAPE;
  if (!(eps >= 0.0f)) return MOE_ERR_SHAPE;
  if (!aligned(residual, 2) || (routed && !aligned(routed, 2)) || (shared && !aligned(shared, 2)) ||
      !aligned(out_sum, 2) || !aligned(norm_w, 4) || (xn && !aligned(xn, 4)) || (xq && !aligned(xq, 4)))
    return MOE_ERR_ALIGN;
  return launch_norm(residual, routed, shared, norm_w, hidden, n_tok, eps, out_sum, xn, xq, 1, as_stream(stream));
}

int add_rmsnorm2_q8(const uint16_t* residual, const uint16_t* attn_out, const float* norm_w, int hidden, int n_tok,
                    float eps, uint16_t* out_sum, float* xn, void* xq, void* stream) {
  if (!attn_out) return MOE_ERR_NULL;
  return add_rmsnorm3(residual, attn_out, nullptr, norm_w, hidden, n_tok, eps, out_sum, xn, xq, stream);
}

int router_topk(const float* xn, const float* w_router, const float* w_shared_gate, int n_tok, int hidden,
                int n_experts, int top_k, float* logits, int32_t* ids, float* weights, float* shared_gate_out,
                void* ws, size_t ws_bytes, void* stream) {
  if (!xn || !w_router || !ids || !weights) return MOE_ERR_NULL;
  if (n_tok <= 0 || n_tok > kCounterSlots || hidden <= 0 || hidden % 256 || hidden > MOE_MAX_HIDDEN) return MOE_ERR_SHAPE;
  if (n_experts <= 0 || n_experts > MOE_MAX_EXPERTS || top_k <= 0 || top_k > n_experts || top_k > MOE_MAX_TOPK)
    return MOE_ERR_SHAPE;
  if (!aligned(xn, 16) || !aligned(w_router, 16) || (w_shared_gate && !aligned(w_shared_gate, 16)) ||
      !aligned(ids, 4) || !aligned(weights, 4) || (logits && !aligned(logits, 4)) ||
      (shared_gate_out && !aligned(shared_gate_out, 4)))
    return MOE_ERR_ALIGN;
  int rc = check_ws(ws, ws_bytes, router_ws_bytes(n_tok, n_experts));
  if (rc) return rc;
  return launch_router(xn, w_router, w_shared_gate, n_tok, hidden, n_experts, top_k, at<float>(ws, kRouterLogitsOff),
                       logits, ids, weights, shared_gate_out, at<unsigned>(ws, 0), as_stream(stream));
}

int expert_ffn_q4k(const moe_layer_desc* desc, const moe_layer_weights* w, const void* xq, const int32_t* ids,
                   const float* weights, const float* shared_gate, int n_tok, uint16_t* routed_out,
                   uint16_t* shared_out, float* h, float* hs, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  rc = check_weights(desc, w);
  if (rc) return rc;
  if (!xq || !ids || !weights || !routed_out) return MOE_ERR_NULL;
  if (desc->shared_ffn > 0 && (!shared_gate || !shared_out)) return MOE_ERR_NULL;
  if (n_tok != 1) return MOE_ERR_UNSUPPORTED;
  if (!aligned(xq, 4) || !aligned(ids, 4) || !aligned(weights, 4) || !aligned(routed_out, 2) ||
      (shared_out && !aligned(shared_out, 2)) || (h && !aligned(h, 4)) || (hs && !aligned(hs, 4)))
    return MOE_ERR_ALIGN;
  const WsLayout L = ws_layout(desc, 0);
  rc = check_ws(ws, ws_bytes, L.total);
  if (rc) return rc;
  float* hb = h ? h : at<float>(ws, L.h);
  float* hsb = hs ? hs : at<float>(ws, L.hs);
  hipStream_t st = as_stream(stream);
  rc = launch_gate_up(desc, w, xq, ids, hb, hsb, st);
  if (rc) return rc;
  return launch_down(desc, w, hb, hsb, ids, weights, shared_gate, routed_out, shared_out, st);
}

int moe_decode_layer(const moe_layer_desc* desc, const moe_layer_weights* w, const moe_layer_io* io, void* ws,
                     size_t ws_bytes, void* stream) {
  int rc = check_layer_call(desc, w, io);
  if (rc) return rc;
  rc = check_ws(ws, ws_bytes, ws_layout(desc, 0).total);
  if (rc) return rc;
  return decode_layer(desc, w, io, ws, as_stream(stream));
}

int moe_decode_layer_noalloc(const moe_layer_desc* desc, const moe_layer_weights* w, const moe_layer_io* io,
                             void* stream) {
  int rc = check_layer_call(desc, w, io);
  if (rc) return rc;
  // the layer's intermediates end where the stack's pointer table would begin
  if (ws_layout(desc, 0).table > kScratchBytes) return MOE_ERR_WORKSPACE;
  void* sp = nullptr;
  hipStream_t st = as_stream(stream);
  rc = scratch_for_current_device(&sp, st);
  if (rc) return rc;
  return decode_layer(desc, w, io, sp, st);
}

size_t moe_batch_workspace_size(const moe_layer_desc* desc, int n_tok) {
  if (check_desc(desc) != MOE_OK || n_tok <= 0 || n_tok > MOE_MAX_BATCH) return 0;
  return batch_ws_layout(desc, n_tok).total;
}

int expert_ffn_grouped(const moe_layer_desc* desc, const moe_layer_weights* w, const float* xn, const void* xq,
                       const int32_t* ids, const float* weights, const float* shared_gate, int n_tok, int group_min,
                       uint16_t* routed_out, uint16_t* shared_out, float* h, float* hs, void* ws, size_t ws_bytes,
                       void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  rc = check_weights(desc, w);
  if (rc) return rc;
  if (!xn || !xq || !ids || !weights || !routed_out) return MOE_ERR_NULL;
  if (desc->shared_ffn > 0 && (!shared_gate || !shared_out)) return MOE_ERR_NULL;
  if (n_tok <= 0 || n_tok > MOE_MAX_BATCH || group_min < 1 || group_min > MOE_MAX_GROUP_MIN) return MOE_ERR_SHAPE;
  if (!aligned(xn, 16) || !aligned(xq, 4) || !aligned(ids, 4) || !aligned(weights, 4) || !aligned(routed_out, 2) ||
      (shared_out && !aligned(shared_out, 2)) || (shared_gate && !aligned(shared_gate, 4)) || (h && !aligned(h, 16)) ||
      (hs && !aligned(hs, 16)))
    return MOE_ERR_ALIGN;
  const BatchWs L = batch_ws_layout(desc, n_tok);
  rc = check_ws(ws, ws_bytes, L.total);
  if (rc) return rc;
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  return launch_grouped_ffn(desc, w, xn, xq, ids, weights, shared_gate, n_tok, group_min, routed_out, shared_out,
                            h ? h : at<float>(ws, L.h), hs ? hs : at<float>(ws, L.hs), wsb, L, as_stream(stream));
}

int moe_decode_layer_batch(const moe_layer_desc* desc, const moe_layer_weights* w, const moe_layer_io* io, int n_tok,
                           int group_min, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  rc = check_weights(desc, w);
  if (rc) return rc;
  if (!io || !io->routed_out) return MOE_ERR_NULL;
  if (desc->norm ? (!io->residual || !io->out_sum) : !io->x) return MOE_ERR_NULL;
  if (desc->shared_ffn > 0 && !io->shared_out) return MOE_ERR_NULL;
  if (io->shared_in && !io->routed_in) return MOE_ERR_NULL;
  if (n_tok <= 0 || n_tok > MOE_MAX_BATCH || group_min < 1 || group_min > MOE_MAX_GROUP_MIN) return MOE_ERR_SHAPE;
  if ((io->x && !aligned(io->x, 16)) || (io->xn && !aligned(io->xn, 16)) || (io->xq && !aligned(io->xq, 4)) ||
      (io->residual && !aligned(io->residual, 2)) || (io->out_sum && !aligned(io->out_sum, 2)) ||
      !aligned(io->routed_out, 2) || (io->shared_out && !aligned(io->shared_out, 2)) ||
      (io->logits && !aligned(io->logits, 4)) || (io->ids && !aligned(io->ids, 4)) ||
      (io->weights && !aligned(io->weights, 4)) || (io->shared_gate && !aligned(io->shared_gate, 4)) ||
      (io->h && !aligned(io->h, 16)) || (io->hs && !aligned(io->hs, 16)))
    return MOE_ERR_ALIGN;
  const BatchWs L = batch_ws_layout(desc, n_tok);
  rc = check_ws(ws, ws_bytes, L.total);
  if (rc) return rc;
  hipStream_t st = as_stream(stream);
  const int H = desc->hidden, E = desc->n_experts, k = desc->top_k;
  float* xn = io->xn ? io->xn : at<float>(ws, L.xn);
  void* xq = io->xq ? io->xq : at<void>(ws, L.xq);
  int32_t* ids = io->ids ? io->ids : at<int32_t>(ws, L.ids);
  float* wts = io->weights ? io->weights : at<float>(ws, L.wts);
  float* sg = io->shared_gate ? io->shared_gate : at<float>(ws, L.sg);
  if (desc->norm) {
    rc = launch_norm(io->residual, io->routed_in, io->shared_in, w->norm_w, H, n_tok, desc->eps, io->out_sum, xn, xq, 1,
                     st);
  } else {
    if (hipMemcpyAsync(xn, io->x, sizeof(float) * (size_t)n_tok * H, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return MOE_ERR_HIP;
    rc = launch_quantize(io->x, n_tok * H, xq, st);
  }
  if (rc) return rc;
  rc = launch_router(xn, w->router_w, desc->shared_ffn > 0 ? w->shared_gate_w : nullptr, n_tok, H, E, k,
                     at<float>(ws, L.router + kRouterLogitsOff), io->logits, ids, wts, sg,
                     at<unsigned>(ws, L.router), st);
  if (rc) return rc;
  return launch_grouped_ffn(desc, w, xn, xq, ids, wts, sg, n_tok, group_min, io->routed_out, io->shared_out,
                            io->h ? io->h : at<float>(ws, L.h), io->hs ? io->hs : at<float>(ws, L.hs),
                            static_cast<uint8_t*>(ws), L, st);
}

int moe_tune_group_min(const moe_layer_desc* desc, const moe_layer_weights* w, const moe_layer_io* io, int n_tok,
                       const int* candidates, int n_candidates, int reps, void* ws, size_t ws_bytes, void* stream,
                       int* best, float* best_us) {
  if (!candidates || !best) return MOE_ERR_NULL;
  if (n_candidates < 1 || n_candidates > MOE_MAX_GROUP_MIN || reps < 1 || reps > 100) return MOE_ERR_SHAPE;
  for (int i = 0; i < n_candidates; ++i)
    if (candidates[i] < 1 || candidates[i] > MOE_MAX_GROUP_MIN) return MOE_ERR_SHAPE;
  hipStream_t st = as_stream(stream);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) return MOE_ERR_HIP;
  if (cs != hipStreamCaptureStatusNone) return MOE_ERR_UNSUPPORTED;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess) return MOE_ERR_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return MOE_ERR_HIP;
  }
  int rc = MOE_OK, pick = candidates[0];
  float pick_us = 0.0f;
  for (int i = 0; i < n_candidates && rc == MOE_OK; ++i) {
    const int g = candidates[i];
    rc = moe_decode_layer_batch(desc, w, io, n_tok, g, ws, ws_bytes, stream);   // warm-up
    if (rc == MOE_OK && hipEventRecord(e0, st) != hipSuccess) rc = MOE_ERR_HIP;
    for (int r = 0; r < reps && rc == MOE_OK; ++r) rc = moe_decode_layer_batch(desc, w, io, n_tok, g, ws, ws_bytes, stream);
    float ms = 0.0f;
    if (rc == MOE_OK && (hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                         hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
      rc = MOE_ERR_HIP;
    const float us = 1000.0f * ms / (float)reps;
    if (rc == MOE_OK && (i == 0 || us < pick_us)) {
      pick = g;
      pick_us = us;
    }
  }
  (void)hipEventDestroy(e1);
  (void)hipEventDestroy(e0);
  if (rc) return rc;
  *best = pick;
  if (best_us) *best_us = pick_us;
  return MOE_OK;
}

int moe_stack_bind(const moe_layer_desc* desc, const moe_layer_weights* layers, int n_layers, void* ws,
                   size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!desc->norm) return MOE_ERR_UNSUPPORTED;
  if (!layers) return MOE_ERR_NULL;
  if (n_layers <= 0 || n_layers > MOE_MAX_LAYERS) return MOE_ERR_SHAPE;
  for (int l = 0; l < n_layers; ++l)
    if ((rc = check_weights(desc, &layers[l]))) return rc;
  const WsLayout L = ws_layout(desc, n_layers);
  rc = check_ws(ws, ws_bytes, L.total);
  if (rc) return rc;
  hipStream_t st = as_stream(stream);
  if (L.stack == 0) return MOE_ERR_UNSUPPORTED;
  {
    // the record goes before the copies: if one of them fails, the workspace
    // holds no complete table and must not count as bound
    std::lock_guard<std::mutex> lock(g_bind_mu);
    bind_forget((uintptr_t)ws, ws_bytes);
  }
  if (hipMemcpyAsync(at<void>(ws, L.table), layers, sizeof(moe_layer_weights) * n_layers, hipMemcpyHostToDevice, st) !=
      hipSuccess)
    return MOE_ERR_HIP;
  const uint64_t hash = layer_table_hash(layers, n_layers);
  const uint32_t bound[4] = {kBoundMagic, (uint32_t)n_layers, (uint32_t)hash, (uint32_t)(hash >> 32)};
  if (hipMemcpyAsync(at<void>(ws, L.bound), bound, sizeof(bound), hipMemcpyHostToDevice, st) != hipSuccess)
    return MOE_ERR_HIP;
  // a fresh generation: control block and exchange words start from zero
  rc = launch_fill(at<void>(ws, L.stack), (L.total - L.stack) / 4, 0u, st);
  if (rc) return rc;
  if (hipStreamSynchronize(st) != hipSuccess) return MOE_ERR_HIP;
  bind_record(ws, ws_bytes, n_layers, hash);
  return MOE_OK;
}

int moe_decode_stack(const moe_layer_desc* desc, const moe_layer_weights* layers, int n_layers, const moe_stack_io* io,
                     int mode, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!desc->norm) return MOE_ERR_UNSUPPORTED;
  if (!layers || !io || !io->input || !io->output) return MOE_ERR_NULL;
  if (n_layers <= 0 || n_layers > MOE_MAX_LAYERS) return MOE_ERR_SHAPE;
  if (mode != MOE_STACK_AUTO && mode != MOE_STACK_KERNELS && mode != MOE_STACK_PERSISTENT &&
      mode != MOE_STACK_COOPERATIVE)
    return MOE_ERR_SHAPE;
  for (int l = 0; l < n_layers; ++l)
    if ((rc = check_weights(desc, &layers[l]))) return rc;
  if (!aligned(io->input, 2) || !aligned(io->output, 2) || (io->ids && !aligned(io->ids, 4)) ||
      (io->resid && !aligned(io->resid, 2)) || (io->routed && !aligned(io->routed, 2)) ||
      (io->shared && !aligned(io->shared, 2)) || (io->attn && !aligned(io->attn, 8)))
    return MOE_ERR_ALIGN;
  const WsLayout L = ws_layout(desc, n_layers);
  rc = check_ws(ws, ws_bytes, L.total);
  if (rc) return rc;
  hipStream_t st = as_stream(stream);
  if (mode == MOE_STACK_PERSISTENT || mode == MOE_STACK_COOPERATIVE || mode == MOE_STACK_AUTO) {
    const bool explicit_persistent = mode == MOE_STACK_PERSISTENT || mode == MOE_STACK_COOPERATIVE;
    const uint64_t hash = layer_table_hash(layers, n_layers);
    const bool bound = bind_holds(ws, n_layers, hash);
    if (explicit_persistent && !bound) return MOE_ERR_NOT_BOUND;
    int G = 0;
    if ((rc = device_cu_count(&G))) return rc;
    StackGeom g;
    rc = (G >= 8 && G % 8 == 0 && L.stack) ? stack_geometry(desc, G, &g) : MOE_ERR_UNSUPPORTED;
    if (rc == MOE_OK && g.lds > kStackMaxLds) rc = MOE_ERR_UNSUPPORTED;
    if (rc == MOE_OK && bound) {
      stack_ws_layout(&g, L.stack);
      return launch_stack(desc, n_layers, at<moe_layer_weights>(ws, L.table), at<uint32_t>(ws, L.bound), hash, io,
                          static_cast<uint8_t*>(ws), g, st, mode == MOE_STACK_COOPERATIVE);
    }
    if (explicit_persistent) return rc;
  }
  const int H = desc->hidden, E = desc->n_experts, k = desc->top_k;
  const bool has_shared = desc->shared_ffn > 0;
  const uint16_t* res_in = io->input;
  const uint16_t* prev_routed = nullptr;
  const uint16_t* prev_shared = nullptr;
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer_weights* w = &layers[l];
    uint16_t* res_out = io->resid ? io->resid + (size_t)l * H : at<uint16_t>(ws, L.res);
    int32_t* ids = io->ids ? io->ids + (size_t)l * k : at<int32_t>(ws, L.ids);
    // the layer's outputs may overwrite the previous layer's in the workspace:
    // the norm that reads those runs first on the stream
    uint16_t* routed = io->routed ? io->routed + (size_t)l * H : at<uint16_t>(ws, L.routed);
    uint16_t* shared = has_shared ? (io->shared ? io->shared + (size_t)l * H : at<uint16_t>(ws, L.shared)) : nullptr;
    // the add-norm (after an attention block: the fold of the previous outputs
    // into u1, then the add-norm on (u1, attn_l)) and the router in one launch
    const uint16_t* nin = res_in;
    const uint16_t* n1 = prev_routed;
    const uint16_t* n2 = prev_shared;
    if (io->attn) {
      if (l > 0) {
        rc = launch_norm(res_in, prev_routed, prev_shared, nullptr, H, 1, desc->eps, at<uint16_t>(ws, L.u1), nullptr,
                         nullptr, 0, st);
        if (rc) return rc;
        nin = at<uint16_t>(ws, L.u1);
      }
      n1 = io->attn + (size_t)l * H;
      n2 = nullptr;
    }
    rc = launch_norm_router(nin, n1, n2, w->norm_w, w->router_w, has_shared ? w->shared_gate_w : nullptr, H, E,
                            desc->eps, nullptr, at<void>(ws, L.xq), at<float>(ws, L.logits), nullptr, st);
    if (rc) return rc;
    const GateUpSelect sel{at<float>(ws, L.logits), ids, at<float>(ws, L.wts), at<float>(ws, L.sg), nin, n1, n2,
                           res_out};
    rc = launch_gate_up(desc, w, at<void>(ws, L.xq), nullptr, at<float>(ws, L.h), at<float>(ws, L.hs), st, &sel);
    if (rc) return rc;
    rc = launch_down(desc, w, at<float>(ws, L.h), at<float>(ws, L.hs), ids, at<float>(ws, L.wts), at<float>(ws, L.sg),
                     routed, shared, st);
    if (rc) return rc;
    res_in = res_out;
    prev_routed = routed;
    prev_shared = shared;
  }
  // the fold the next layer's norm would do: output = bf16(res_L + bf16(routed + shared))
  return launch_norm(res_in, prev_routed, prev_shared, nullptr, H, 1, desc->eps, io->output, nullptr, nullptr, 0, st);
}

size_t moe_stack_status_offset(const moe_layer_desc* desc, int n_layers) {
  if (check_desc(desc) != MOE_OK || n_layers <= 0 || n_layers > MOE_MAX_LAYERS) return 0;
  const WsLayout L = ws_layout(desc, n_layers);
  if (!L.stack) return 0;
  StackGeom g;
  if (stack_geometry(desc, 256, &g) != MOE_OK) return 0;
  stack_ws_layout(&g, L.stack);
  return g.w_ctrl + 4 * kErrWord;
}

int moe_stack_kernel_shape(const moe_layer_desc* desc) {
  if (check_desc(desc) != MOE_OK || !desc->norm) return -1;
  int G = 0;
  if (device_cu_count(&G) != MOE_OK) return -1;
  StackGeom g;
  if (G < 8 || G % 8 || stack_geometry(desc, G, &g) != MOE_OK || g.lds > kStackMaxLds) return -1;
  int shape = -1;
  return stack_kernel_for(desc, g, &shape) ? shape : -1;
}

size_t moe_stack_trace_offset(const moe_layer_desc* desc, int n_layers) {
  if (check_desc(desc) != MOE_OK || n_layers <= 0 || n_layers > MOE_MAX_LAYERS) return 0;
  const WsLayout L = ws_layout(desc, n_layers);
  if (!L.stack) return 0;
  StackGeom g;
  if (stack_geometry(desc, 256, &g) != MOE_OK) return 0;
  stack_ws_layout(&g, L.stack);
  return g.w_trace;
}

int moe_test_subblock_dots(const void* rows, int type, int K, int n_rows, const void* xq, int32_t* out, void* stream) {
  if (!rows || !xq || !out) return MOE_ERR_NULL;
  if (type != MOE_TYPE_Q4_K && type != MOE_TYPE_Q5_K && type != MOE_TYPE_Q8_0) return MOE_ERR_TYPE;
  if (K <= 0 || K % 256 || K > MOE_MAX_HIDDEN || n_rows <= 0 || n_rows > 65535) return MOE_ERR_SHAPE;
  if (!aligned(rows, 16) || !aligned(xq, 4) || !aligned(out, 4)) return MOE_ERR_ALIGN;
  return launch_subblock_dots(rows, type, K, n_rows, xq, out, as_stream(stream));
}

int moe_requant_q4k(const void* src, int src_type, int n_rows, int K, void* dst, void* stream) {
  if (!src || !dst) return MOE_ERR_NULL;
  if (src_type != MOE_TYPE_Q8_0 && src_type != MOE_TYPE_Q5_K && src_type != MOE_TYPE_Q4_K) return MOE_ERR_TYPE;
  if (n_rows <= 0 || K <= 0 || K % 256 || (long)n_rows * (K / 256) > (1L << 30)) return MOE_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(dst, 2)) return MOE_ERR_ALIGN;
  return launch_requant_q4k(src, src_type, n_rows, K, dst, as_stream(stream));
}

int moe_stream_read(const void* p, size_t bytes, uint32_t* out, int blocks, void* stream) {
  if (!p || !out) return MOE_ERR_NULL;
  if (bytes == 0 || bytes % 16 || blocks <= 0 || blocks > 65535) return MOE_ERR_SHAPE;
  if (!aligned(p, 16) || !aligned(out, 4)) return MOE_ERR_ALIGN;
  return launch_stream_read(p, bytes, out, blocks, as_stream(stream));
}

int moe_test_quantize_q81(const float* x, int n, void* xq, void* stream) {
  if (!x || !xq) return MOE_ERR_NULL;
  if (n <= 0 || n % 32 || n > (1 << 26)) return MOE_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(xq, 2)) return MOE_ERR_ALIGN;
  return launch_test_q81_groups(x, n, xq, as_stream(stream));
}

int moe_test_stack_select(const float* logits, int n_sets, int n_experts, int top_k, int with_gate, int32_t* ids,
                          float* weights, float* gate, void* stream) {
  if (!logits || !ids || !weights) return MOE_ERR_NULL;
  if (with_gate && !gate) return MOE_ERR_NULL;
  if (n_sets <= 0 || n_sets > 65535 || n_experts <= 0 || n_experts > MOE_MAX_EXPERTS || top_k <= 0 ||
      top_k > n_experts || top_k > MOE_MAX_TOPK)
    return MOE_ERR_SHAPE;
  if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(weights, 4) || (gate && !aligned(gate, 4)))
    return MOE_ERR_ALIGN;
  return launch_test_stack_select(logits, n_sets, n_experts, top_k, with_gate, ids, weights, with_gate ? gate : nullptr,
                                  as_stream(stream));
}

}  // extern "C"
