// moe_internal.h -- host/device declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_decode.h"

namespace moe {

constexpr int kNormThreads = 256;
constexpr int kRouterThreads = 512;
constexpr int kRouterTok = 8;      // tokens per router workgroup (a row is read once for them)
constexpr int kFfnThreads = 512;
constexpr int kTopkPerLane = MOE_MAX_EXPERTS / 64;
constexpr int kCounterSlots = 4096;
constexpr int kGateUpRows = 16;
constexpr int kDownRows = 8;
constexpr size_t kLdsBudget = 64 * 1024;

// Byte offsets of the workspace regions (all 256-byte aligned).
struct WsLayout {
  size_t counters, xn, xq, logits, ids, wts, sg, h, hs, res, routed, shared, u1, table, bound, stack, total;
};
WsLayout ws_layout(const moe_layer_desc* d, int n_layers);

int check_desc(const moe_layer_desc* d);
int check_weights(const moe_layer_desc* d, const moe_layer_weights* w);

int launch_norm(const uint16_t* res, const uint16_t* rt, const uint16_t* sh, const float* w, int H, int n_tok,
                float eps, uint16_t* out_sum, float* xn, void* xq, int do_norm, hipStream_t st);
int launch_quantize(const float* x, int n, void* xq, hipStream_t st);
int launch_router(const float* xn, const float* W, const float* wsg, int n_tok, int H, int E, int k, float* logits,
                  float* user_logits, int32_t* ids, float* wts, float* sg, unsigned* counters, hipStream_t st);
// a1 + a2 of one token in one launch (the residual fold and norm, the router
// rows): logits [E + 1], xq, and xn when given.
int launch_norm_router(const uint16_t* res, const uint16_t* rt, const uint16_t* sh, const float* norm_w, const float* W,
                       const float* wsg, int H, int E, float eps, float* xn, void* xq, float* logits,
                       float* user_logits, hipStream_t st);
// k_gate_up selecting its experts itself from the router launch's logits (a3)
// and writing the folded residual sum (res, rt, sh -> out_sum, may alias).
struct GateUpSelect {
  const float* logits;
  int32_t* ids;
  float* wts;
  float* sg;
  const uint16_t* res;
  const uint16_t* rt;
  const uint16_t* sh;
  uint16_t* out_sum;
};
int launch_gate_up(const moe_layer_desc* d, const moe_layer_weights* w, const void* xq, const int32_t* ids, float* h,
                   float* hs, hipStream_t st, const GateUpSelect* sel = nullptr);
int launch_down(const moe_layer_desc* d, const moe_layer_weights* w, const float* h, const float* hs, const int32_t* ids,
                const float* wts, const float* sg, uint16_t* routed, uint16_t* shared, hipStream_t st);
int launch_fill(void* p, size_t n_u32, uint32_t v, hipStream_t st);

// workspace of the grouped (batch > 1) path
struct BatchWs {
  size_t router, cnt, moff, members, dlist, nd, blist, nb, err, xn, xq, ids, wts, sg, h, hs, y, ys, total;
};
BatchWs batch_ws_layout(const moe_layer_desc* d, int n_tok);
int launch_grouped_ffn(const moe_layer_desc* d, const moe_layer_weights* w, const float* xn, const void* xq,
                       const int32_t* ids, const float* wts, const float* sg, int n, int gmin, uint16_t* routed,
                       uint16_t* shared, float* h, float* hs, uint8_t* ws, const BatchWs& L, hipStream_t st);
int launch_subblock_dots(const void* rows, int type, int K, int n_rows, const void* xq, int32_t* out, hipStream_t st);
int launch_test_q81_groups(const float* x, int n, void* xq, hipStream_t st);
int launch_stream_read(const void* p, size_t bytes, uint32_t* out, int blocks, hipStream_t st);
int launch_requant_q4k(const void* src, int src_type, int n_rows, int K, void* dst, hipStream_t st);

}  // namespace moe
